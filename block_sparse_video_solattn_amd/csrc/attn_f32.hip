// Steps 2-5 of Sol-Attn for fp32 inputs (the same routing device code as the
// bf16 kernel; fp32 vector arithmetic end to end, for fp32-accurate results).
//
// One workgroup = four wavefronts = one 64-row query block; lane r of every
// wave owns query row r.  Wave w takes d/4 of the head dimension: its slice
// of each logit's dot product (fp64) and its d/4 output columns.  Key and
// value rows are staged through LDS, 16 at a time, and read back as
// wave-wide broadcasts; the four partial logits of a (row, key) pair meet in
// LDS and every wave adds them in the same order, so all four run the same
// softmax on the same values.  Exact blocks contribute their rows; pooled
// tiles contribute kbar_j / vbar_j with logit bias log2(n_j) (-inf for kept
// blocks), exactly as in the bf16 kernel (page "NVIDIA 团队开源 Sol-H3 的 DGX
// Spark 版本", section "119.68 GiB 的内存池", Sol-Attn item).
#include "common.h"
#include "launch.h"
#include "route.h"

namespace solattn {

constexpr int kF32Waves = 4;   // waves per query block
constexpr int kF32Sub = 16;    // keys staged per step

// LDS of attn_f32_kernel (floats): per wave its score row [Nbp] and kept
// list [Nb] (uint16), then the staged key and value rows [SUB][D] each, the
// step's column biases [SUB] and the partial logits [waves][SUB][64] (fp64).
inline size_t f32_lds_floats(int64_t Nb, int64_t Nbp, int64_t d) {
    return kF32Waves * (Nbp + (Nb + 15) / 16 * 8) + 2 * kF32Sub * d + kF32Sub +
           2 * kF32Waves * kF32Sub * 64;
}

template <int D>
__global__ __launch_bounds__(64 * kF32Waves) void attn_f32_kernel(AttnArgs a) {
    constexpr int SUB = kF32Sub, DW = D / kF32Waves;
    extern __shared__ float smem[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t N = a.N, Nb = a.Nb, Nbp = a.Nbp;
    const int64_t w = xcd_remap(blockIdx.x, a.BH * Nb);
    const int64_t bh = w / Nb, i = w % Nb;
    const int64_t per_wave = Nbp + (Nb + 15) / 16 * 8;
    float* srow = smem + wave * per_wave;
    uint16_t* klist = reinterpret_cast<uint16_t*>(srow + Nbp);
    float* ks = smem + kF32Waves * per_wave;  // [SUB][D]
    float* vs = ks + SUB * D;                 // [SUB][D]
    float* kb = vs + SUB * D;                 // [SUB] bias
    double* xp = reinterpret_cast<double*>(kb + SUB);  // [waves][SUB][64] partial logits
    // (kb + SUB is 8-byte aligned: every term before it is a multiple of 16 floats)

    // Every wave routes the block into its own LDS slice (the same code on
    // the same values: identical lists; every wave reaches the routing's
    // barriers); only wave 0 writes the debug exports.
    AttnArgs ar = a;
    if (__builtin_amdgcn_readfirstlane(wave) != 0) {
        ar.mask_out = nullptr;
        ar.score_out = nullptr;
        ar.thr_out = nullptr;
    }
    int n_kept;
    uint64_t tile_mask;
    if (a.mode != kDense) {
        const RouteResult r = route_query_block<D>(ar, bh, i, srow, klist);
        n_kept = r.n_kept;
        tile_mask = r.tile_mask;
    } else {
        if (wave == 0) export_dense_route(a, bh, i);
        n_kept = (int)Nb;
        tile_mask = 0;
    }
    __syncthreads();  // the routing's LDS lists are complete

    const float* qp = reinterpret_cast<const float*>(a.q) + bh * N * D;
    const float* kp = reinterpret_cast<const float*>(a.k) + bh * N * D;
    const float* vp = reinterpret_cast<const float*>(a.v) + bh * N * D;
    const float* kbarp = a.kbar + bh * Nb * D;
    const float* vbarp = a.vbar + bh * Nb * D;
    const double scale2d = 1.4426950408889634 / sqrt((double)D);
    const int d0 = wave * DW;

    int64_t row = i * 64 + lane;
    if (row > N - 1) row = N - 1;
    // acc sums whole tiles; part sums the <= 64 terms of the current tile.
    // Two-level summation keeps fp32 rounding from growing linearly with N
    // when many equal terms are added (e.g. blocks of identical keys).
    float qr[DW], acc[DW], part[DW];
#pragma unroll
    for (int d = 0; d < DW; d += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(qp + row * D + d0 + d);
        qr[d] = x[0]; qr[d + 1] = x[1]; qr[d + 2] = x[2]; qr[d + 3] = x[3];
        acc[d] = acc[d + 1] = acc[d + 2] = acc[d + 3] = 0.f;
        part[d] = part[d + 1] = part[d + 2] = part[d + 3] = 0.f;
    }
    double m = -__builtin_inf();
    float l = 0.f, lpart = 0.f;

    const int n_tiles = n_kept + __popcll(tile_mask);
    uint64_t tm = tile_mask;
    for (int t = 0; t < n_tiles; ++t) {
        // the 64 columns of this tile: rows of K/V (exact) or of kbar/vbar (pooled)
        const float* ksrc;
        const float* vsrc;
        int nrows, ptile = -1;
        if (t < n_kept) {
            const int64_t j = (a.mode != kDense) ? (int64_t)klist[t] : (int64_t)t;
            ksrc = kp + j * 64 * D;
            vsrc = vp + j * 64 * D;
            nrows = (int)((j + 1) * 64 <= N ? 64 : N - j * 64);
        } else {
            ptile = __builtin_ctzll(tm);
            tm &= tm - 1;
            ksrc = kbarp + (int64_t)ptile * 64 * D;
            vsrc = vbarp + (int64_t)ptile * 64 * D;
            nrows = (int)((ptile + 1) * 64 <= Nb ? 64 : Nb - ptile * 64);
        }
        for (int sub = 0; sub < 64; sub += SUB) {
            __syncthreads();
            // stage SUB rows (coalesced 16-byte loads), zero past nrows
            for (int e = (int)threadIdx.x * 4; e < SUB * D; e += 4 * 64 * kF32Waves) {
                const int r = e / D, c = e % D;
                f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
                if (sub + r < nrows) {
                    kx = *reinterpret_cast<const f32x4*>(ksrc + (int64_t)(sub + r) * D + c);
                    vx = *reinterpret_cast<const f32x4*>(vsrc + (int64_t)(sub + r) * D + c);
                }
                *reinterpret_cast<f32x4*>(ks + e) = kx;
                *reinterpret_cast<f32x4*>(vs + e) = vx;
            }
            if (threadIdx.x < SUB) {
                const int key = sub + (int)threadIdx.x;
                if (ptile >= 0)
                    kb[threadIdx.x] = srow[64 * ptile + key];
                else
                    kb[threadIdx.x] = key < nrows ? 0.f : -__builtin_inff();
            }
            __syncthreads();
            // logits in fp64: products of fp32 values are exact in fp64 and the
            // d-term sums keep 53 bits, so the logit error does not grow with
            // |q||k| (fp32 sums of large-magnitude rows would move the
            // softmax weights by ~1e-5).  This wave's d/4 terms first.
#pragma unroll
            for (int r = 0; r < SUB; ++r) {
                double s = 0.0;
#pragma unroll
                for (int d = 0; d < DW; d += 4) {
                    const f32x4 kv = *reinterpret_cast<const f32x4*>(ks + r * D + d0 + d);
                    s += (double)qr[d] * (double)kv[0];
                    s += (double)qr[d + 1] * (double)kv[1];
                    s += (double)qr[d + 2] * (double)kv[2];
                    s += (double)qr[d + 3] * (double)kv[3];
                }
                xp[(wave * SUB + r) * 64 + lane] = s;
            }
            __syncthreads();
            double x[SUB];
            double mx = -__builtin_inf();
#pragma unroll
            for (int r = 0; r < SUB; ++r) {
                double s = xp[r * 64 + lane];
#pragma unroll
                for (int u = 1; u < kF32Waves; ++u) s += xp[(u * SUB + r) * 64 + lane];
                x[r] = s * scale2d + (double)kb[r];
                mx = fmax(mx, x[r]);
            }
            if (mx == -__builtin_inf()) continue;  // every column of this step masked
            const double mnew = fmax(m, mx);
            const float alpha = exp2f((float)(m - mnew));
            l *= alpha;
            lpart *= alpha;
#pragma unroll
            for (int d = 0; d < DW; ++d) {
                acc[d] *= alpha;
                part[d] *= alpha;
            }
            m = mnew;
#pragma unroll
            for (int r = 0; r < SUB; ++r) {
                const float p = exp2f((float)(x[r] - m));
                lpart += p;
#pragma unroll
                for (int d = 0; d < DW; d += 4) {
                    const f32x4 vv = *reinterpret_cast<const f32x4*>(vs + r * D + d0 + d);
                    part[d] += p * vv[0];
                    part[d + 1] += p * vv[1];
                    part[d + 2] += p * vv[2];
                    part[d + 3] += p * vv[3];
                }
            }
        }
        l += lpart;
        lpart = 0.f;
#pragma unroll
        for (int d = 0; d < DW; ++d) {
            acc[d] += part[d];
            part[d] = 0.f;
        }
    }

    const int64_t orow = i * 64 + lane;
    if (orow < N) {
        float* op = reinterpret_cast<float*>(a.out) + (bh * N + orow) * D + d0;
        const float inv = 1.0f / l;
#pragma unroll
        for (int d = 0; d < DW; d += 4) {
            f32x4 o = {acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv};
            *reinterpret_cast<f32x4*>(op + d) = o;
        }
    }
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
    const size_t lds = sizeof(float) * f32_lds_floats(a.Nb, a.Nbp, a.d);
    const dim3 grid((unsigned)(a.BH * a.Nb));
    const void* fn = a.d == 128 ? reinterpret_cast<const void*>(&attn_f32_kernel<128>)
                                : reinterpret_cast<const void*>(&attn_f32_kernel<64>);
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (a.d == 128)
        hipLaunchKernelGGL((attn_f32_kernel<128>), grid, dim3(64 * kF32Waves), lds, s, a);
    else
        hipLaunchKernelGGL((attn_f32_kernel<64>), grid, dim3(64 * kF32Waves), lds, s, a);
    return hipGetLastError();
}

}  // namespace solattn
