// Steps 2-5 of Sol-Attn for bf16 inputs: routing, exact attention on kept
// 64x64 tiles, one pooled term per skipped block, all inside one online
// softmax (page "NVIDIA 团队开源 Sol-H3 的 DGX Spark 版本", section "119.68 GiB
// 的内存池", Sol-Attn item; page "MiniMax 官宣 NVIDIA Sol 团队 H3 加速",
// section "提速来自流水线每一段的叠加").
//
// Work decomposition (gfx950, wave64):
//   * one workgroup = one wavefront = one (head slice, 64-row query block);
//     the routing granularity fixes the query tile at 64 rows, and holding
//     all 64 rows in one wave gives every K/V element loaded into registers
//     64 rows of reuse;
//   * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16 with
//     fp32 accumulation.  Q^T is parked in LDS in operand order.  Key and
//     value tiles come pre-arranged in A-operand order from the pooling pass,
//     so every operand load reads a contiguous 1 KiB run, and P^T is the S^T
//     accumulator converted to bf16 with no lane shuffles;
//   * each 64-key tile is consumed as two 32-key halves; a half's values are
//     fetched behind its S^T products and the next half's keys behind its
//     softmax, so keys and values are never live at once next to the 64 x d
//     fp32 output accumulator;
//   * skipped blocks enter as "pooled tiles": 64 pooled keys kbar_j (bf16)
//     with logit bias log2(n_j), or -inf where block j is kept or padding.
//     The pooled term n_j exp(c q.kbar_j) vbar_j is exactly a softmax column
//     with logit c q.kbar_j + ln n_j, so it shares the MFMA body and the
//     online-softmax state with the exact tiles;
//   * the online softmax runs in log2 units (exp2) with a lazy rescale: the
//     reference maximum moves only when the row maximum grows by more than
//     2^8, which keeps P <= 256 in bf16 and skips most rescales of the
//     accumulators.  The denominator adds the bf16-rounded weights the MFMA
//     consumes (v_dot2 against (1, 1)), so numerator and denominator agree;
//   * workgroups are remapped so that the query blocks of one head run on
//     one XCD and share its L2 for the K/V tiles they keep.
#include "common.h"
#include "launch.h"
#include "route.h"

namespace solattn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;

// One 32-key half of a 64-key tile (exact block or pooled tile).
struct Half {
    const bf16* ktile;  // operand-ordered key tile
    const bf16* vtile;  // operand-ordered value tile
    int u;              // which half (0, 1)
    int kind;           // 0 exact, 1 exact with masked keys, 2 pooled
    int nvalid;         // kind 1: valid keys in this half (1..31)
    int bias_off;       // kind 2: srow index of key 0 of this half
};

template <int D>
__device__ inline void load_k(const Half& h, int lane, bf16x8 (&kA)[D / 16]) {
    constexpr int KS = D / 16;
#pragma unroll
    for (int s = 0; s < KS; ++s)
        kA[s] = *reinterpret_cast<const bf16x8*>(h.ktile + ktile_offset(KS, h.u, s, lane, 0));
}

template <int D>
__device__ inline void load_v(const Half& h, int lane, bf16x8 (&vA)[D / 32][2]) {
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int s = 0; s < 2; ++s)
            vA[mt][s] = *reinterpret_cast<const bf16x8*>(h.vtile +
                                                         vtile_offset(mt, 2 * h.u + s, lane, 0));
}

}  // namespace

template <int D>
__global__ __launch_bounds__(64, 1) void attn_bf16_kernel(AttnArgs a) {
    constexpr int KS = D / 16;  // k-steps of S^T = K Q^T
    constexpr int MT = D / 32;  // 32-row d tiles of O^T
    extern __shared__ float smem[];

    const int lane = threadIdx.x, half = lane >> 5, l32 = lane & 31;
    const int64_t N = a.N, Nb = a.Nb, Nbp = a.Nbp;
    const int64_t w = xcd_remap(blockIdx.x, a.BH * Nb);
    const int64_t bh = w / Nb, i = w % Nb;
    float* srow = smem;
    uint16_t* klist = reinterpret_cast<uint16_t*>(smem + Nbp);
    bf16x8* qs = reinterpret_cast<bf16x8*>(smem + Nbp + (Nb + 15) / 16 * 8);

    int n_kept;
    uint64_t tile_mask;
    if (a.mode == kSparse) {
        const RouteResult r = route_query_block<D>(a, bh, i, srow, klist);
        n_kept = r.n_kept;
        tile_mask = r.tile_mask;
    } else {
        export_dense_route(a, bh, i);
        n_kept = (int)Nb;
        tile_mask = 0;
    }

    const bf16* qp = reinterpret_cast<const bf16*>(a.q) + bh * N * D;
    const bf16* kp = reinterpret_cast<const bf16*>(a.kP) + bh * Nb * D * 64;
    const bf16* vp = reinterpret_cast<const bf16*>(a.vP) + bh * Nb * D * 64;
    const bf16* kbp = reinterpret_cast<const bf16*>(a.kbarP) + bh * Nbp * D;
    const bf16* vbp = reinterpret_cast<const bf16*>(a.vbarP) + bh * Nbp * D;
    const int tail = (int)(N - (Nb - 1) * 64);  // keys in the last block (1..64)

    // Q^T as the B operand of S^T = K Q^T, parked in LDS in operand order:
    // 16-byte slot (nt*KS + s)*64 + lane holds query 32*nt + l32,
    // d = 16*s + 8*half .. +7; read back with conflict-free ds_read_b128.
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        int64_t row = i * 64 + 32 * nt + l32;
        if (row > N - 1) row = N - 1;
        const bf16* qrow = qp + row * D + 8 * half;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qs[(nt * KS + s) * 64 + lane] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
    }
    __syncthreads();

    f32x16 oacc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int v = 0; v < 16; ++v) oacc[mt][nt][v] = 0.f;
    float mref[2] = {-__builtin_inff(), -__builtin_inff()};
    float lsum[2] = {0.f, 0.f};
    const float scale2 = kLog2e / sqrtf((float)D);
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    // Sequence of halves: exact tiles in kept-list order, then the pooled
    // tiles holding a skipped block in ascending order.  An exact tail tile of
    // <= 32 keys has only its first half.
    const int n_tiles = n_kept + __popcll(tile_mask);
    // (the kept-list entry is wave-uniform: readfirstlane keeps the tile
    // pointers in scalar registers)
    auto exact_block = [&](int t) -> int64_t {
        return (a.mode == kSparse) ? (int64_t)__builtin_amdgcn_readfirstlane((int)klist[t])
                                   : (int64_t)t;
    };
    auto half_at = [&](int t, int u, int T) -> Half {
        Half h;
        h.u = u;
        if (t < n_kept) {
            const int64_t j = exact_block(t);
            const int nv = ((j == Nb - 1) ? tail : 64) - 32 * u;
            h.ktile = kp + j * (int64_t)D * 64;
            h.vtile = vp + j * (int64_t)D * 64;
            h.kind = nv < 32 ? 1 : 0;
            h.nvalid = nv;
            h.bias_off = 0;
        } else {
            h.ktile = kbp + (int64_t)T * D * 64;
            h.vtile = vbp + (int64_t)T * D * 64;
            h.kind = 2;
            h.nvalid = 32;
            h.bias_off = 64 * T + 32 * u;
        }
        return h;
    };
    auto halves_of = [&](int t) -> int {
        return (t < n_kept && exact_block(t) == Nb - 1 && tail <= 32) ? 1 : 2;
    };

    uint64_t ptm = tile_mask;  // pooled tiles not yet finished
    int t = 0, u = 0, pT = ptm ? __builtin_ctzll(ptm) : 0;
    bf16x8 kA[KS];
    bf16x8 vA[MT][2];
    Half h = half_at(0, 0, pT);
    load_k<D>(h, lane, kA);

    while (t < n_tiles) {
        // which half comes next
        int tn = t, un = u + 1, pTn = pT;
        if (un >= halves_of(t)) {
            tn = t + 1;
            un = 0;
            if (t >= n_kept) {  // leaving pooled tile pT
                ptm &= ptm - 1;
                pTn = ptm ? __builtin_ctzll(ptm) : 0;
            }
        }
        const bool more = tn < n_tiles;
        const Half hn = more ? half_at(tn, un, pTn) : h;

        // keep the Q operand reads inside the loop (no hoisting into VGPRs)
        __asm__ volatile("" ::: "memory");
        // S^T = K Q^T: 32 keys x 64 queries, two 32x32 accumulators
        f32x16 st[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int v = 0; v < 16; ++v) st[nt][v] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 q0 = qs[s * 64 + lane];
            const bf16x8 q1 = qs[(KS + s) * 64 + lane];
            st[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kA[s], q0, st[0], 0, 0, 0);
            st[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kA[s], q1, st[1], 0, 0, 0);
        }
        // this half's values, needed after the softmax (the scheduling barrier
        // keeps the loads behind the S^T products)
        __builtin_amdgcn_sched_barrier(0);
        load_v<D>(h, lane, vA);

        // Logits in log2 units are st * sc (+ bias).  Pooled halves add the
        // per-key bias log2(n_j) / -inf here (sc becomes 1); the exact tail
        // masks keys past the block; exact halves keep the raw scores and
        // fold the scale into the exp2 argument.  Register v holds key
        // 8*(v/4) + 4*half + v%4 of this half.
        float sc = scale2;
        if (h.kind == 2) {
            const float* b = srow + h.bias_off + 4 * half;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 bb = *reinterpret_cast<const f32x4*>(b + 8 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        st[nt][4 * g + r] = st[nt][4 * g + r] * scale2 + bb[r];
            }
            sc = 1.0f;
        } else if (h.kind == 1) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = 8 * (v >> 2) + 4 * half + (v & 3);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    if (key >= h.nvalid) st[nt][v] = -__builtin_inff();
            }
        }

        // online softmax of both query halves -> P^T (bf16), the B operand of
        // the PV product: k-step s holds keys 16*s + 4*half + {0..3, 8..11} of
        // this half = accumulator registers 8*s .. 8*s+7
        bf16x8 pB[2][2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            float mx = fmaxf(st[nt][0], st[nt][1]);
#pragma unroll
            for (int v = 2; v < 16; v += 2) mx = fmaxf(mx, fmaxf(st[nt][v], st[nt][v + 1]));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sc;
            const float mcand = fmaxf(mref[nt], mx);
            const bool grow = mcand > mref[nt] + kRescaleSlack;
            if (__ballot(grow)) {
                const float mnew = grow ? mcand : mref[nt];
                const float alpha = __builtin_amdgcn_exp2f(mref[nt] - mnew);
                lsum[nt] *= alpha;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int v = 0; v < 16; ++v) oacc[mt][nt][v] *= alpha;
                mref[nt] = mnew;
            }
            // (A pooled half whose keys are all kept blocks has only -inf
            // logits; while no finite logit has been seen, subtract 0 so that
            // such a half yields p = 0 rather than exp2(-inf + inf).)
            const float msub = mref[nt] == -__builtin_inff() ? 0.f : mref[nt];
            float ps = lsum[nt];
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
                f32x2 pp;
                pp[0] = __builtin_amdgcn_exp2f(st[nt][v] * sc - msub);
                pp[1] = __builtin_amdgcn_exp2f(st[nt][v + 1] * sc - msub);
                const bf16x2 pr = __builtin_convertvector(pp, bf16x2);
                ps = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps, false);
                pB[nt][v >> 3][v & 7] = pr[0];
                pB[nt][v >> 3][(v & 7) + 1] = pr[1];
            }
            lsum[nt] = ps;
        }

        // the K registers are free: fetch the next half's keys while the PV
        // products run
        __builtin_amdgcn_sched_barrier(0);
        if (more) load_k<D>(hn, lane, kA);

        // O^T += V^T P^T
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    oacc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vA[mt][s], pB[nt][s],
                                                                           oacc[mt][nt], 0, 0, 0);
        h = hn;
        t = tn;
        u = un;
        pT = pTn;
    }

    // epilogue: O = acc / l, rounded to bf16; lane holds query 32*nt + l32 and
    // d = 32*mt + 8*g + 4*half + r
    bf16* op = reinterpret_cast<bf16*>(a.out) + bh * N * D;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const float l = lsum[nt] + __shfl_xor(lsum[nt], 32, 64);
        const float inv = 1.0f / l;
        const int64_t row = i * 64 + 32 * nt + l32;
        if (row < N) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    bf16x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = to_bf16(oacc[mt][nt][4 * g + r] * inv);
                    *reinterpret_cast<bf16x4*>(op + row * D + 32 * mt + 8 * g + 4 * half) = o;
                }
        }
    }
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
    const size_t lds = sizeof(float) * (a.Nbp + (a.Nb + 15) / 16 * 8) + 2 * 64 * (size_t)a.d;
    const dim3 grid((unsigned)(a.BH * a.Nb));
    if (a.d == 128)
        hipLaunchKernelGGL((attn_bf16_kernel<128>), grid, dim3(64), lds, s, a);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<64>), grid, dim3(64), lds, s, a);
    return hipGetLastError();
}

}  // namespace solattn
