// Step 1 of Sol-Attn: 64-token block pooling (page "NVIDIA 团队开源 Sol-H3 的
// DGX Spark 版本", section "119.68 GiB 的内存池", Sol-Attn item: the pooled
// K/V summaries; page "MiniMax 官宣 NVIDIA Sol 团队 H3 加速", section
// "提速来自流水线每一段的叠加": 64-token query blocks and pooled K/V).
//
// One workgroup (256 threads) per (head slice, 64-token block).  Rows are read
// with fully coalesced 16-byte loads, summed in fp32 in a fixed order, and the
// means written in the layouts the routing and attention kernels read.  For
// bf16 inputs the same pass relays the block's V rows out into the MFMA
// operand order of the attention kernel (a transpose through LDS), so the PV
// contraction reads whole 1 KiB runs per load instruction.
//
// Bound: HBM bandwidth (reads 3 x 64 x d elements per block, writes the value
// tile once more for bf16).
#include "common.h"
#include "launch.h"

namespace solattn {

template <typename T>
struct Vec16;  // 16 bytes of T
template <>
struct Vec16<float> {
    static constexpr int n = 4;
    typedef f32x4 type;
};
template <>
struct Vec16<bf16> {
    static constexpr int n = 8;
    typedef bf16x8 type;
};

template <typename T, int D>
__device__ inline void load_rows(const T* __restrict__ base, int n, int tid,
                                 float (&acc)[Vec16<T>::n], typename Vec16<T>::type* keep) {
    constexpr int VEC = Vec16<T>::n;
    constexpr int CPR = D / VEC;           // 16-byte chunks per row
    constexpr int RPP = 256 / CPR;         // rows per pass
    constexpr int PASSES = 64 / RPP;
    const int c = tid % CPR, r0 = tid / CPR;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = r0 + p * RPP;
        typename Vec16<T>::type x;
        if (r < n) {
            x = *reinterpret_cast<const typename Vec16<T>::type*>(base + (int64_t)r * D + c * VEC);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) x[e] = (T)0.f;
        }
        if (keep) keep[p] = x;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += (float)x[e];
    }
}

// Column sums of the per-thread partials -> block mean in red[0..D) (LDS).
template <typename T, int D>
__device__ inline void reduce_mean(const float (&acc)[Vec16<T>::n], int n, int tid, float* red,
                                   float* mean) {
    constexpr int VEC = Vec16<T>::n;
    constexpr int CPR = D / VEC;
    constexpr int RPP = 256 / CPR;
    const int c = tid % CPR, g = tid / CPR;
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[g * D + c * VEC + e] = acc[e];
    __syncthreads();
    if (tid < D) {
        float s = 0.f;
        for (int gg = 0; gg < RPP; ++gg) s += red[gg * D + tid];
        mean[tid] = s / (float)n;
    }
    __syncthreads();
}

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
    constexpr int VEC = Vec16<T>::n;
    constexpr int CPR = D / VEC;
    constexpr int RPP = 256 / CPR;
    constexpr int PASSES = 64 / RPP;
    __shared__ float red[RPP * D];
    __shared__ float mean[D];
    __shared__ bf16 vt[64][D + 8];  // value tile staging for the relayout (bf16 only)

    const int tid = threadIdx.x;
    const int64_t j = blockIdx.x, bh = blockIdx.y;
    const int64_t Nb = a.Nb, Nbp = a.Nbp, N = a.N;

    if (j >= Nb) {
        // padding of the pooled-key tiles: zero keys and values (their logits
        // are masked to -inf, zeros keep 0 * value finite)
        if (!a.pooled) return;
        if (tid < D) {
            a.kbarT[(bh * D + tid) * Nbp + j] = 0.f;
            if (a.dtype == kBF16) {
                reinterpret_cast<bf16*>(a.kbar16)[(bh * Nbp + j) * D + tid] = (bf16)0.f;
                int s, half, e, kk = (int)(j & 63);
                vtile_slot(kk, &s, &half, &e);
                const int mt = tid / 32, lane = 32 * half + (tid & 31);
                reinterpret_cast<bf16*>(a.vbarP)[(bh * (Nbp / 64) + j / 64) * D * 64 +
                                                 vtile_offset(mt, s, lane, e)] = (bf16)0.f;
            }
        }
        return;
    }

    const int n = (int)((j + 1) * 64 <= N ? 64 : N - j * 64);
    const int64_t row0 = bh * N + j * 64;
    float acc[VEC];

    if (a.pooled) {
        // Q
        load_rows<T, D>(reinterpret_cast<const T*>(a.q) + row0 * D, n, tid, acc, nullptr);
        reduce_mean<T, D>(acc, n, tid, red, mean);
        if (tid < D) a.qbar[(bh * Nb + j) * D + tid] = mean[tid];
        // K
        load_rows<T, D>(reinterpret_cast<const T*>(a.k) + row0 * D, n, tid, acc, nullptr);
        reduce_mean<T, D>(acc, n, tid, red, mean);
        if (tid < D) {
            const float m = mean[tid];
            a.kbar[(bh * Nb + j) * D + tid] = m;
            a.kbarT[(bh * D + tid) * Nbp + j] = m;
            if (a.dtype == kBF16) reinterpret_cast<bf16*>(a.kbar16)[(bh * Nbp + j) * D + tid] = to_bf16(m);
        }
    }
    // V (means and/or the operand-ordered tile)
    typename Vec16<T>::type keep[PASSES];
    load_rows<T, D>(reinterpret_cast<const T*>(a.v) + row0 * D, n, tid, acc, keep);
    if (a.pooled) {
        reduce_mean<T, D>(acc, n, tid, red, mean);
        if (tid < D) {
            const float m = mean[tid];
            a.vbar[(bh * Nb + j) * D + tid] = m;
            if (a.dtype == kBF16) {
                int s, half, e, kk = (int)(j & 63);
                vtile_slot(kk, &s, &half, &e);
                const int mt = tid / 32, lane = 32 * half + (tid & 31);
                reinterpret_cast<bf16*>(a.vbarP)[(bh * (Nbp / 64) + j / 64) * D * 64 +
                                                 vtile_offset(mt, s, lane, e)] = to_bf16(m);
            }
        }
    }
    if constexpr (sizeof(T) == 2) {
        if (a.pack_v) {
            const int c = tid % CPR, r0 = tid / CPR;
#pragma unroll
            for (int p = 0; p < PASSES; ++p) {
                const int r = r0 + p * RPP;
#pragma unroll
                for (int e = 0; e < VEC; ++e) vt[r][c * VEC + e] = keep[p][e];
            }
            __syncthreads();
            // 16-byte output groups: D*64/8 of them, consecutive threads write
            // consecutive groups
            bf16* dst = reinterpret_cast<bf16*>(a.vP) + (bh * Nb + j) * (int64_t)D * 64;
            for (int gidx = tid; gidx < D * 8; gidx += 256) {
                const int lane = gidx & 63, ms = gidx >> 6;
                const int mt = ms >> 2, s = ms & 3;
                const int dcol = 32 * mt + (lane & 31), half = lane >> 5;
                bf16x8 o;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = vt[vtile_key(s, half, e)][dcol];
                *reinterpret_cast<bf16x8*>(dst + gidx * 8) = o;
            }
        }
    }
}

hipError_t launch_pool(const PoolArgs& a, int64_t BH, hipStream_t s) {
    const dim3 grid((unsigned)(a.pooled ? a.Nbp : a.Nb), (unsigned)BH);
    if (a.dtype == kBF16) {
        if (a.d == 128)
            hipLaunchKernelGGL((pool_kernel<bf16, 128>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((pool_kernel<bf16, 64>), grid, dim3(256), 0, s, a);
    } else {
        if (a.d == 128)
            hipLaunchKernelGGL((pool_kernel<float, 128>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((pool_kernel<float, 64>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace solattn
