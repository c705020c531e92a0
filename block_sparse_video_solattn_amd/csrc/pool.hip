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

// Relayout of one staged 64-row tile (LDS, row-major, zero rows past the
// block) into MFMA operand order; consecutive threads write consecutive
// 16-byte groups.
template <int D>
__device__ inline void write_key_tile(const bf16 (*tile)[D + 8], bf16* dst, int tid) {
    constexpr int KS = D / 16;
    for (int g = tid; g < D * 8; g += 256) {
        const int lane = g & 63, us = g >> 6;
        const int u = us / KS, s = us % KS;
        const int row = 32 * u + (lane & 31), col = 16 * s + 8 * (lane >> 5);
        *reinterpret_cast<bf16x8*>(dst + g * 8) = *reinterpret_cast<const bf16x8*>(&tile[row][col]);
    }
}

template <int D>
__device__ inline void write_value_tile(const bf16 (*tile)[D + 8], bf16* dst, int tid) {
    for (int g = tid; g < D * 8; g += 256) {
        const int lane = g & 63, ms = g >> 6;
        const int mt = ms >> 2, s = ms & 3;
        const int dcol = 32 * mt + (lane & 31), half = lane >> 5;
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = tile[vtile_key(s, half, e)][dcol];
        *reinterpret_cast<bf16x8*>(dst + g * 8) = o;
    }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
    constexpr int VEC = Vec16<T>::n;
    constexpr int CPR = D / VEC;
    constexpr int RPP = 256 / CPR;
    constexpr int PASSES = 64 / RPP;
    constexpr int KS = D / 16;
    __shared__ float red[RPP * D];
    __shared__ float mean[D];
    __shared__ bf16 tile[64][D + 8];  // staging for the operand relayout (bf16 only)

    const int tid = threadIdx.x;
    const int64_t j = blockIdx.x, bh = blockIdx.y;
    const int64_t Nb = a.Nb, Nbp = a.Nbp, N = a.N;
    const bool bf = a.dtype == kBF16;

    // pooled-operand slot of pooled key j (tile j/64, key j%64 of that tile)
    const int kk = (int)(j & 63);
    bf16* kbarP = bf ? reinterpret_cast<bf16*>(a.kbarP) + (bh * (Nbp / 64) + j / 64) * D * 64 : nullptr;
    bf16* vbarP = bf ? reinterpret_cast<bf16*>(a.vbarP) + (bh * (Nbp / 64) + j / 64) * D * 64 : nullptr;
    auto put_pooled = [&](int dcol, float km, float vm) {
        // key: row kk of the tile, column dcol
        const int s = dcol / 16, half = (dcol / 8) & 1, e = dcol & 7;
        kbarP[ktile_offset(KS, kk / 32, s, 32 * half + (kk & 31), e)] = to_bf16(km);
        int vs, vh, ve;
        vtile_slot(kk, &vs, &vh, &ve);
        vbarP[vtile_offset(dcol / 32, vs, 32 * vh + (dcol & 31), ve)] = to_bf16(vm);
    };

    if (j >= Nb) {
        // padding of the pooled tiles: zero keys and values (their logits are
        // masked to -inf; zeros keep 0 * value finite)
        if (!a.pooled) return;
        if (tid < D) {
            a.kbarT[(bh * D + tid) * Nbp + j] = 0.f;
            if (bf) put_pooled(tid, 0.f, 0.f);
        }
        return;
    }

    const int n = (int)((j + 1) * 64 <= N ? 64 : N - j * 64);
    const int64_t row0 = bh * N + j * 64;
    const bool pack = bf && a.pack;
    float acc[VEC];
    typename Vec16<T>::type keep[PASSES];
    auto stage = [&]() {
        const int c = tid % CPR, r0 = tid / CPR;
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
#pragma unroll
            for (int e = 0; e < VEC; ++e) tile[r0 + p * RPP][c * VEC + e] = (bf16)keep[p][e];
    };

    if (a.pooled) {
        load_rows<T, D>(reinterpret_cast<const T*>(a.q) + row0 * D, n, tid, acc, nullptr);
        reduce_mean<T, D>(acc, n, tid, red, mean);
        if (tid < D) a.qbar[(bh * Nb + j) * D + tid] = mean[tid];
    }
    // K: means, and the operand-ordered key tile
    if (a.pooled || pack) {
        load_rows<T, D>(reinterpret_cast<const T*>(a.k) + row0 * D, n, tid, acc, keep);
        if (a.pooled) {
            reduce_mean<T, D>(acc, n, tid, red, mean);
            if (tid < D) {
                a.kbar[(bh * Nb + j) * D + tid] = mean[tid];
                a.kbarT[(bh * D + tid) * Nbp + j] = mean[tid];
            }
        }
        if (pack) {
            stage();
            __syncthreads();
            write_key_tile<D>(tile, reinterpret_cast<bf16*>(a.kP) + (bh * Nb + j) * (int64_t)D * 64, tid);
            __syncthreads();
        }
    }
    // V: means, and the operand-ordered value tile
    load_rows<T, D>(reinterpret_cast<const T*>(a.v) + row0 * D, n, tid, acc, keep);
    if (a.pooled) {
        const float km = tid < D ? mean[tid] : 0.f;  // K mean, still in LDS
        __syncthreads();
        reduce_mean<T, D>(acc, n, tid, red, mean);
        if (tid < D) {
            a.vbar[(bh * Nb + j) * D + tid] = mean[tid];
            if (bf) put_pooled(tid, km, mean[tid]);
        }
    }
    if (pack) {
        stage();
        __syncthreads();
        write_value_tile<D>(tile, reinterpret_cast<bf16*>(a.vP) + (bh * Nb + j) * (int64_t)D * 64, tid);
    }
}

hipError_t launch_pool(const PoolArgs& a, int64_t BH, hipStream_t s) {
    const dim3 grid((unsigned)(a.pooled ? a.Nbp : a.Nb), (unsigned)BH);
    if (a.dtype != kBF16 && !a.pooled) return hipSuccess;
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
