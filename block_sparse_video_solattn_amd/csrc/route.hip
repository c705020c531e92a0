// Routing alone (steps 1-2 without attention): the same device code the fused
// attention kernels run as their prologue, launched on its own so that the
// routing "setup" can be timed and exported (page "NVIDIA 與 SANA Sol-Engine"
// news, section "技術組成": the pages report Sol-Attn's setup time on its own).
// For fp32 inputs routing reads only the pooled means; for bf16 each query
// block's mean is formed from its rows by the wave that routes it, as the
// fused kernels' prologue forms it.
#include "common.h"
#include "launch.h"
#include "route.h"

namespace solattn {

// One workgroup of G = 4 waves routes G consecutive query blocks of one head.
// The scores of all G blocks are computed together -- wave w takes the key
// columns j = 64w + lane (mod 256) and accumulates the G dot products of
// each column, so every kbarT element read from L2 serves G query blocks --
// with the same per-column arithmetic as the fused kernels' prologue
// (acc = fma(qbar_d, kbar_dj, acc) over ascending d, then the scale), so the
// scores are bit-identical to theirs.  Then wave w runs the selection of
// block i0 + w on its own LDS slice.
constexpr int kRouteG = 4;

template <int D>
__global__ __launch_bounds__(64 * kRouteG) void route_kernel(AttnArgs a) {
    extern __shared__ float smem[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t Nb = a.Nb, Nbp = a.Nbp;
    const int64_t groups = (Nb + kRouteG - 1) / kRouteG;
    const int64_t gw = xcd_remap(blockIdx.x, a.BH * groups);
    const int64_t bh = gw / groups, i0 = (gw % groups) * kRouteG;
    // LDS: scores [G][Nbp] | pooled queries [G][D] | kept lists [G][Nb]
    float* qs = smem + kRouteG * Nbp;
    uint16_t* klists = reinterpret_cast<uint16_t*>(qs + kRouteG * D);
    const int64_t klist_len = (Nb + 15) / 16 * 16;
    if (a.dtype == kBF16) {
        // (wave-uniform branch: each wave forms its own block's mean)
        if (i0 + wave < Nb) {
            const int64_t i = i0 + wave;
            const int n = (int)(a.N - i * 64 < 64 ? a.N - i * 64 : 64);
            QueryRows<D> qr;
            query_rows_load<D>(reinterpret_cast<const bf16*>(a.q) + (bh * a.N + i * 64) * D, n, qr);
            query_rows_mean<D>(qr, n, qs + wave * D);
        } else {
            for (int c = lane; c < D; c += 64) qs[wave * D + c] = 0.f;
        }
    } else {
        for (int e = threadIdx.x; e < kRouteG * D; e += 64 * kRouteG) {
            const int g = e / D, c = e % D;
            qs[e] = i0 + g < Nb ? a.qbar[(bh * Nb + i0 + g) * D + c] : 0.f;
        }
    }
    __syncthreads();
    const float* __restrict__ kt = a.kbarT + bh * D * Nbp;
    const float scale = 1.0f / sqrtf((float)D);
    for (int64_t j = 64 * wave + lane; j < Nbp; j += 64 * kRouteG) {
        float acc[kRouteG];
#pragma unroll
        for (int g = 0; g < kRouteG; ++g) acc[g] = 0.f;
#pragma unroll 16
        for (int d = 0; d < D; ++d) {
            const float kv = kt[(int64_t)d * Nbp + j];
#pragma unroll
            for (int g = 0; g < kRouteG; ++g) acc[g] = __builtin_fmaf(qs[g * D + d], kv, acc[g]);
        }
#pragma unroll
        for (int g = 0; g < kRouteG; ++g) smem[g * Nbp + j] = acc[g] * scale;
    }
    __syncthreads();
    if (i0 + wave < Nb)
        (void)route_select(a, bh, i0 + wave, smem + wave * Nbp, klists + wave * klist_len);
}

hipError_t launch_route(const AttnArgs& a, hipStream_t s) {
    const size_t lds = sizeof(float) * kRouteG * (a.Nbp + a.d) +
                       sizeof(uint16_t) * kRouteG * ((a.Nb + 15) / 16 * 16);
    const dim3 grid((unsigned)(a.BH * ((a.Nb + kRouteG - 1) / kRouteG)));
    // (past 64 KiB -- N above ~120k tokens -- the kernel's dynamic LDS limit
    // is raised to what it needs; gfx950 has 160 KiB per compute unit)
    const void* fn = a.d == 128 ? reinterpret_cast<const void*>(&route_kernel<128>)
                                : reinterpret_cast<const void*>(&route_kernel<64>);
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (a.d == 128)
        hipLaunchKernelGGL((route_kernel<128>), grid, dim3(64 * kRouteG), lds, s, a);
    else
        hipLaunchKernelGGL((route_kernel<64>), grid, dim3(64 * kRouteG), lds, s, a);
    return hipGetLastError();
}

}  // namespace solattn
