// Routing alone (steps 1-2 without attention; page "NVIDIA 與 SANA
// Sol-Engine" news, section "技術組成", reports Sol-Attn's setup time on its
// own): the same device code the fused attention kernels run as their
// prologue, launched on its own so that the routing can be timed and
// exported -- and ahead of a planned attention launch, for which it also
// writes each query block's keep bits and tile count to the workspace (the
// order kernel below then fixes the dispatch order from the counts).
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
    if (i0 + wave < Nb) {
        const RouteResult r =
            route_select(a, bh, i0 + wave, smem + wave * Nbp, klists + wave * klist_len);
        // tiles the attention kernel will run for this block: kept blocks
        // plus pooled tiles (the dispatch order's cost estimate)
        if (a.plan_cost && lane == 0)
            a.plan_cost[bh * Nb + i0 + wave] = r.n_kept + __popcll(r.tile_mask);
    }
}

// Dispatch order of a planned attention launch.  The launch gives XCD x the
// contiguous range of launch positions xcd_remap assigns it; position p runs
// work item plan_perm[p].  Within the part of one head that falls in one
// XCD's range, items are placed in decreasing tile count (ties: ascending
// index), longest-processing-time-first list scheduling: the XCD's compute
// units take positions in order as they free up, so its last dispatch round
// holds its shortest items instead of whichever items the sequence put last.
// Items of one head stay together, so the head's key/value tiles stay shared
// in that XCD's L2.  With dense prefix rows the range's prefix query blocks
// (every key block exact, several times a routed block's tiles) come first,
// in head order, ahead of every head's routed blocks, as in the fused
// launch's order.  One workgroup ranks 256 items of one head against the
// head's counts in LDS; four threads share each item's comparisons, a
// quarter of its range each, and their counts are added in LDS.
constexpr int kOrderItems = 256, kOrderParts = 4;

__global__ __launch_bounds__(kOrderItems * kOrderParts) void order_kernel(AttnArgs a) {
    extern __shared__ int32_t cnt[];  // counts [Nb] | partial ranks [parts][items]
    // (B*H*Nb < 2^31 is checked on the host: 32-bit indices)
    const int Nb = (int)a.Nb, T = (int)(a.BH * a.Nb);
    const int Pb = (a.prefix_rows && a.Pb < a.Nb) ? (int)a.Pb : 0;  // heavy items: e < Pb
    const int chunks = (Nb + kOrderItems - 1) / kOrderItems;
    const int bh = (int)blockIdx.x / chunks, h0 = bh * Nb;
    for (int e = threadIdx.x; e < Nb; e += kOrderItems * kOrderParts) cnt[e] = a.plan_cost[h0 + e];
    __syncthreads();
    const int item = (int)threadIdx.x % kOrderItems, part = (int)threadIdx.x / kOrderItems;
    const int e = ((int)blockIdx.x % chunks) * kOrderItems + item;
    const bool valid = e < Nb;
    // the XCD range holding position h0 + e (xcd_remap: 8 ranges, the first
    // T % 8 of them one position longer), clipped to this head
    const int g = h0 + e, q = T / 8, m = T % 8;
    const int x = g < m * (q + 1) ? g / (q + 1) : m + (g - m * (q + 1)) / (q > 0 ? q : 1);
    const int x_lo = x * q + (x < m ? x : m), x_hi = x_lo + q + (x < m ? 1 : 0);
    const int lo = (x_lo > h0 ? x_lo : h0) - h0;
    const int hi = (x_hi < h0 + Nb ? x_hi : h0 + Nb) - h0;
    // items of the range ahead of e: by decreasing count within the head,
    // this thread's quarter [f0, f1) of [lo, hi)
    int ahead = 0;
    if (valid && e >= Pb) {
        const int32_t c = cnt[e];
        const int f0 = lo + (hi - lo) * part / kOrderParts;
        const int f1 = lo + (hi - lo) * (part + 1) / kOrderParts;
        // (the lanes of a wave read the same count at once: LDS broadcasts;
        // unrolled so that several reads are in flight)
#pragma unroll 8
        for (int f = f0; f < f1; ++f) {
            const int32_t cf = cnt[f];
            ahead += (f >= Pb) & ((cf > c) | ((cf == c) & (f < e)));
        }
    }
    int32_t* pr = cnt + Nb;
    pr[part * kOrderItems + item] = ahead;
    __syncthreads();
    if (!valid || part != 0) return;
    // heavy items among the first n items of the launch, and in this range
    auto heavy_before = [&](int n) { return n / Nb * Pb + (n % Nb < Pb ? n % Nb : Pb); };
    const int hx = heavy_before(x_hi) - heavy_before(x_lo);
    int pos;
    if (e < Pb) {
        pos = x_lo + heavy_before(g) - heavy_before(x_lo);
    } else {
        // after the range's heavy items and the other items of earlier heads
        // in the range
        const int s0 = h0 + lo;
        pos = x_lo + hx + (s0 - x_lo) - (heavy_before(s0) - heavy_before(x_lo));
#pragma unroll
        for (int u = 0; u < kOrderParts; ++u) pos += pr[u * kOrderItems + item];
    }
    a.plan_perm[pos] = g;
}

hipError_t launch_order(const AttnArgs& a, hipStream_t s) {
    const size_t lds = sizeof(int32_t) * (a.Nb + kOrderItems * kOrderParts);
    const dim3 grid((unsigned)(a.BH * ((a.Nb + kOrderItems - 1) / kOrderItems)));
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&order_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(order_kernel, grid, dim3(kOrderItems * kOrderParts), lds, s, a);
    return hipGetLastError();
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
