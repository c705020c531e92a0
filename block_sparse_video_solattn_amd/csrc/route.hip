// Routing alone (steps 1-2 without attention): the same device code the fused
// attention kernels run as their prologue, launched on its own so that the
// routing "setup" can be timed and exported (page "NVIDIA 與 SANA Sol-Engine"
// news, section "技術組成": the pages report Sol-Attn's setup time on its own).
// Routing reads only the fp32 pooled means, so one kernel serves both dtypes.
#include "common.h"
#include "launch.h"
#include "route.h"

namespace solattn {

template <int D>
__global__ __launch_bounds__(64) void route_kernel(AttnArgs a) {
    extern __shared__ float smem[];
    const int64_t Nb = a.Nb;
    const int64_t w = xcd_remap(blockIdx.x, a.BH * Nb);
    const int64_t bh = w / Nb, i = w % Nb;
    (void)route_query_block<D>(a, bh, i, smem, reinterpret_cast<uint16_t*>(smem + a.Nbp));
}

hipError_t launch_route(const AttnArgs& a, hipStream_t s) {
    const size_t lds = sizeof(float) * (a.Nbp + (a.Nb + 15) / 16 * 8);
    const dim3 grid((unsigned)(a.BH * a.Nb));
    if (a.d == 128)
        hipLaunchKernelGGL((route_kernel<128>), grid, dim3(64), lds, s, a);
    else
        hipLaunchKernelGGL((route_kernel<64>), grid, dim3(64), lds, s, a);
    return hipGetLastError();
}

}  // namespace solattn
