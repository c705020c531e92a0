// In-run peak probe for the bf16 matrix cores: every wave keeps eight
// independent 32x32x16 bf16 MFMA accumulation chains busy from register
// operands, with no memory traffic in the loop.  The achieved FLOP rate of a
// launch that fills the GPU is the practical MFMA ceiling that the attention
// kernel's roofline fraction can be read against (the published dense peak
// assumes the 2.4 GHz peak clock).
#include "common.h"
#include "launch.h"

namespace solattn {

namespace {

__global__ __launch_bounds__(64, 1) void probe_mfma_kernel(float* __restrict__ sink, int64_t iters) {
    const int lane = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (bf16)(0.001f * (float)((lane * 8 + e) % 17));
        b[e] = (bf16)(0.001f * (float)((lane * 3 + e) % 13));
    }
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[c][v];
    sink[(int64_t)blockIdx.x * 64 + lane] = s;
}

}  // namespace

hipError_t launch_probe_mfma(float* sink, int64_t waves, int64_t iters, hipStream_t s) {
    hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)waves), dim3(64), 0, s, sink, iters);
    return hipGetLastError();
}

}  // namespace solattn
