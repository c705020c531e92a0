// Launch of the first-order (Taylor) accuracy mode of the bf16 attention
// kernel (the kernel lives with the other bf16 attention code).
#pragma once
#include <hip/hip_runtime.h>

#include "launch.h"

namespace solattn {

// Steps 2-5 with the first-order term of every skipped block; a.mode must
// be kSparse and the workspace must hold the bf16 pooling pass's output.
hipError_t launch_attn_bf16_taylor(const AttnArgs& a, hipStream_t s);

}  // namespace solattn
