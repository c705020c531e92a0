// Launch arguments of the fused Q/K producer (QKNorm then partial RoPE) and
// its pooling epilogue.  Host and device share this header.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace solattn {

struct ProducerArgs {
    const float* gamma_q;   // [d] norm weights, NULL = all ones
    const float* gamma_k;
    const float* rope_cos;  // [N][rope_half] fp32, NULL when rope_half == 0
    const float* rope_sin;
    void* q_out;            // [B][H][N][d], element type of the inputs
    void* k_out;            // same, NULL = not written (bf16 with pooling only)
    float eps;              // > 0
    int rope_half;          // rotated channel pairs: rope_dim / 2
    int vec_tables;         // the tables may be read a thread's pairs at a time
};

// Pooling workspace `a` as launch_pool fills it, computed from the produced
// q', k' instead of the raw inputs (a.q, a.k); with neither a.pooled nor
// a.pack only q' and k' are written (the producer alone).
hipError_t launch_produce_pool(const PoolArgs& a, const ProducerArgs& p, int64_t BH,
                               hipStream_t s);

}  // namespace solattn
