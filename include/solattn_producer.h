/*
 * solattn_producer.h -- the Q/K producer of Sol-Attn fused with its block
 * pooling (AMD Instinct MI355X, gfx950).
 *
 * The pages list "QKNorm + partial RoPE" among the chains the engine fuses so
 * that their intermediates stay on chip instead of making extra HBM round
 * trips (page "MiniMax 官宣 NVIDIA Sol 团队 H3 加速:5 秒视频 1.653 秒生成并
 * 开源", section "提速来自流水线每一段的叠加", fused-operator item; page
 * "NVIDIA 與 SANA Sol-Engine" news, section "技術組成": QKNorm + RoPE among the
 * fused lossless kernels).  Neither page fixes the norm's parameters or the
 * rotary layout; this library reads them as:
 *
 *   QKNorm: per token and head, over the d channels,
 *     y_c = x_c / sqrt(mean_c'(x_c'^2) + eps) * gamma_c,
 *   with one weight vector gamma (length d, shared by all heads; NULL = all
 *   ones) for Q and another for K.
 *   Partial RoPE: afterwards the first rope_dim channels turn in adjacent
 *   pairs (2i, 2i+1), i < rope_dim/2, by the angle tabulated for the row's
 *   token t (t = 0 .. N-1, the same for every batch entry and head):
 *     (y_2i, y_2i+1) -> (y_2i c - y_2i+1 s, y_2i s + y_2i+1 c),
 *   c = rope_cos[t][i], s = rope_sin[t][i]; channels rope_dim .. d-1 pass
 *   through.  (A model that pairs channels differently, e.g. i with
 *   i + rope_dim/2, maps onto this by permuting its Q/K projection rows.)
 *
 * Arithmetic in fp32, one rounding to the element type at the end (bf16:
 * nearest, ties to even).  All other conventions (shapes, dtypes, streams,
 * host-side checks, return codes, workspace rules) are those of solattn.h.
 * Additionally:
 *   - gamma_q, gamma_k: device fp32 [d], 4-byte aligned, or NULL.
 *   - eps: finite and > 0.
 *   - rope_dim: even, 0 <= rope_dim <= d.  rope_cos, rope_sin: device fp32
 *     [N][rope_dim/2] row-major, 4-byte aligned; ignored (may be NULL) when
 *     rope_dim is 0.
 *   - q_out, k_out: caller-owned device [B][H][N][d] tensors of `dtype`,
 *     16-byte aligned, overlapping neither each other nor any input.
 *   - The kernel reads the tables four entries at a time when rope_dim/2 is
 *     a multiple of four (two for fp32) and both tables are aligned to that
 *     many floats; results do not depend on it.
 */
#ifndef SOLATTN_PRODUCER_H
#define SOLATTN_PRODUCER_H

#include <stddef.h>
#include <stdint.h>

#include "solattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The producer alone: q_out = RoPE(QKNorm_q(q)), k_out = RoPE(QKNorm_k(k)).
 * Reads q and k once and writes q_out and k_out once (no pooling, no
 * workspace).  q_out and k_out are required.
 */
int solattn_qknorm_rope(const void* q, const void* k, const float* gamma_q,
                        const float* gamma_k, float eps, int64_t rope_dim,
                        const float* rope_cos, const float* rope_sin, void* q_out, void* k_out,
                        int64_t B, int64_t H, int64_t N, int64_t d, int dtype, void* stream);

/*
 * The producer fused with step 1 (pooling) in one pass over q, k and v:
 * writes q_out (and k_out, if given) as solattn_qknorm_rope does and leaves
 * in `ws` exactly what solattn_prepare_ws(q_out, k_out, v, ...) would leave
 * there, bit for bit, without reading q_out or k_out back.  solattn_attend_ws
 * (q_out, k_out, v, out, ...) on the same ws then completes the forward pass.
 * k_out may be NULL for bf16 (the attention reads keys from the workspace);
 * fp32 needs it (the fp32 attention reads k directly).  `mode` is as for
 * solattn_prepare_ws.
 */
int solattn_prepare_qknorm_rope_ws(const void* q, const void* k, const void* v,
                                   const float* gamma_q, const float* gamma_k, float eps,
                                   int64_t rope_dim, const float* rope_cos,
                                   const float* rope_sin, void* q_out, void* k_out, int64_t B,
                                   int64_t H, int64_t N, int64_t d, int mode, int dtype,
                                   void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SOLATTN_PRODUCER_H */
