/*
 * solattn_transport.h -- the one-GPU half of the sequence-parallel exchange
 * around Sol-Attn, for AMD Instinct MI355X (gfx950).
 *
 * With P GPUs each holding a sequence shard of Q/K/V for every head, Q/K/V
 * are packed per destination GPU and exchanged with one all-to-all, so that
 * each GPU holds every token of H/P heads; the attention output goes back the
 * same way.  The fastest setting sends Q/K/V as INT8 with block quantization
 * and the output as FP8 (page "MiniMax 官宣 NVIDIA Sol 团队 H3 加速:5 秒视频
 * 1.653 秒生成并开源", section "提速来自流水线每一段的叠加", multi-GPU item),
 * in records aligned from 132 to 144 bytes (page "英伟达开源 Sol-H3，给 MiniMax-H3
 * 加速，5 秒视频 1.4 秒出", section "2.2 剩下三层加速").  These calls are the
 * packing and unpacking kernels; the exchange itself (an all-to-all of
 * equal chunks, chunk p of rank s's send buffer arriving as chunk s of rank
 * p's receive buffer) is the caller's.
 *
 * Record: one token's d-vector of one head: d codes, the fp32 scale, zero
 * bytes up to a multiple of 16 (solattn_transport_record_bytes: 144 at
 * d = 128, 80 at d = 64).
 *   INT8 (Q/K/V): s = amax / 127 and inv = 127 / amax (fp32 divisions,
 *     nearest even), code = clamp(rint(x * inv), -127, 127) with x * inv an
 *     fp32 product; amax = max |x| over the row; a zero row has s = 0.
 *   FP8 (output): OCP E4M3 (bias 7, largest finite 448); s = amax / 448,
 *     inv = 448 / amax, code = E4M3 of clamp(x * inv, -448, 448), nearest
 *     even.
 *   Unpacking: bf16 of the fp32 product code * s (nearest even).
 *
 * All tensors are bf16, contiguous, row-major, 16-byte aligned, caller-owned
 * device memory; send/receive buffers are caller-owned device memory,
 * 16-byte aligned, laid out as below (P ranks, H = P * Hp heads, sequence
 * shards of Ns tokens, rec = record bytes).  Inputs must be finite.  Outputs
 * must not overlap inputs.  Every call validates on the host (SOLATTN_EINVAL,
 * text in solattn_last_error(), nothing enqueued), enqueues one kernel on
 * `stream` (hipStream_t, NULL = default) and returns without synchronising;
 * SOLATTN_EHIP reports a launch error.  d must be 64 or 128.
 */
#ifndef SOLATTN_TRANSPORT_H
#define SOLATTN_TRANSPORT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Record bytes for head dimension d (0 when d is not 64 or 128). */
size_t solattn_transport_record_bytes(int64_t d);

/* Sequence shard -> per-destination INT8 records.
 *   q, k, v: [B][H][Ns][d] (this rank's tokens of every head).
 *   send:    [P][B][H/P][Ns][3][rec] bytes; chunk p holds heads
 *            p*H/P .. p*H/P + H/P - 1, tensor order q, k, v.
 *   H must be a multiple of P. */
int solattn_pack_qkv_int8(const void* q, const void* k, const void* v, int64_t B, int64_t H,
                          int64_t Ns, int64_t d, int64_t P, void* send, void* stream);

/* Received INT8 records -> this rank's heads over the whole sequence.
 *   recv: [P][B][Hp][Ns][3][rec]; chunk s came from rank s (sequence shard s).
 *   q, k, v: [B][Hp][P*Ns][d]; token s*Ns + t from chunk s, row t. */
int solattn_unpack_qkv_int8(const void* recv, int64_t B, int64_t Hp, int64_t Ns, int64_t d,
                            int64_t P, void* q, void* k, void* v, void* stream);

/* The receive side fused with step 1 of Sol-Attn: the received INT8 records
 * (recv as for solattn_unpack_qkv_int8, N = P*Ns tokens per slice) are
 * dequantized in registers (bf16 of code * s, as solattn_unpack_qkv_int8
 * computes it) and pooled, so the bf16 K and V rows are never written.
 * Writes q_out [B][Hp][N][d] bf16 (the queries, as solattn_unpack_qkv_int8
 * would write q) and fills the workspace ws (ws_bytes >=
 * solattn_workspace_bytes(B, Hp, N, d, SOLATTN_BF16), 256-byte aligned) bit
 * for bit as solattn_prepare_ws(q, k, v, B, Hp, N, d, mode, SOLATTN_BF16)
 * would from the unpacked tensors.  solattn_attend_ws(q_out, NULL, NULL, ...)
 * then completes the attention (the bf16 kernel reads keys and values from
 * the workspace only).  mode: as for solattn_prepare_ws (include/solattn.h).
 * B*Hp <= 65535; recv, q_out and ws must not overlap.  Allocates nothing. */
int solattn_prepare_int8_ws(const void* recv, int64_t B, int64_t Hp, int64_t Ns, int64_t d,
                            int64_t P, int mode, void* q_out, void* ws, size_t ws_bytes,
                            void* stream);

/* Attention output of this rank's heads -> per-destination FP8 records.
 *   o:    [B][Hp][P*Ns][d].
 *   send: [P][B][Hp][Ns][rec]; chunk r holds tokens r*Ns .. r*Ns + Ns - 1. */
int solattn_pack_out_fp8(const void* o, int64_t B, int64_t Hp, int64_t Ns, int64_t d, int64_t P,
                         void* send, void* stream);

/* Received FP8 records -> the output of this rank's sequence shard.
 *   recv: [P][B][Hp][Ns][rec]; chunk s came from rank s (heads s*Hp ..).
 *   o:    [B][P*Hp][Ns][d]. */
int solattn_unpack_out_fp8(const void* recv, int64_t B, int64_t Hp, int64_t Ns, int64_t d,
                           int64_t P, void* o, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SOLATTN_TRANSPORT_H */
