/*
 * solattn_probe.h -- measurement aid shipped with the Sol-Attn library for
 * AMD Instinct MI355X (gfx950).  Not part of the attention operation.
 *
 * The roofline of the fused attention kernel is read against the bf16
 * matrix-core peak.  The published dense figure assumes the 2.4 GHz peak
 * clock; this probe measures, in the same process and on the same device,
 * what the matrix cores sustain from register operands, so a benchmark can
 * report both.
 */
#ifndef SOLATTN_PROBE_H
#define SOLATTN_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue `waves` wavefronts (one 64-thread workgroup each) that each issue
 * iters x 16 v_mfma_f32_32x32x16_bf16 in eight independent accumulation
 * chains, from register operands, with no memory traffic in the loop.
 * Work: waves * iters * 16 * 32768 FLOP.
 *   sink:   caller-owned device buffer of waves * 64 floats, 16-byte aligned;
 *           receives one checksum per lane (keeps the loop from being
 *           removed; its values carry no meaning).
 *   waves:  1 .. 2^20.  At least 4 x 256 (one per SIMD) to fill the GPU;
 *           a multiple of 1024 balances the SIMDs.
 *   iters:  1 .. 2^20.
 *   stream: hipStream_t (NULL = default); the call returns after enqueueing.
 * Returns SOLATTN_OK, SOLATTN_EINVAL (checked on the host, nothing enqueued;
 * text in solattn_last_error()) or SOLATTN_EHIP. */
int solattn_probe_mfma_bf16(float* sink, int64_t waves, int64_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SOLATTN_PROBE_H */
