// Shared device-side definitions of the Sol-Attn HIP library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace solattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Element offset of (mt, s, lane, e) inside one 64-key value tile laid out in
// the A-operand order of v_mfma_f32_32x32x16_bf16 for O^T = V^T P^T:
// 16-byte group (mt*4 + s)*64 + lane holds V[key(s, lane/32, e)][32*mt + lane%32]
// for e = 0..7.  The key order inside each 16-key step matches the row order
// of the 32x32 MFMA accumulator (rows 4h..4h+3 and 4h+8..4h+11 of each
// 16-row half belong to lane half h), so P^T needs no shuffle.
__host__ __device__ inline int vtile_offset(int mt, int s, int lane, int e) {
    return ((mt * 4 + s) * 64 + lane) * 8 + e;
}
__host__ __device__ inline int vtile_key(int s, int half, int e) {
    return 16 * s + 4 * half + (e < 4 ? e : e + 4);
}
// Inverse: (s, half, e) of key kk (0..63) inside a tile.
__host__ __device__ inline void vtile_slot(int kk, int* s, int* half, int* e) {
    int r = kk & 15;
    *s = kk >> 4;
    *half = (r >> 2) & 1;
    *e = (r & 3) + 4 * (r >> 3);
}

// Element offset of (u, s, lane, e) inside one 64-key key tile laid out in the
// A-operand order of v_mfma_f32_32x32x16_bf16 for S^T = K Q^T, consumed in
// 32-key halves u: 16-byte group (u*KS + s)*64 + lane (KS = d/16) holds
// K[32*u + lane%32][16*s + 8*(lane/32) + e], e = 0..7 -- a whole 16-byte chunk
// of one key row, so the relayout only permutes chunks.
__host__ __device__ inline int ktile_offset(int KS, int u, int s, int lane, int e) {
    return ((u * KS + s) * 64 + lane) * 8 + e;
}

// Round-to-nearest-even fp32 -> bf16 (finite inputs).
__device__ inline bf16 to_bf16(float x) { return (bf16)x; }

// Sum over the 64 lanes, the same bits in every lane, without LDS round
// trips: pairs within quads, quads within 8 lanes, 8-lane groups within
// rows of 16 (DPP quad_perm, row_half_mirror, row_mirror), then rows 0+1 /
// 2+3 and the two halves (v_permlane16_swap, v_permlane32_swap).  Every
// step adds two values that the partner lane adds in the other order, so
// all lanes hold bit-identical partial sums throughout.
template <int CTRL>
__device__ inline float dpp_add(float x) {
    const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false);
    return x + __int_as_float(y);
}

__device__ inline float wave_sum(float x) {
    x = dpp_add<0xb1>(x);   // quad_perm [1, 0, 3, 2]
    x = dpp_add<0x4e>(x);   // quad_perm [2, 3, 0, 1]
    x = dpp_add<0x141>(x);  // row_half_mirror
    x = dpp_add<0x140>(x);  // row_mirror
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                      false);
    x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                      false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Workgroup index -> work item, so that consecutive work items (query blocks
// of one head) land on the same XCD.  The dispatcher deals workgroups to the
// 8 XCDs round robin; XCD x receives ids x, x+8, ... and is given the
// contiguous range of work items starting at x*(T/8) + min(x, T%8).
__device__ inline int64_t xcd_remap(int64_t g, int64_t T) {
    int64_t x = g % 8, r = g / 8;
    int64_t q = T / 8, m = T % 8;
    return x * q + (x < m ? x : m) + r;
}

}  // namespace solattn
