// Steps 2-5 of Sol-Attn for bf16 inputs: routing, exact attention on kept
// 64x64 tiles, one pooled term per skipped block, all inside one online
// softmax (page "NVIDIA 团队开源 Sol-H3 的 DGX Spark 版本", section "119.68 GiB
// 的内存池", Sol-Attn item; page "MiniMax 官宣 NVIDIA Sol 团队 H3 加速",
// section "提速来自流水线每一段的叠加").
//
// Work decomposition (gfx950, wave64):
//   * one workgroup = one wavefront = one (head slice, 64-row query block);
//     the routing granularity fixes the query tile at 64 rows, and holding
//     all 64 rows in one wave gives every K/V element loaded into registers
//     64 rows of reuse;
//   * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16 with
//     fp32 accumulation.  Q^T stays in registers.  Key and
//     value tiles come pre-arranged in A-operand order from the pooling pass,
//     so every operand load reads a contiguous 1 KiB run, and P^T is the S^T
//     accumulator converted to bf16 with no lane shuffles;
//   * each 64-key tile is consumed as two 32-key halves in a software
//     pipeline whose phases pair matrix-core and vector work: the S^T
//     products of half h+1 run beside the exp2 work of half h, and the PV
//     products of half h beside the logits of half h+1, with the MFMAs and
//     vector instructions interleaved one by one.  Each key or value
//     register buffer is refilled as soon as the product that reads it has
//     issued (keys about two halves ahead of use, values about one and a
//     half);
//   * one wave per SIMD: the 64 x d fp32 output accumulator and the value
//     buffers live in the accumulation VGPRs (the PV MFMAs are inline asm),
//     the arch VGPRs hold Q^T, S^T, P and the key buffers;
//   * skipped blocks enter as "pooled tiles": 64 pooled keys kbar_j (bf16)
//     with logit bias log2(n_j), or -inf where block j is kept or padding.
//     The pooled term n_j exp(c q.kbar_j) vbar_j is exactly a softmax column
//     with logit c q.kbar_j + ln n_j, so it shares the MFMA body and the
//     online-softmax state with the exact tiles;
//   * the online softmax runs in log2 units (exp2).  The fast path fixes
//     each row's reference mref at the maximum of the first half and never
//     rescales: weights up to 2^64 above it stay far from the fp32/bf16
//     range limit.  Every later S^T accumulation starts from -mref/scale2
//     instead of zero, so its logits come out relative to the reference and
//     the exp2 needs no subtraction.  No row maximum is tracked after the
//     first half: a row whose logits later rose more than 64 above the
//     reference has a weight, and so a denominator, above 2^64, and that
//     is checked once at the end.  If some row's first half has no finite
//     logit, or some denominator ends above 2^64 (or inf / NaN), the fast
//     path's result is discarded and the query block is recomputed from
//     the start by the rescaling path (VGPR accumulators, lazy rescale when
//     the maximum grows by more than 2^8).  The denominator adds the
//     bf16-rounded weights the MFMA consumes (v_dot2 against (1, 1)), so
//     numerator and denominator agree;
//   * the routing prologue issues the query block's Q loads between its
//     score pass and its keep-mask pass, so they arrive under the latter;
//     in a planned launch (large launches: the routing kernel and the order
//     kernel ran first) the wave instead takes its query block from the
//     longest-first dispatch order and rebuilds the same lists from the
//     block's keep bits, requested ahead of the Q loads;
//     the epilogue writes each output row with 16-byte stores after a
//     v_permlane32_swap between the lane halves;
//   * workgroups are remapped so that the query blocks of one head run on
//     one XCD and share its L2 for the K/V tiles they keep (in a planned
//     launch, within that XCD's range, longest first).
// The file also holds attn_bf16_taylor_kernel, the first-order (Taylor)
// accuracy mode: the same routing, the rescaling path over the exact and
// pooled tiles, then a pass over every skipped block (see
// taylor_first_order).
#include "common.h"
#include "launch.h"
#include "taylor.h"
#include "route.h"

namespace solattn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;   // rescaling path: lazy-rescale margin (log2)
// Fast path: largest denominator share a lane may end with (2^64).  Every
// weight is at most its row's denominator, so a row whose logits rose more
// than 64 (log2 units) above the fixed reference ends above it.
constexpr float kFixedSumMax = 18446744073709551616.0f;

// One 64-key tile of the sequence: an exact key block or a pooled tile.
struct TileRef {
    const bf16* ktile;  // operand-ordered key tile
    const bf16* vtile;  // operand-ordered value tile
    int nvalid;         // keys in the block (64, or 1..63 for an exact tail block)
    int bias_off;       // LDS index (bias array) of key 0 of the tile
};

template <int D>
__device__ inline void load_k(const TileRef& t, int u, int lane, bf16x8 (&kA)[D / 16]) {
    constexpr int KS = D / 16;
#pragma unroll
    for (int s = 0; s < KS; ++s)
        kA[s] = *reinterpret_cast<const bf16x8*>(t.ktile + ktile_offset(KS, u, s, lane, 0));
}

template <int D>
__device__ inline void load_v(const TileRef& t, int u, int lane, bf16x8 (&vA)[D / 32][2]) {
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int s = 0; s < 2; ++s)
            vA[mt][s] = *reinterpret_cast<const bf16x8*>(t.vtile + vtile_offset(mt, 2 * u + s, lane, 0));
}

// Scheduling pattern for one phase: N groups of one MFMA followed by up to
// V vector-ALU instructions, so the wave issues softmax work while the
// matrix core runs.
template <int N, int V>
__device__ __forceinline__ void interleave() {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    }
}

// Wait states after the inline-asm PV MFMAs before any other instruction
// touches their accumulation registers (or the registers are reused):
// 8 x 16 wait states, several times the latency of a 16-pass MFMA.
__device__ __forceinline__ void acc_fence() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile(
        "s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15\n\t"
        "s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15");
    __builtin_amdgcn_sched_barrier(0);
}

// The fast path's accumulators copied out of the accumulation registers
// by asm of its own, after acc_fence (volatile asm keeps its order): with
// every later use an asm operand in accumulation registers, the compiler
// has no reason to place copies of its own -- which could land between the
// last MFMA and the fence -- on the way out of the loop.
template <int D>
__device__ __forceinline__ void acc_read(const f32x16 (&acc)[D / 32][2], f32x16 (&out)[D / 32][2]) {
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(out[mt][nt][v]) : "a"(acc[mt][nt][v]));
}

// max(x, x of lane ^ 32) without an LDS round trip: v_permlane32_swap
// exchanges the upper 32 lanes of one copy with the lower 32 lanes of the
// other, so each lane ends up holding both values.
__device__ __forceinline__ float max_across_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Shared state of one wave's 64 query rows.
template <int D>
struct RowState {
    f32x16 oacc[D / 32][2];  // O^T accumulators: d = 32*mt + ..., queries 32*nt + l32
    float mref[2];           // reference maximum (log2 units) per query half
    float lsum[2];           // this lane's share of the denominator per query half
};

// State of the fast path: the output accumulators are bound to
// accumulation VGPRs by the inline-asm PV MFMAs; the reference maximum is
// fixed once per row.
template <int D>
struct FixedState {
    f32x16 oacc[D / 32][2];
    float mref[2];
    float lsum[2];
};

// S^T = K Q^T for one 32-key half: 32 keys x 64 queries, two 32x32
// accumulators (queries 0..31 and 32..63); Q^T held in registers.
template <int D>
__device__ __forceinline__ void s_product(const bf16x8 (&kA)[D / 16],
                                          const bf16x8 (&qB)[2][D / 16], f32x16 (&st)[2]) {
    constexpr int KS = D / 16;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int v = 0; v < 16; ++v) st[nt][v] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        st[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kA[s], qB[0][s], st[0], 0, 0, 0);
        st[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kA[s], qB[1][s], st[1], 0, 0, 0);
    }
}

// S^T for one half with the accumulation started from `c` instead of zero:
// the fast path starts from -mref / scale2 per query column, so that the
// logits come out relative to the row's fixed reference.
template <int D>
__device__ __forceinline__ void s_product_from(const bf16x8 (&kA)[D / 16],
                                               const bf16x8 (&qB)[2][D / 16],
                                               const f32x16 (&c)[2], f32x16 (&st)[2]) {
    constexpr int KS = D / 16;
    st[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kA[0], qB[0][0], c[0], 0, 0, 0);
    st[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kA[0], qB[1][0], c[1], 0, 0, 0);
#pragma unroll
    for (int s = 1; s < KS; ++s) {
        st[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kA[s], qB[0][s], st[0], 0, 0, 0);
        st[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kA[s], qB[1][s], st[1], 0, 0, 0);
    }
}

// Softmax, first part, for half u of tile `cur`: logits in log2 units with
// the per-key bias, row maxima, and the (rare) rescale of the accumulators.
// Returns in msub the reference each query half subtracts before exp2.
template <int D>
__device__ __forceinline__ void softmax_head(f32x16 (&st)[2], const TileRef& cur, int u,
                                             const float* srow, int half, float scale2,
                                             RowState<D>& rs, float (&msub)[2]) {
    constexpr int MT = D / 32;
    // Logits in log2 units: st * scale2 + bias, with the per-key bias read
    // from LDS for every tile: 0 for exact keys, -inf for the zero-padded
    // keys past an exact tail block, log2(n_j) / -inf for pooled keys (kept
    // blocks and padding masked).  Register v of an accumulator holds key
    // 32*u + 8*(v/4) + 4*half + v%4 of the tile.
    const float* b = srow + cur.bias_off + 32 * u + 4 * half;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const f32x4 bb = *reinterpret_cast<const f32x4*>(b + 8 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                st[nt][4 * g + r] = st[nt][4 * g + r] * scale2 + bb[r];
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        float mx = fmaxf(st[nt][0], st[nt][1]);
#pragma unroll
        for (int v = 2; v < 16; v += 2) mx = fmaxf(mx, fmaxf(st[nt][v], st[nt][v + 1]));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mcand = fmaxf(rs.mref[nt], mx);
        const bool grow = mcand > rs.mref[nt] + kRescaleSlack;
        if (__ballot(grow)) {
            const float mnew = grow ? mcand : rs.mref[nt];
            const float alpha = __builtin_amdgcn_exp2f(rs.mref[nt] - mnew);
            rs.lsum[nt] *= alpha;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 16; ++v) rs.oacc[mt][nt][v] *= alpha;
            rs.mref[nt] = mnew;
        }
        // (while no finite logit has been seen -- a pooled or tail half whose
        // keys are all masked -- subtract 0 so the half yields p = 0 rather
        // than exp2(-inf + inf))
        msub[nt] = rs.mref[nt] == -__builtin_inff() ? 0.f : rs.mref[nt];
    }
}

// Fast path, first half of a query block: logits in log2 units with the
// per-key bias (as in softmax_head) and each row's maximum, which becomes
// the row's fixed reference (-inf when the half has no finite logit for that
// row; the caller then takes the rescaling path).
template <int D>
__device__ __forceinline__ void first_half_reference(f32x16 (&st)[2], const TileRef& cur,
                                                     const float* srow, int half, float scale2,
                                                     FixedState<D>& fs) {
    const float* b = srow + cur.bias_off + 4 * half;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const f32x4 bb = *reinterpret_cast<const f32x4*>(b + 8 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                st[nt][4 * g + r] = st[nt][4 * g + r] * scale2 + bb[r];
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        float mx = fmaxf(st[nt][0], st[nt][1]);
#pragma unroll
        for (int v = 2; v < 16; v += 2) mx = fmaxf(mx, fmaxf(st[nt][v], st[nt][v + 1]));
        fs.mref[nt] = max_across_halves(mx);
    }
}

// Softmax, second part: P^T in bf16 (the B operand of the PV product: k-step
// s holds keys 16*s + 4*half + {0..3, 8..11} of the half = accumulator
// registers 8*s .. 8*s+7) and the denominators, which add the bf16-rounded
// weights the MFMA consumes (v_dot2 against (1, 1)).
template <typename State>
__device__ __forceinline__ void softmax_tail(const f32x16 (&st)[2], const float (&msub)[2],
                                             State& rs, bf16x8 (&pB)[2][2]) {
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        float ps = rs.lsum[nt];
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
            f32x2 pp;
            pp[0] = __builtin_amdgcn_exp2f(st[nt][v] - msub[nt]);
            pp[1] = __builtin_amdgcn_exp2f(st[nt][v + 1] - msub[nt]);
            const bf16x2 pr = __builtin_convertvector(pp, bf16x2);
            ps = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps, false);
            pB[nt][v >> 3][v & 7] = pr[0];
            pB[nt][v >> 3][(v & 7) + 1] = pr[1];
        }
        rs.lsum[nt] = ps;
    }
}

// Fast-path softmax tail: the logits are already relative to the fixed
// reference, so P = exp2(logit) directly.
template <typename State>
__device__ __forceinline__ void softmax_tail_rel(const f32x16 (&st)[2], State& rs,
                                                 bf16x8 (&pB)[2][2]) {
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        float ps = rs.lsum[nt];
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
            f32x2 pp;
            pp[0] = __builtin_amdgcn_exp2f(st[nt][v]);
            pp[1] = __builtin_amdgcn_exp2f(st[nt][v + 1]);
            const bf16x2 pr = __builtin_convertvector(pp, bf16x2);
            ps = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps, false);
            pB[nt][v >> 3][v & 7] = pr[0];
            pB[nt][v >> 3][(v & 7) + 1] = pr[1];
        }
        rs.lsum[nt] = ps;
    }
}

// O^T += V^T P^T for one half.
template <int D>
__device__ __forceinline__ void pv_product(const bf16x8 (&vA)[D / 32][2], const bf16x8 (&pB)[2][2],
                                           RowState<D>& rs) {
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                rs.oacc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vA[mt][s], pB[nt][s],
                                                                          rs.oacc[mt][nt], 0, 0, 0);
}

// O^T += V^T P^T for one half on the fast path, with the output
// accumulators in accumulation VGPRs: written as inline assembly so the
// compiler keeps the 128 accumulator registers out of the arch VGPRs.  The
// hazards the compiler would otherwise cover are handled here: the leading
// s_nop gives the wait states a VALU write of P (the bf16 conversion)
// needs before an MFMA reads it, and the k-step-major order puts 2*MT - 1
// other MFMAs between two MFMAs that accumulate into the same registers.
__device__ __forceinline__ void mfma_pv_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "a"(a), "v"(b));
}

// PV of one half on the fast path with the logits of the next half (log2
// units plus the per-key bias) spread between its MFMAs by hand: the asm
// MFMAs are invisible to the scheduler's grouping, so the order is written
// out and pinned with scheduling barriers.  Slice m of 16 handles two of
// the 32 values a lane holds.  The logits are already relative to the
// reference (the S^T accumulation started from -mref / scale2).
__device__ __forceinline__ void head_slice(int m, f32x16 (&st)[2], const f32x4 (&bb)[4],
                                           float scale2) {
    const int g = m >> 2, nt = (m >> 1) & 1, r0 = (m & 1) * 2;
#pragma unroll
    for (int r = r0; r < r0 + 2; ++r) st[nt][4 * g + r] = st[nt][4 * g + r] * scale2 + bb[g][r];
}

template <int D>
__device__ __forceinline__ void pv_then_head(const bf16x8 (&vA)[D / 32][2], const bf16x8 (&pB)[2][2],
                                             FixedState<D>& fs, f32x16 (&st)[2], const TileRef& cur,
                                             int u, const float* srow, int half, float scale2) {
    constexpr int NM = 4 * (D / 32);  // PV MFMAs of a half
    const float* b = srow + cur.bias_off + 32 * u + 4 * half;
    f32x4 bb[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) bb[g] = *reinterpret_cast<const f32x4*>(b + 8 * g);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int k = (s * (D / 32) + mt) * 2 + nt;
                mfma_pv_acc(fs.oacc[mt][nt], vA[mt][s], pB[nt][s]);
#pragma unroll
                for (int m = k * 16 / NM; m < (k + 1) * 16 / NM; ++m)
                    head_slice(m, st, bb, scale2);
                __builtin_amdgcn_sched_barrier(0);
            }
}

// x + (x of lane ^ 32), the same bits in both lanes (v_permlane32_swap, no LDS)
__device__ __forceinline__ float sum_across_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// O = acc / l rounded to bf16.  Lane holds query 32*nt + l32 and, for each
// 8-column group g of a 32-column tile mt, columns 8g + 4*half .. +3.  One
// v_permlane32_swap per dword trades half of each pair of groups between
// the lane halves, so that a lane holds 8 whole columns of one group (half
// 0: odd groups, half 1: even groups) and writes them with one 16-byte store.
template <int D>
__device__ __forceinline__ void store_rows(const f32x16 (&oacc)[D / 32][2], const float (&lsum)[2],
                                           bf16* op, int64_t i, int64_t N, int half, int l32) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const float inv = 1.0f / sum_across_halves(lsum[nt]);
        const int64_t row = i * 64 + 32 * nt + l32;
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                uint32_t w[2][2];  // [group 2pr, 2pr+1][dword]: 4 bf16 of this lane's half
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int v = 4 * (2 * pr + q) + 2 * j;
                        bf16x2 b;
                        b[0] = to_bf16(oacc[mt][nt][v] * inv);
                        b[1] = to_bf16(oacc[mt][nt][v + 1] * inv);
                        w[q][j] = __builtin_bit_cast(uint32_t, b);
                    }
                uint4 out;
                const auto s0 = __builtin_amdgcn_permlane32_swap(w[1][0], w[0][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(w[1][1], w[0][1], false, false);
                out.x = s0[0];
                out.y = s1[0];
                out.z = s0[1];
                out.w = s1[1];
                if (row < N)
                    *reinterpret_cast<uint4*>(op + row * D + 32 * mt + 16 * pr + 8 * (1 - half)) = out;
            }
    }
}

// First-order (Taylor) term of the skipped blocks of one query block, added
// after its exact and pooled tiles, so that the running reference already
// covers every pooled logit (up to the lazy-rescale slack).  Expanding block
// j's exact sum around its pooled key to first order adds w_rj c C_j^T q_r to
// the numerator, w_rj = n_j exp(c q_r.kbar_j) the pooled term's weight and
// C_j the block's key/value cross-covariance; the denominator's first-order
// term is zero.  Since the centred keys sum to zero, w_rj c C_j^T q_r =
// sum_t (w_rj / n_j) c (q_r.k_t - q_r.kbar_j) v_t: a pass over the block's
// raw key and value tiles with linear weights, no d x d matrix.  Here
// q_r.kbar_j is the mean over the tile's keys of the S^T products themselves
// (zero-padded keys past a tail block add zero to the sum; their value rows
// are zero), and (w_rj / n_j) relative to the row reference is
// exp2(scale2 * that mean - mref).
template <int D>
__device__ __forceinline__ void taylor_first_order(const bf16x8 (&qB)[2][D / 16], const bf16* kp,
                                                   const bf16* vp, int64_t Nb, int tail,
                                                   const uint16_t* slist, int n_skip,
                                                   float scale2, int lane, RowState<D>& rs) {
    constexpr int KS = D / 16;
    constexpr int MT = D / 32;
    const float c = 1.0f / sqrtf((float)D);
    if (n_skip == 0) return;
    auto tile = [&](int x) -> TileRef {
        const int64_t j = __builtin_amdgcn_readfirstlane((int)slist[x]);
        TileRef t;
        t.ktile = kp + j * (int64_t)D * 64;
        t.vtile = vp + j * (int64_t)D * 64;
        t.nvalid = (j == Nb - 1) ? tail : 64;
        t.bias_off = 0;
        return t;
    };
    // software pipeline in the operand registers themselves: the keys of
    // block x+1 are requested once the S^T products of block x have read
    // theirs, the values of block x+1 once its PV products have
    bf16x8 kA0[KS], kA1[KS];
    bf16x8 vA0[MT][2], vA1[MT][2];
    TileRef t = tile(0);
    load_k<D>(t, 0, lane, kA0);
    load_k<D>(t, 1, lane, kA1);
    load_v<D>(t, 0, lane, vA0);
    load_v<D>(t, 1, lane, vA1);
    for (int x = 0; x < n_skip; ++x) {
        const TileRef tn = x + 1 < n_skip ? tile(x + 1) : t;
        f32x16 s0[2], s1[2];
        s_product<D>(kA0, qB, s0);
        s_product<D>(kA1, qB, s1);
        if (x + 1 < n_skip) {
            load_k<D>(tn, 0, lane, kA0);
            load_k<D>(tn, 1, lane, kA1);
        }
        float sbar[2], coef[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            float part = 0.f;
#pragma unroll
            for (int v = 0; v < 16; ++v) part += s0[nt][v] + s1[nt][v];
            sbar[nt] = sum_across_halves(part) / (float)t.nvalid;
            coef[nt] = c * __builtin_amdgcn_exp2f(sbar[nt] * scale2 - rs.mref[nt]);
        }
        bf16x8 pB[2][2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int v = 0; v < 16; ++v) pB[nt][v >> 3][v & 7] = to_bf16(coef[nt] * (s0[nt][v] - sbar[nt]));
        pv_product<D>(vA0, pB, rs);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int v = 0; v < 16; ++v) pB[nt][v >> 3][v & 7] = to_bf16(coef[nt] * (s1[nt][v] - sbar[nt]));
        pv_product<D>(vA1, pB, rs);
        if (x + 1 < n_skip) {
            load_v<D>(tn, 0, lane, vA0);
            load_v<D>(tn, 1, lane, vA1);
        }
        t = tn;
    }
}

}  // namespace

// Rescaling path, for query blocks whose logits grow too far past the
// first half's maximum: the block is recomputed from the start with a
// moving reference (lazy rescale).  A separate, never-inlined function, so
// that its register needs stay out of the fast path's allocation.  The S^T
// products of half h+1 are issued before the exp2 work of half h; keys are
// fetched two halves ahead and values one half ahead, into two register
// buffers each (buffer = u).
template <int D, bool TAYLOR>
__device__ __forceinline__ void rescaling_path(
    const bf16* qp, const bf16* kp, const bf16* vp, const bf16* kbp, const bf16* vbp, bf16* op,
    int64_t N, int64_t Nb, int64_t Nbp, int sparse, int64_t i, int n_kept, uint64_t tile_mask,
    const float* srow, const uint16_t* klist, const uint16_t* plist, const uint16_t* slist,
    int n_skip) {
    constexpr int KS = D / 16;
    constexpr int MT = D / 32;
    const int lane = threadIdx.x, half = lane >> 5, l32 = lane & 31;
    const int zero_bias = (int)Nbp, tail_bias = (int)Nbp + 64;
    const int tail = (int)(N - (Nb - 1) * 64);
    bf16x8 qB[2][KS];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        int64_t row = i * 64 + 32 * nt + l32;
        if (row > N - 1) row = N - 1;
        const bf16* qrow = qp + row * D + 8 * half;
#pragma unroll
        for (int s = 0; s < KS; ++s) qB[nt][s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
    }
    const int n_tiles = n_kept + __popcll(tile_mask);
    auto tile_at = [&](int t) -> TileRef {
        TileRef r;
        if (t < n_kept) {
            const int64_t j = sparse ? (int64_t)__builtin_amdgcn_readfirstlane((int)klist[t])
                                     : (int64_t)t;
            r.ktile = kp + j * (int64_t)D * 64;
            r.vtile = vp + j * (int64_t)D * 64;
            r.nvalid = (j == Nb - 1) ? tail : 64;
            r.bias_off = r.nvalid < 64 ? tail_bias : zero_bias;
        } else {
            const int T = __builtin_amdgcn_readfirstlane((int)plist[t - n_kept]);
            r.ktile = kbp + (int64_t)T * D * 64;
            r.vtile = vbp + (int64_t)T * D * 64;
            r.nvalid = 64;
            r.bias_off = 64 * T;
        }
        return r;
    };
    const float scale2 = kLog2e / sqrtf((float)D);
    RowState<D> rs;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int v = 0; v < 16; ++v) rs.oacc[mt][nt][v] = 0.f;
    rs.mref[0] = rs.mref[1] = -__builtin_inff();
    rs.lsum[0] = rs.lsum[1] = 0.f;
    bf16x8 kB0[KS], kB1[KS];
    bf16x8 vB0[MT][2], vB1[MT][2];
    f32x16 st0[2], st1[2];
    bf16x8 pB[2][2];
    float msub[2];
    TileRef t0 = tile_at(0);
    TileRef t1 = n_tiles > 1 ? tile_at(1) : t0;
    load_k<D>(t0, 0, lane, kB0);
    load_k<D>(t0, 1, lane, kB1);
    load_v<D>(t0, 0, lane, vB0);
    s_product<D>(kB0, qB, st0);
    load_k<D>(t1, 0, lane, kB0);

    for (int t = 0; t < n_tiles; ++t) {
        const TileRef t2 = t + 2 < n_tiles ? tile_at(t + 2) : t1;
        softmax_head<D>(st0, t0, 0, srow, half, scale2, rs, msub);
        s_product<D>(kB1, qB, st1);
        load_k<D>(t1, 1, lane, kB1);
        load_v<D>(t0, 1, lane, vB1);
        softmax_tail(st0, msub, rs, pB);
        pv_product<D>(vB0, pB, rs);
        softmax_head<D>(st1, t0, 1, srow, half, scale2, rs, msub);
        s_product<D>(kB0, qB, st0);
        load_k<D>(t2, 0, lane, kB0);
        load_v<D>(t1, 0, lane, vB0);
        softmax_tail(st1, msub, rs, pB);
        pv_product<D>(vB1, pB, rs);
        t0 = t1;
        t1 = t2;
    }
    if constexpr (TAYLOR) taylor_first_order<D>(qB, kp, vp, Nb, tail, slist, n_skip, scale2, lane, rs);
    store_rows<D>(rs.oacc, rs.lsum, op, i, N, half, l32);
}

template <int D>
__device__ __attribute__((noinline)) void attend_rescaling(
    const bf16* qp, const bf16* kp, const bf16* vp, const bf16* kbp, const bf16* vbp, bf16* op,
    int64_t N, int64_t Nb, int64_t Nbp, int sparse, int64_t i, int n_kept, uint64_t tile_mask,
    const float* srow, const uint16_t* klist, const uint16_t* plist) {
    rescaling_path<D, false>(qp, kp, vp, kbp, vbp, op, N, Nb, Nbp, sparse, i, n_kept, tile_mask,
                             srow, klist, plist, nullptr, 0);
}

// Sol-Attn with the first-order (Taylor) term of the skipped blocks: the
// rescaling path over the exact and pooled tiles, then taylor_first_order.
template <int D>
__device__ __attribute__((noinline)) void attend_taylor(
    const bf16* qp, const bf16* kp, const bf16* vp, const bf16* kbp, const bf16* vbp, bf16* op,
    int64_t N, int64_t Nb, int64_t Nbp, int64_t i, int n_kept, uint64_t tile_mask,
    const float* srow, const uint16_t* klist, const uint16_t* plist, const uint16_t* slist,
    int n_skip) {
    rescaling_path<D, true>(qp, kp, vp, kbp, vbp, op, N, Nb, Nbp, 1, i, n_kept, tile_mask, srow,
                            klist, plist, slist, n_skip);
}

// Work item of workgroup g: xcd_remap's contiguous (head, query block) range
// per XCD, in order -- except that with dense prefix rows the prefix query
// blocks of the range (i < Pb: every key block exact, ~7x a routed block's
// work at the refine shape) come first, so that the dispatch does not end
// on them.
__device__ inline int64_t work_order(int64_t g, int64_t T, int64_t Nb, int64_t Pb,
                                     bool heavy_first) {
    const int64_t x = g % 8, r = g / 8, q = T / 8, m = T % 8;
    const int64_t start = x * q + (x < m ? x : m);
    if (!heavy_first || Pb < 1 || Pb >= Nb) return start + r;   // = xcd_remap(g, T)
    const int64_t nbx = q + (x < m ? 1 : 0);
    // prefix items (block index < Pb) among the first n items, head-major
    auto P = [&](int64_t n) { return n / Nb * Pb + (n % Nb < Pb ? n % Nb : Pb); };
    const int64_t p0 = P(start), npx = P(start + nbx) - p0;
    if (r < npx) {
        const int64_t k = p0 + r;                 // the k-th prefix item
        return k / Pb * Nb + k % Pb;
    }
    const int64_t k = (start - p0) + (r - npx);   // the k-th other item
    return k / (Nb - Pb) * Nb + Pb + k % (Nb - Pb);
}

template <int D>
__global__ __launch_bounds__(64, 1) void attn_bf16_kernel(AttnArgs a) {
    constexpr int KS = D / 16;  // k-steps of S^T = K Q^T
    constexpr int MT = D / 32;  // 32-row d tiles of O^T
    extern __shared__ float smem[];

    const int lane = threadIdx.x, half = lane >> 5, l32 = lane & 31;
    const int64_t N = a.N, Nb = a.Nb, Nbp = a.Nbp;
    // A planned launch (the routing kernel and the order kernel ran first)
    // takes its work item from the dispatch order and its routing from the
    // keep bits; otherwise the work item follows work_order and the wave
    // routes its query block itself.
    const bool planned = a.plan_perm != nullptr;
    const int64_t w = planned ? (int64_t)__builtin_amdgcn_readfirstlane(
                                    a.plan_perm[xcd_remap(blockIdx.x, a.BH * Nb)])
                              : work_order(blockIdx.x, a.BH * Nb, Nb, a.Pb,
                                           a.mode != kDense && a.prefix_rows);
    const int64_t bh = w / Nb, i = w % Nb;
    // LDS: srow[Nbp] routing scores, then pooled-key biases; two 64-entry
    // bias rows for exact tiles (all zero; zero then -inf past the tail
    // block's last key; before that, the block's query mean while the
    // scores are formed); the kept list; the pooled-tile list; a planned
    // launch's keep bits (Nbp / 32 words)
    float* srow = smem;
    const int zero_bias = (int)Nbp, tail_bias = (int)Nbp + 64;
    uint16_t* klist = reinterpret_cast<uint16_t*>(smem + Nbp + 128);
    uint16_t* plist = reinterpret_cast<uint16_t*>(smem + Nbp + 128 + (Nb + 15) / 16 * 8);
    uint32_t* kbits = reinterpret_cast<uint32_t*>(smem + Nbp + 128 + (Nb + 15) / 16 * 8 + 32);

    const bf16* qp = reinterpret_cast<const bf16*>(a.q) + bh * N * D;
    const bf16* kp = reinterpret_cast<const bf16*>(a.kP) + bh * Nb * D * 64;
    const bf16* vp = reinterpret_cast<const bf16*>(a.vP) + bh * Nb * D * 64;
    const bf16* kbp = reinterpret_cast<const bf16*>(a.kbarP) + bh * Nbp * D;
    const bf16* vbp = reinterpret_cast<const bf16*>(a.vbarP) + bh * Nbp * D;
    const int tail = (int)(N - (Nb - 1) * 64);  // keys in the last block (1..64)

    // Q^T as the B operand of S^T = K Q^T, held in registers for the whole
    // query block: lane holds query 32*nt + l32, d = 16*s + 8*half .. +7.
    // Loaded between the two parts of the routing, so that the block's trip
    // from HBM overlaps the threshold and keep-mask work.
    // (planned: the row's keep bits are requested ahead of the Q loads, lane
    // l taking word l; rows of more than 64 words take the rest after them)
    const int64_t W = (Nb + 31) / 32;
    const uint32_t* brow = planned ? a.plan_mask + (bh * Nb + i) * W : nullptr;
    uint32_t bits0 = 0;
    if (planned) {
        if (lane < W) bits0 = brow[lane];
    } else if (a.mode != kDense) {
        route_scores<D, true>(a, bh, i, srow, srow + Nbp);
    }
    bf16x8 qB[2][KS];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        int64_t row = i * 64 + 32 * nt + l32;
        if (row > N - 1) row = N - 1;
        const bf16* qrow = qp + row * D + 8 * half;
#pragma unroll
        for (int s = 0; s < KS; ++s) qB[nt][s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
    }
    int n_kept;
    uint64_t tile_mask;
    if (planned) {
        if (lane < W) kbits[lane] = bits0;
        for (int64_t k = 64 + lane; k < W; k += 64) kbits[k] = brow[k];
        __syncthreads();
        const RouteResult r = route_from_bits(a, bh, i, kbits, srow, klist);
        n_kept = r.n_kept;
        tile_mask = r.tile_mask;
    } else if (a.mode != kDense) {
        const RouteResult r = route_select(a, bh, i, srow, klist);
        n_kept = r.n_kept;
        tile_mask = r.tile_mask;
    } else {
        export_dense_route(a, bh, i);
        n_kept = (int)Nb;
        tile_mask = 0;
    }
    srow[zero_bias + lane] = 0.f;
    srow[tail_bias + lane] = lane < tail ? 0.f : -__builtin_inff();
    __syncthreads();

    const float scale2 = kLog2e / sqrtf((float)D);

    // Tile sequence: exact blocks in kept-list order, then the pooled tiles
    // holding a skipped block in ascending order (plist).  Each tile is two
    // 32-key halves (an exact tail block keeps its zero-padded keys masked).
    const int n_tiles = n_kept + __popcll(tile_mask);
    if (tile_mask >> lane & 1) plist[__popcll(tile_mask & ((1ull << lane) - 1))] = (uint16_t)lane;
    __syncthreads();
    // (list entries are wave-uniform: readfirstlane keeps the tile pointers in
    // scalar registers)
    auto tile_at = [&](int t) -> TileRef {
        TileRef r;
        if (t < n_kept) {
            const int64_t j = (a.mode != kDense)
                                  ? (int64_t)__builtin_amdgcn_readfirstlane((int)klist[t])
                                  : (int64_t)t;
            r.ktile = kp + j * (int64_t)D * 64;
            r.vtile = vp + j * (int64_t)D * 64;
            r.nvalid = (j == Nb - 1) ? tail : 64;
            r.bias_off = r.nvalid < 64 ? tail_bias : zero_bias;
        } else {
            const int T = __builtin_amdgcn_readfirstlane((int)plist[t - n_kept]);
            r.ktile = kbp + (int64_t)T * D * 64;
            r.vtile = vbp + (int64_t)T * D * 64;
            r.nvalid = 64;
            r.bias_off = 64 * T;
        }
        return r;
    };
    bf16* op = reinterpret_cast<bf16*>(a.out) + bh * N * D;

    // Fast path.  Phases (sched barriers keep them, and so the order of the
    // loads that the in-order vmcnt waits rely on, in place):
    //   loads of the values of half h+1 (into the buffer that the PV
    //   product of half h-1 has just read);
    //   S^T of half h+1 beside the exp2 work of half h;
    //   loads of the keys of half h+3 (into the buffer S^T has just read);
    //   PV of half h with the logits (scale and bias) of half h+1 placed
    //   between its MFMAs by hand (pv_then_head).
    // Past the end the prefetches and the S^T products re-read the last tile
    // (their results are never used), so every iteration runs the same
    // straight-line code.
    bool abandoned = false;
    {
        FixedState<D> fs;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int v = 0; v < 16; ++v) fs.oacc[mt][nt][v] = 0.f;
        fs.mref[0] = fs.mref[1] = -__builtin_inff();
        fs.lsum[0] = fs.lsum[1] = 0.f;
        bf16x8 kB0[KS], kB1[KS];            // keys of even / odd halves
        bf16x8 vB0[MT][2], vB1[MT][2];      // values (accumulation VGPRs)
        f32x16 st0[2], st1[2];
        bf16x8 pB[2][2];
        TileRef t0 = tile_at(0);
        TileRef t1 = n_tiles > 1 ? tile_at(1) : t0;
        // First half: its row maxima fix the reference (a row whose first
        // half has no finite logit -- only possible when the first tile is a
        // pooled tile -- sends the block to the rescaling path).  Later S^T
        // products start from -mref / scale2 so their logits come out
        // relative to it.  (The loads outstanding when the loop is entered
        // are issued in the order of the loop's own, so the wait counts at
        // the loop head hold on both paths.)
        load_k<D>(t0, 0, lane, kB0);
        __builtin_amdgcn_sched_barrier(0);
        load_k<D>(t0, 1, lane, kB1);
        __builtin_amdgcn_sched_barrier(0);
        load_v<D>(t0, 0, lane, vB0);
        __builtin_amdgcn_sched_barrier(0);
        s_product<D>(kB0, qB, st0);
        __builtin_amdgcn_sched_barrier(0);
        load_k<D>(t1, 0, lane, kB0);
        __builtin_amdgcn_sched_barrier(0);
        first_half_reference<D>(st0, t0, srow, half, scale2, fs);
        abandoned = __ballot(fs.mref[0] == -__builtin_inff() || fs.mref[1] == -__builtin_inff()) != 0;
        f32x16 cinit[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const float m = abandoned ? 0.f : fs.mref[nt];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                cinit[nt][v] = -m / scale2;
                st0[nt][v] -= m;  // the first half's logits, made relative
            }
        }
        __builtin_amdgcn_sched_barrier(0);

        // Each buffer is refilled as soon as the product that reads it has
        // issued: values two S^T phases and one PV phase ahead of their PV
        // product, keys two PV phases and one S^T phase ahead of their S^T
        // product.  The loads go out in the order of their use (V(h),
        // K(h+2), V(h+1), K(h+3), ...), so waiting for one operand never
        // waits for a later one.
        for (int t = 0; t < n_tiles && !abandoned; ++t) {
            const TileRef t2 = t + 2 < n_tiles ? tile_at(t + 2) : t1;
            load_v<D>(t0, 1, lane, vB1);
            __builtin_amdgcn_sched_barrier(0);
            s_product_from<D>(kB1, qB, cinit, st1);          // S^T (t, 1)
            softmax_tail_rel(st0, fs, pB);                   // exp2 (t, 0)
            interleave<16, 6>();
            __builtin_amdgcn_sched_barrier(0);
            load_k<D>(t1, 1, lane, kB1);
            __builtin_amdgcn_sched_barrier(0);
            pv_then_head<D>(vB0, pB, fs, st1, t0, 1, srow, half, scale2);  // PV (t, 0)
            __builtin_amdgcn_sched_barrier(0);
            load_v<D>(t1, 0, lane, vB0);
            __builtin_amdgcn_sched_barrier(0);
            s_product_from<D>(kB0, qB, cinit, st0);          // S^T (t+1, 0)
            softmax_tail_rel(st1, fs, pB);                   // exp2 (t, 1)
            interleave<16, 6>();
            __builtin_amdgcn_sched_barrier(0);
            load_k<D>(t2, 0, lane, kB0);
            __builtin_amdgcn_sched_barrier(0);
            pv_then_head<D>(vB1, pB, fs, st0, t1, 0, srow, half, scale2);  // PV (t, 1)
            __builtin_amdgcn_sched_barrier(0);
            t0 = t1;
            t1 = t2;
        }
        // (the loop runs to its end even when some row rose far past its
        // reference -- inf or NaN may then have reached the accumulators --
        // and the results are discarded here; a NaN denominator fails the
        // comparison and is discarded too)
        abandoned = abandoned ||
                    __ballot(!(fs.lsum[0] <= kFixedSumMax && fs.lsum[1] <= kFixedSumMax)) != 0;
        acc_fence();
        if (!abandoned) {
            f32x16 o[MT][2];
            acc_read<D>(fs.oacc, o);
            store_rows<D>(o, fs.lsum, op, i, N, half, l32);
        }
    }
    if (!abandoned) return;

    attend_rescaling<D>(qp, kp, vp, kbp, vbp, op, N, Nb, Nbp, a.mode != kDense, i, n_kept, tile_mask,
                        srow, klist, plist);
}

// Sol-Attn with the first-order (Taylor) correction of the skipped blocks
// (page "MiniMax 官推背书 Sol Engine：H3 的 10 秒 768p 生成从 414s 压到
// 14.93s", section "同一项目页上的另一种口径：3.95× 近无损": the skipped
// blocks' compensation as a Taylor approximation).  An accuracy mode: every
// skipped block is read and multiplied like an exact tile, so it costs about
// as much as dense attention.  The routing is the sparse kernel's; the list
// of skipped blocks comes from the pooled-key biases route_select leaves
// (finite exactly for the skipped blocks).
template <int D>
__global__ __launch_bounds__(64, 1) void attn_bf16_taylor_kernel(AttnArgs a) {
    extern __shared__ float smem[];
    const int lane = threadIdx.x;
    const int64_t N = a.N, Nb = a.Nb, Nbp = a.Nbp;
    const int64_t w = xcd_remap(blockIdx.x, a.BH * Nb);
    const int64_t bh = w / Nb, i = w % Nb;
    // LDS as in attn_bf16_kernel, then the skipped-block list
    float* srow = smem;
    const int zero_bias = (int)Nbp, tail_bias = (int)Nbp + 64;
    uint16_t* klist = reinterpret_cast<uint16_t*>(smem + Nbp + 128);
    uint16_t* plist = reinterpret_cast<uint16_t*>(smem + Nbp + 128 + (Nb + 15) / 16 * 8);
    uint16_t* slist = reinterpret_cast<uint16_t*>(smem + Nbp + 128 + (Nb + 15) / 16 * 8 + 32);
    const bf16* qp = reinterpret_cast<const bf16*>(a.q) + bh * N * D;
    const bf16* kp = reinterpret_cast<const bf16*>(a.kP) + bh * Nb * D * 64;
    const bf16* vp = reinterpret_cast<const bf16*>(a.vP) + bh * Nb * D * 64;
    const bf16* kbp = reinterpret_cast<const bf16*>(a.kbarP) + bh * Nbp * D;
    const bf16* vbp = reinterpret_cast<const bf16*>(a.vbarP) + bh * Nbp * D;
    const int tail = (int)(N - (Nb - 1) * 64);

    route_scores<D, true>(a, bh, i, srow, srow + Nbp);
    const RouteResult r = route_select(a, bh, i, srow, klist);
    srow[zero_bias + lane] = 0.f;
    srow[tail_bias + lane] = lane < tail ? 0.f : -__builtin_inff();
    int n_skip = 0;
    for (int64_t j0 = 0; j0 < Nb; j0 += 64) {
        const int64_t j = j0 + lane;
        const bool sk = j < Nb && srow[j] != -__builtin_inff();
        const uint64_t b = __ballot(sk);
        if (sk) slist[n_skip + __popcll(b & ((1ull << lane) - 1))] = (uint16_t)j;
        n_skip += __popcll(b);
    }
    if (r.tile_mask >> lane & 1)
        plist[__popcll(r.tile_mask & ((1ull << lane) - 1))] = (uint16_t)lane;
    __syncthreads();
    attend_taylor<D>(qp, kp, vp, kbp, vbp, reinterpret_cast<bf16*>(a.out) + bh * N * D, N, Nb, Nbp,
                     i, r.n_kept, r.tile_mask, srow, klist, plist, slist, n_skip);
}

hipError_t launch_attn_bf16_taylor(const AttnArgs& a, hipStream_t s) {
    const size_t lds = sizeof(float) * (a.Nbp + 128 + (a.Nb + 15) / 16 * 8 + 32) +
                       sizeof(uint16_t) * ((a.Nb + 15) / 16 * 16);
    const dim3 grid((unsigned)(a.BH * a.Nb));
    if (a.d == 128)
        hipLaunchKernelGGL((attn_bf16_taylor_kernel<128>), grid, dim3(64), lds, s, a);
    else
        hipLaunchKernelGGL((attn_bf16_taylor_kernel<64>), grid, dim3(64), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
    const size_t lds = sizeof(float) * (a.Nbp + 128 + (a.Nb + 15) / 16 * 8 + 32 + a.Nbp / 32);
    const dim3 grid((unsigned)(a.BH * a.Nb));
    if (a.d == 128)
        hipLaunchKernelGGL((attn_bf16_kernel<128>), grid, dim3(64), lds, s, a);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<64>), grid, dim3(64), lds, s, a);
    return hipGetLastError();
}

}  // namespace solattn
