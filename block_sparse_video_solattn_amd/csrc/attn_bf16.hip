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
//     pipeline: the S^T products of the next half are issued before the
//     exp2 work of the current one, keys are fetched two halves ahead and
//     values one half ahead into register double buffers.  One wave per
//     SIMD leaves the whole register file (arch + accumulation VGPRs) to
//     the 64 x d fp32 output accumulator, Q^T and these buffers;
//   * skipped blocks enter as "pooled tiles": 64 pooled keys kbar_j (bf16)
//     with logit bias log2(n_j), or -inf where block j is kept or padding.
//     The pooled term n_j exp(c q.kbar_j) vbar_j is exactly a softmax column
//     with logit c q.kbar_j + ln n_j, so it shares the MFMA body and the
//     online-softmax state with the exact tiles;
//   * the online softmax runs in log2 units (exp2) with a lazy rescale: the
//     reference maximum moves only when the row maximum grows by more than
//     2^8, which keeps P <= 256 in bf16 and skips most rescales of the
//     accumulators.  The denominator adds the bf16-rounded weights the MFMA
//     consumes (v_dot2 against (1, 1)), so numerator and denominator agree;
//   * workgroups are remapped so that the query blocks of one head run on
//     one XCD and share its L2 for the K/V tiles they keep.
#include "common.h"
#include "launch.h"
#include "route.h"

namespace solattn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;

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

// Shared state of one wave's 64 query rows.
template <int D>
struct RowState {
    f32x16 oacc[D / 32][2];  // O^T accumulators: d = 32*mt + ..., queries 32*nt + l32
    float mref[2];           // reference maximum (log2 units) per query half
    float lsum[2];           // this lane's share of the denominator per query half
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

// Softmax, second part: P^T in bf16 (the B operand of the PV product: k-step
// s holds keys 16*s + 4*half + {0..3, 8..11} of the half = accumulator
// registers 8*s .. 8*s+7) and the denominators, which add the bf16-rounded
// weights the MFMA consumes (v_dot2 against (1, 1)).
template <int D>
__device__ __forceinline__ void softmax_tail(const f32x16 (&st)[2], const float (&msub)[2],
                                             RowState<D>& rs, bf16x8 (&pB)[2][2]) {
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

}  // namespace

template <int D>
__global__ __launch_bounds__(64, 1) void attn_bf16_kernel(AttnArgs a) {
    constexpr int KS = D / 16;  // k-steps of S^T = K Q^T
    constexpr int MT = D / 32;  // 32-row d tiles of O^T
    extern __shared__ float smem[];

    const int lane = threadIdx.x, half = lane >> 5, l32 = lane & 31;
    const int64_t N = a.N, Nb = a.Nb, Nbp = a.Nbp;
    const int64_t w = xcd_remap(blockIdx.x, a.BH * Nb);
    const int64_t bh = w / Nb, i = w % Nb;
    // LDS: srow[Nbp] routing scores, then pooled-key biases; two 64-entry
    // bias rows for exact tiles (all zero; zero then -inf past the tail
    // block's last key); the kept list; the pooled-tile list
    float* srow = smem;
    const int zero_bias = (int)Nbp, tail_bias = (int)Nbp + 64;
    uint16_t* klist = reinterpret_cast<uint16_t*>(smem + Nbp + 128);
    uint16_t* plist = reinterpret_cast<uint16_t*>(smem + Nbp + 128 + (Nb + 15) / 16 * 8);

    int n_kept;
    uint64_t tile_mask;
    if (a.mode == kSparse) {
        const RouteResult r = route_query_block<D>(a, bh, i, srow, klist);
        n_kept = r.n_kept;
        tile_mask = r.tile_mask;
    } else {
        export_dense_route(a, bh, i);
        n_kept = (int)Nb;
        tile_mask = 0;
    }

    const bf16* qp = reinterpret_cast<const bf16*>(a.q) + bh * N * D;
    const bf16* kp = reinterpret_cast<const bf16*>(a.kP) + bh * Nb * D * 64;
    const bf16* vp = reinterpret_cast<const bf16*>(a.vP) + bh * Nb * D * 64;
    const bf16* kbp = reinterpret_cast<const bf16*>(a.kbarP) + bh * Nbp * D;
    const bf16* vbp = reinterpret_cast<const bf16*>(a.vbarP) + bh * Nbp * D;
    const int tail = (int)(N - (Nb - 1) * 64);  // keys in the last block (1..64)
    srow[zero_bias + lane] = 0.f;
    srow[tail_bias + lane] = lane < tail ? 0.f : -__builtin_inff();

    // Q^T as the B operand of S^T = K Q^T, held in registers for the whole
    // query block: lane holds query 32*nt + l32, d = 16*s + 8*half .. +7
    bf16x8 qB[2][KS];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        int64_t row = i * 64 + 32 * nt + l32;
        if (row > N - 1) row = N - 1;
        const bf16* qrow = qp + row * D + 8 * half;
#pragma unroll
        for (int s = 0; s < KS; ++s) qB[nt][s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
    }
    __syncthreads();

    RowState<D> rs;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int v = 0; v < 16; ++v) rs.oacc[mt][nt][v] = 0.f;
    rs.mref[0] = rs.mref[1] = -__builtin_inff();
    rs.lsum[0] = rs.lsum[1] = 0.f;
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
            const int64_t j = (a.mode == kSparse)
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

    // Software pipeline over halves h = (tile, u): the S^T products of half
    // h+1 are issued before the exp2 work of half h, so the matrix cores and
    // the vector ALU can run side by side; keys are fetched two
    // halves ahead and values one half ahead, into two register buffers each
    // (buffer = u).  Past the end the prefetches re-read the last tile, so
    // every half runs the same straight-line code.
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
        // half (t, 0): softmax head of (t, 0); S^T of (t, 1) with the softmax
        // tail of (t, 0); PV of (t, 0)
        softmax_head<D>(st0, t0, 0, srow, half, scale2, rs, msub);
        s_product<D>(kB1, qB, st1);
        load_k<D>(t1, 1, lane, kB1);
        load_v<D>(t0, 1, lane, vB1);
        softmax_tail<D>(st0, msub, rs, pB);
        pv_product<D>(vB0, pB, rs);
        // half (t, 1): the same with S^T of (t+1, 0)
        softmax_head<D>(st1, t0, 1, srow, half, scale2, rs, msub);
        s_product<D>(kB0, qB, st0);
        load_k<D>(t2, 0, lane, kB0);
        load_v<D>(t1, 0, lane, vB0);
        softmax_tail<D>(st1, msub, rs, pB);
        pv_product<D>(vB1, pB, rs);
        t0 = t1;
        t1 = t2;
    }

    // epilogue: O = acc / l, rounded to bf16; lane holds query 32*nt + l32 and
    // d = 32*mt + 8*g + 4*half + r
    bf16* op = reinterpret_cast<bf16*>(a.out) + bh * N * D;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const float l = rs.lsum[nt] + __shfl_xor(rs.lsum[nt], 32, 64);
        const float inv = 1.0f / l;
        const int64_t row = i * 64 + 32 * nt + l32;
        if (row < N) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    bf16x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = to_bf16(rs.oacc[mt][nt][4 * g + r] * inv);
                    *reinterpret_cast<bf16x4*>(op + row * D + 32 * mt + 8 * g + 4 * half) = o;
                }
        }
    }
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
    const size_t lds = sizeof(float) * (a.Nbp + 128 + (a.Nb + 15) / 16 * 8 + 32);
    const dim3 grid((unsigned)(a.BH * a.Nb));
    if (a.d == 128)
        hipLaunchKernelGGL((attn_bf16_kernel<128>), grid, dim3(64), lds, s, a);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<64>), grid, dim3(64), lds, s, a);
    return hipGetLastError();
}

}  // namespace solattn
