// Step 2 of Sol-Attn: block scores, the query-adaptive threshold and the keep
// mask of one query block, computed by one wavefront into LDS.
//
// The rule (page "MiniMax 官宣 NVIDIA Sol 团队 H3 加速:5 秒视频 1.653 秒生成并
// 开源", section "提速来自流水线每一段的叠加"; page "NVIDIA 团队开源 Sol-H3 的
// DGX Spark 版本", section "119.68 GiB 的内存池"): every query block scores all
// key blocks with a lightweight score and keeps those that clear its own
// threshold, mean + tau * standard deviation of its score row.  Key blocks of
// the packed prefix are always kept (page "英伟达开源 Sol-H3", section 2.2).
// Readings taken where the pages are silent: the score is the pooled-mean dot
// product scaled by 1/sqrt(d); the standard deviation is the population one
// over all Nb key blocks; a score equal to the threshold is kept; tau = -inf
// keeps all, tau = +inf keeps only the prefix, sigma = 0 uses the mean.
// Two variants take the other reading of a passage: prefix_rows (query
// blocks of the prefix keep every key block: the packed prefix's exact
// attention read on the query side too, page "英伟达开源 Sol-H3", section 2.2)
// and video_stats (mean and standard deviation over the video key blocks
// only; +inf when there is none).
//
// In the fixed-ratio mode the threshold is instead the k-th largest video
// score of the row (kth_largest_video) and skipped blocks get no pooled term.
//
// In a fused launch nothing of the routing reaches device memory except
// through the debug exports: the mask lives as ballot words, the kept-block
// list and the pooled-term biases in LDS.  A planning launch (the routing
// kernel, ahead of a planned attention launch) also writes each row's keep
// bits and tile count to the workspace, and the planned attention kernel
// rebuilds the same lists and biases from those bits.
#pragma once

#include "common.h"
#include "launch.h"

namespace solattn {

// Fixed-ratio routing (the draft stage's block-sparse attention at a fixed
// video sparsity, page "NVIDIA 团队开源 Sol-H3 的 DGX Spark 版本", section
// "潜空间直传：384p 草稿到 768p 精修"): the k-th largest of the video scores
// s[Pb..Nb) of a row, k >= 1, exactly, or +inf for k = 0.  Scores are mapped
// to order-preserving unsigned keys and the key of the k-th largest is built
// bit by bit from the top: a bit stays set when at least k keys are >= the
// candidate.  One wavefront; the row is in LDS.
__device__ inline uint32_t order_key(float x) {
    const uint32_t b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ inline float kth_largest_video(const float* srow, int64_t Pb, int64_t Nb, int64_t k) {
    if (k < 1) return __builtin_inff();
    const int lane = threadIdx.x & 63;
    uint32_t key = 0;
    // Rows of up to 64 * R blocks keep their keys in registers for the 32
    // rounds (a video column's key, or 0 -- which no candidate reaches, every
    // candidate having a bit set -- elsewhere); longer rows re-read the LDS.
    constexpr int R = 16;
    if (Nb <= 64 * R) {
        uint32_t kr[R];
#pragma unroll
        for (int c = 0; c < R; ++c) {
            const int64_t j = 64 * c + lane;
            kr[c] = (j >= Pb && j < Nb) ? order_key(srow[j]) : 0u;
        }
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = key | (1u << bit);
            int64_t count = 0;
#pragma unroll
            for (int c = 0; c < R; ++c)
                if (64 * c < Nb) count += __popcll(__ballot(kr[c] >= cand));
            if (count >= k) key = cand;
        }
    } else {
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = key | (1u << bit);
            int64_t count = 0;
            for (int64_t j0 = 0; j0 < Nb; j0 += 64) {
                const int64_t j = j0 + lane;
                const bool ge = j >= Pb && j < Nb && order_key(srow[j]) >= cand;
                count += __popcll(__ballot(ge));
            }
            if (count >= k) key = cand;
        }
    }
    const uint32_t b = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
    return __uint_as_float(b);
}

struct RouteResult {
    int n_kept;          // kept key blocks, listed ascending in klist[0..n_kept)
    uint64_t tile_mask;  // bit T set when pooled tile T (key blocks 64T..64T+63)
                         // holds at least one skipped block
};

// Step 1 for the query side of one bf16 query block, done by the wave that
// routes it: the block's query mean from its rows (the pooling pass then
// reads no queries).  Lane l takes the 16-byte chunk c = l % CPR of rows
// g, g + RPI, g + 2 RPI, ... (g = l / CPR); query_rows_load issues those
// loads, query_rows_mean sums them in fp32 in row order, adds the RPI
// partial sums of each chunk across lanes (xor butterfly over the row
// groups; every lane ends with the same sums) and writes sum / n to
// qm[0..D) in LDS.  Rows past the block's n rows count as zero.  Every lane
// of the wave calls both.
template <int D>
struct QueryRows {
    static constexpr int CPR = D / 8;       // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;    // rows per load instruction
    static constexpr int ITER = 64 / RPI;   // load instructions per block
    bf16x8 x[ITER];
};

template <int D>
__device__ inline void query_rows_load(const bf16* qblk, int n, QueryRows<D>& qr) {
    using R = QueryRows<D>;
    const int lane = threadIdx.x & 63, c = lane % R::CPR, g = lane / R::CPR;
    // (every load is issued -- rows past n re-read the last row and are
    // zeroed afterwards -- so that no branch sits between the loads and the
    // waits on them stay exact)
#pragma unroll
    for (int it = 0; it < R::ITER; ++it) {
        const int r = g + R::RPI * it;
        qr.x[it] = *reinterpret_cast<const bf16x8*>(qblk + (int64_t)(r < n ? r : n - 1) * D + 8 * c);
    }
#pragma unroll
    for (int it = 0; it < R::ITER; ++it) {
        if (g + R::RPI * it >= n) {
#pragma unroll
            for (int e = 0; e < 8; ++e) qr.x[it][e] = (bf16)0.f;
        }
    }
}

template <int D>
__device__ inline void query_rows_mean(const QueryRows<D>& qr, int n, float* qm) {
    using R = QueryRows<D>;
    const int lane = threadIdx.x & 63;
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.f;
#pragma unroll
    for (int it = 0; it < R::ITER; ++it)
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += (float)qr.x[it][e];
#pragma unroll
    for (int m = R::CPR; m < 64; m <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += __shfl_xor(s[e], m, 64);
    if (lane < R::CPR) {
        const float fn = (float)n;
#pragma unroll
        for (int e = 0; e < 8; ++e) qm[8 * lane + e] = s[e] / fn;
    }
}

// Routing in two parts, so that a caller can issue other memory loads
// between them (route_scores waits for all of its own loads; route_select
// issues none).  One wavefront (all 64 lanes of the workgroup).
//
// route_scores: srow[0..Nbp) = s_ij for every key block j (padding: 0).
// The query mean comes from the pooled means in the workspace (fp32 inputs)
// or, with FROM_Q (bf16), from the block's rows, formed in qm (D floats of
// LDS) before the scores.
template <int D, bool FROM_Q = false>
__device__ inline void route_scores(const AttnArgs& a, int64_t bh, int64_t i, float* srow,
                                    float* qm = nullptr) {
    const int lane = threadIdx.x & 63;
    const int64_t Nb = a.Nb, Nbp = a.Nbp;
    const float scale = 1.0f / sqrtf((float)D);

    if constexpr (FROM_Q) {
        const int n = (int)(a.N - i * 64 < 64 ? a.N - i * 64 : 64);
        QueryRows<D> qr;
        query_rows_load<D>(reinterpret_cast<const bf16*>(a.q) + (bh * a.N + i * 64) * D, n, qr);
        query_rows_mean<D>(qr, n, qm);
        __syncthreads();
    }
    const float* __restrict__ qb = FROM_Q ? qm : a.qbar + (bh * Nb + i) * D;

    // scores s_ij = qbar_i . kbar_j / sqrt(d); kbar is stored transposed so each
    // load instruction reads 1 KiB of consecutive key blocks.
    const float* __restrict__ kt = a.kbarT + bh * D * Nbp;
    // (rows of kbarT are loaded in batches of DB, DEPTH batches in flight:
    // the loads of batch b + DEPTH - 1 are issued before the FMAs of batch
    // b, so that the wave's memory latency is paid about once per 256 key
    // blocks rather than once per batch; the accumulation order over d is
    // plain ascending d)
    constexpr int DB = 16, NB = D / DB, DEPTH = 3;
    for (int64_t j0 = 4 * lane; j0 < Nbp; j0 += 256) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        f32x4 kv[DEPTH][DB];
#pragma unroll
        for (int b = 0; b < DEPTH - 1; ++b)
#pragma unroll
            for (int d = 0; d < DB; ++d)
                kv[b][d] = *reinterpret_cast<const f32x4*>(kt + (int64_t)(b * DB + d) * Nbp + j0);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b + DEPTH - 1 < NB) {
#pragma unroll
                for (int d = 0; d < DB; ++d)
                    kv[(b + DEPTH - 1) % DEPTH][d] = *reinterpret_cast<const f32x4*>(
                        kt + (int64_t)((b + DEPTH - 1) * DB + d) * Nbp + j0);
            }
#pragma unroll
            for (int d = 0; d < DB; ++d) acc += qb[b * DB + d] * kv[b % DEPTH][d];
        }
        *reinterpret_cast<f32x4*>(srow + j0) = acc * scale;
    }
    __syncthreads();
}

// The lists of a routed query block from its keep decisions: keep(j, s_j)
// for every key block j < Nb (s_j = srow[j]; a planned launch passes keep
// bits instead and its srow holds no scores yet).  On return:
//   klist[0..n_kept)  kept key-block indices (ascending)
//   srow[0..Nbp)      log2(n_j) for skipped blocks, -inf for kept and padding
//                     (the per-column bias of the pooled tiles, log2 units)
// and the keep bits, with the scores for score_out, are written to any of
// the given destinations ([BH][Nb][ceil(Nb/32)] words, [BH][Nb][Nb] floats).
template <class Keep>
__device__ inline RouteResult route_lists(const AttnArgs& a, int64_t bh, int64_t i, float* srow,
                                          uint16_t* klist, Keep keep, float* score_out,
                                          uint32_t* mask_out, uint32_t* plan_out) {
    const int lane = threadIdx.x & 63;
    const int64_t Nb = a.Nb, Nbp = a.Nbp;
    // keep bits, kept list, pooled-tile flags, pooled biases (log2 n_j: 6
    // for a full block, log2 of its key count for a ragged last block)
    int n_kept = 0;
    uint64_t tile_mask = 0;
    const int64_t W = (Nb + 31) / 32;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int nb = (int)Nb, nbp = (int)Nbp;
    const float log2_last = log2f((float)(a.N - (Nb - 1) * 64));
    for (int j0 = 0; j0 < nbp; j0 += 64) {
        const int j = j0 + lane;
        const bool valid = j < nb;
        const float s = srow[j];
        const bool kp = valid && keep(j, s);
        const bool skip = valid && !kp;
        const uint64_t kb = __ballot(kp);
        const uint64_t sb = __ballot(skip);
        if (score_out && valid) score_out[(bh * Nb + i) * Nb + j] = s;
        const int64_t w0 = j0 / 32;
        for (uint32_t* dst : {mask_out, plan_out}) {
            if (!dst) continue;
            if (lane == 0 && w0 < W) dst[(bh * Nb + i) * W + w0] = (uint32_t)kb;
            if (lane == 1 && w0 + 1 < W) dst[(bh * Nb + i) * W + w0 + 1] = (uint32_t)(kb >> 32);
        }
        if (kp) klist[n_kept + __popcll(kb & lt)] = (uint16_t)j;
        n_kept += __popcll(kb);
        if (sb && a.mode == kSparse) tile_mask |= 1ull << (j0 / 64);  // pooled terms: Sol-Attn only
        srow[j] = skip ? (j == nb - 1 ? log2_last : 6.0f) : -__builtin_inff();
    }
    // (no workgroup barrier here: the lists are this wave's own LDS; callers
    // synchronise before other waves, or later code, read them)
    return RouteResult{n_kept, tile_mask};
}

// route_select, from the scores in srow (one wavefront): the threshold, then
// route_lists with keep_j = (j < Pb or s_j >= threshold), writing the debug
// exports and, in a planning launch, the keep bits to plan_mask.
__device__ inline RouteResult route_select(const AttnArgs& a, int64_t bh, int64_t i, float* srow,
                                           uint16_t* klist) {
    const int lane = threadIdx.x & 63;
    const int64_t Nb = a.Nb;
    float thr;
    if (a.prefix_rows && i < a.Pb) {
        thr = -__builtin_inff();  // a prefix query block keeps every key block
    } else if (a.mode == kTopk) {
        thr = kth_largest_video(srow, a.Pb, Nb, a.topk);
    } else if (__builtin_isinf(a.tau)) {
        thr = a.tau;
    } else {
        // row statistics, two passes (mean, then squared deviations), over the
        // whole row or, with video_stats, over the video blocks [Pb, Nb)
        const int64_t lo = a.video_stats ? a.Pb : 0;
        if (lo >= Nb) {
            thr = __builtin_inff();  // no video block: only the prefix is kept
        } else {
            const float n = (float)(Nb - lo);
            float part = 0.f;
            for (int64_t j = lo + lane; j < Nb; j += 64) part += srow[j];
            const float mu = wave_sum(part) / n;
            part = 0.f;
            for (int64_t j = lo + lane; j < Nb; j += 64) {
                const float t = srow[j] - mu;
                part += t * t;
            }
            const float sigma = sqrtf(wave_sum(part) / n);
            thr = sigma == 0.f ? mu : mu + a.tau * sigma;
        }
    }
    const int pb = (int)a.Pb;
    const RouteResult r = route_lists(
        a, bh, i, srow, klist, [&](int j, float s) { return j < pb || s >= thr; }, a.score_out,
        a.mask_out, a.plan_mask);
    if (a.thr_out && lane == 0) a.thr_out[bh * Nb + i] = thr;
    return r;
}

// The routing of query block i from its keep bits (a planned launch): the
// row's ceil(Nb/32) words, already in LDS at words[], through route_lists;
// the same lists and biases route_select leaves for the same bits.
__device__ inline RouteResult route_from_bits(const AttnArgs& a, int64_t bh, int64_t i,
                                              const uint32_t* words, float* srow,
                                              uint16_t* klist) {
    return route_lists(
        a, bh, i, srow, klist, [&](int j, float) { return (words[j >> 5] >> (j & 31)) & 1u; },
        nullptr, nullptr, nullptr);
}

template <int D>
__device__ inline RouteResult route_query_block(const AttnArgs& a, int64_t bh, int64_t i,
                                                float* srow, uint16_t* klist) {
    route_scores<D>(a, bh, i, srow);
    return route_select(a, bh, i, srow, klist);
}

// Dense mode exports: every bit set, threshold -inf.
__device__ inline void export_dense_route(const AttnArgs& a, int64_t bh, int64_t i) {
    const int lane = threadIdx.x & 63;
    const int64_t Nb = a.Nb, W = (Nb + 31) / 32;
    if (a.mask_out) {
        for (int64_t w = lane; w < W; w += 64) {
            const int64_t bits = Nb - 32 * w;
            a.mask_out[(bh * Nb + i) * W + w] = bits >= 32 ? 0xffffffffu : ((1u << bits) - 1u);
        }
    }
    if (a.thr_out && lane == 0) a.thr_out[bh * Nb + i] = -__builtin_inff();
}

}  // namespace solattn
