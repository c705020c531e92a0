/*
 * Sol-Attn CPU oracle, fp64.  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow reference that the HIP path is checked
 * against.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load it; the product path never does.  It shares no code, header,
 * table or helper with the GPU library.
 *
 * Every step below is pinned by tests/test_oracle_pins.py against closed
 * forms, invariants, library routines and hand-worked threshold rows.  The
 * pages themselves print no formula or numeric example of the operator, so
 * against the pages the semantics are parity unpinned: the score form, the
 * standard-deviation convention, the tie rule and the zeroth-order
 * correction are readings, stated where they are taken.
 *
 * What it computes (per batch b, head h; Q, K, V are [N][d] row-major):
 *
 *   1. 64-token blocks.  Nb = ceil(N/64), block j holds tokens
 *      [64j, min(N, 64j+64)), n_j tokens.  Routing works on 64-token blocks
 *      on both the query and the key side (page "英伟达开源 Sol-H3",
 *      section 2.2: scoring per 64-token block; page "MiniMax 官宣 NVIDIA Sol
 *      团队 H3 加速", section "提速来自流水线每一段的叠加": query blocks of
 *      64 tokens).
 *   2. Pooling.  qbar_j, kbar_j, vbar_j = mean of the block's n_j rows
 *      (pooled K/V summaries: page "NVIDIA 团队开源 Sol-H3 的 DGX Spark
 *      版本", section "119.68 GiB 的内存池", Sol-Attn item).
 *   3. Lightweight score.  s_ij = (qbar_i . kbar_j) / sqrt(d).  The pages do
 *      not print the score; the pooled-mean dot product is the reading taken.
 *   4. Query-adaptive threshold (page "MiniMax 官宣 ...", same section: mean
 *      plus tau times standard deviation of the query block's own scores):
 *      mu_i = mean_j s_ij, sigma_i = population standard deviation over all
 *      Nb key blocks (two passes), thr_i = mu_i + tau*sigma_i, with
 *      tau = -inf -> thr = -inf, tau = +inf -> thr = +inf, and sigma_i = 0
 *      with finite tau -> thr = mu_i.  keep_ij = (j < Pb) or (s_ij >= thr_i),
 *      Pb = ceil(prefix_len/64): prefix key blocks are always exact (page
 *      "英伟达开源 Sol-H3", section 2.2: the packed text / conditioning video /
 *      audio prefix always takes exact attention).
 *   5. Output for query row r: exact softmax terms for every token t of every
 *      kept block, exp((q_r . k_t)/sqrt(d)) * v_t; one pooled term per skipped
 *      block, n_j * exp((q_r . kbar_j)/sqrt(d)) * vbar_j, with
 *      n_j * exp((q_r . kbar_j)/sqrt(d)) in the denominator (the pages call
 *      the skipped-block term an approximate correction from pooled K/V and,
 *      on page "MiniMax 官推背书 Sol Engine", section "同一项目页上的另一种
 *      口径：3.95× 近无损", a Taylor approximation; its zeroth-order form is
 *      the reading taken).  O_r = numerator / denominator, evaluated as a
 *      plain two-pass softmax (first the maximum exponent, then the sums),
 *      deliberately not in online form.
 *
 * DENSE mode keeps every block (plain softmax attention).  A mask override
 * replaces the routing decision with the caller's keep bits.
 *
 * TOPK mode is the draft stage's fixed-ratio block-sparse attention (page
 * "NVIDIA 团队开源 Sol-H3 的 DGX Spark 版本", section "潜空间直传：384p 草稿到
 * 768p 精修": the draft runs its attention at a fixed 90 % video sparsity
 * with 64-token blocks on a block-sparse attention backend).  tau is then the kept fraction f of the
 * video (non-prefix) key blocks: with Nv = Nb - Pb and k = ceil(f * Nv),
 * query block i keeps the prefix and every video block whose score is at
 * least the k-th largest video score of its row (ties at that score are all
 * kept).  The pages do not say how the draft picks its blocks; ranking by the
 * same pooled score is the reading taken.  Skipped blocks contribute nothing
 * (plain block-sparse attention, no pooled term).
 *
 * Two routing variants, as flag bits added to the mode (other readings of
 * passages the main reading resolves one way):
 *   PREFIX_ROWS (0x10, with SPARSE or TOPK): the prefix takes exact
 *     attention on the query side too -- query blocks i < Pb keep every key
 *     block (thr_i = -inf).  Page "英伟达开源 Sol-H3", section 2.2, says the
 *     packed prefix always takes exact attention without naming a side.
 *   VIDEO_STATS (0x20, with SPARSE): mu_i and sigma_i are taken over the
 *     video key blocks j >= Pb only (the prefix blocks are kept anyway); a
 *     row with no video block has thr_i = +inf.  Page "MiniMax 官宣 ...",
 *     section "提速来自流水线每一段的叠加", speaks of the query block's own
 *     score statistics without saying whether the always-kept prefix enters
 *     them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BLOCK 64

enum { ORACLE_DENSE = 0, ORACLE_SPARSE = 1, ORACLE_TOPK = 2 };
enum { ORACLE_BASE_MASK = 0x0f, ORACLE_PREFIX_ROWS = 0x10, ORACLE_VIDEO_STATS = 0x20 };

/* Number of tokens in block j. */
static int64_t block_len(int64_t N, int64_t j) {
    int64_t lo = j * ORACLE_BLOCK;
    int64_t hi = lo + ORACLE_BLOCK;
    if (hi > N) hi = N;
    return hi - lo;
}

static double dot(const double* a, const double* b, int64_t d) {
    double s = 0.0;
    for (int64_t c = 0; c < d; ++c) s += a[c] * b[c];
    return s;
}

/* Step 2: block means of x [N][d] into xbar [Nb][d]. */
static void pool_blocks(const double* x, int64_t N, int64_t d, double* xbar) {
    int64_t Nb = (N + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    for (int64_t j = 0; j < Nb; ++j) {
        int64_t n = block_len(N, j);
        for (int64_t c = 0; c < d; ++c) {
            double s = 0.0;
            for (int64_t t = 0; t < n; ++t) s += x[(j * ORACLE_BLOCK + t) * d + c];
            xbar[j * d + c] = s / (double)n;
        }
    }
}

/* Step 4 for one query block: threshold of a score row, with the statistics
 * taken over the blocks [lo, Nb) (lo = 0: the whole row; lo = Pb: the video
 * blocks; +inf when that range is empty). */
static double row_threshold(const double* s, int64_t lo, int64_t Nb, double tau) {
    if (isinf(tau)) return tau;  /* -inf keeps all, +inf keeps only the prefix */
    if (lo >= Nb) return INFINITY;
    const double n = (double)(Nb - lo);
    double mu = 0.0;
    for (int64_t j = lo; j < Nb; ++j) mu += s[j];
    mu /= n;
    double var = 0.0;
    for (int64_t j = lo; j < Nb; ++j) var += (s[j] - mu) * (s[j] - mu);
    double sigma = sqrt(var / n);
    if (sigma == 0.0) return mu;
    return mu + tau * sigma;
}

static int cmp_desc(const void* a, const void* b) {
    double x = *(const double*)a, y = *(const double*)b;
    return (x < y) - (x > y);
}

/* TOPK mode: the k-th largest of the video scores s[Pb..Nb) (k >= 1), found
 * by sorting a copy; +inf when k = 0 (nothing but the prefix is kept). */
static double kth_largest(const double* s, int64_t Pb, int64_t Nb, int64_t k, double* scratch) {
    if (k < 1) return INFINITY;
    int64_t nv = Nb - Pb;
    memcpy(scratch, s + Pb, sizeof(double) * nv);
    qsort(scratch, (size_t)nv, sizeof(double), cmp_desc);
    return scratch[k - 1];
}

/* Number of video key blocks TOPK mode keeps per row: ceil(f * (Nb - Pb)),
 * evaluated in double. */
static int64_t topk_count(double f, int64_t Pb, int64_t Nb) {
    int64_t nv = Nb - Pb;
    int64_t k = (int64_t)ceil(f * (double)nv);
    return k > nv ? nv : k;
}

/* Step 5 for one query row.  `pooled` = skipped blocks add their pooled term
 * (Sol-Attn); 0 = they contribute nothing (TOPK's block-sparse attention). */
static void attend_row(const double* qr, const double* k, const double* v,
                       const double* kbar, const double* vbar, const uint8_t* keep, int pooled,
                       int64_t N, int64_t d, double* logit_buf, double* o) {
    int64_t Nb = (N + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    double scale = 1.0 / sqrt((double)d);
    /* pass 1: every exponent, and their maximum */
    double m = -INFINITY;
    int64_t n_terms = 0;
    for (int64_t j = 0; j < Nb; ++j) {
        if (keep[j]) {
            for (int64_t t = j * ORACLE_BLOCK; t < j * ORACLE_BLOCK + block_len(N, j); ++t) {
                double e = dot(qr, k + t * d, d) * scale;
                logit_buf[n_terms++] = e;
                if (e > m) m = e;
            }
        } else if (pooled) {
            double e = dot(qr, kbar + j * d, d) * scale;
            logit_buf[n_terms++] = e;
            if (e > m) m = e;
        }
    }
    /* pass 2: weighted sums */
    double den = 0.0;
    for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
    n_terms = 0;
    for (int64_t j = 0; j < Nb; ++j) {
        if (keep[j]) {
            for (int64_t t = j * ORACLE_BLOCK; t < j * ORACLE_BLOCK + block_len(N, j); ++t) {
                double w = exp(logit_buf[n_terms++] - m);
                den += w;
                for (int64_t c = 0; c < d; ++c) o[c] += w * v[t * d + c];
            }
        } else if (pooled) {
            double w = (double)block_len(N, j) * exp(logit_buf[n_terms++] - m);
            den += w;
            for (int64_t c = 0; c < d; ++c) o[c] += w * vbar[j * d + c];
        }
    }
    for (int64_t c = 0; c < d; ++c) o[c] /= den;
}

/*
 * One (b, h) slice.
 *   q, k, v      [N][d] fp64.
 *   mode         0 dense, 1 sparse (Sol-Attn), 2 topk (tau = kept fraction of
 *                the video key blocks, 0 < tau <= 1; no pooled terms), plus
 *                the flags PREFIX_ROWS (0x10, sparse or topk) and
 *                VIDEO_STATS (0x20, sparse).
 *   mask_override [Nb][Nb] keep bits (0/1) or NULL; when given it is used
 *                as is (no prefix forcing) in either mode.
 *   qblocks      list of query blocks to produce, or NULL for all of them.
 *   out          [N][d] or NULL: rows of the listed query blocks are written.
 *   mask_out     [Nb][Nb] or NULL; score_out [Nb][Nb] or NULL; thr_out [Nb]
 *                or NULL: rows of the listed query blocks are written.
 *   qbar_out, kbar_out, vbar_out  [Nb][d] or NULL (all blocks).
 * Returns 0, or -1 for invalid arguments (d < 1, N < 1, prefix_len outside
 * [0, N], NaN tau, unknown mode or flag, a flag its mode does not take, topk
 * fraction outside (0, 1]), or -2 when memory runs out.
 */
int solattn_oracle_head(const double* q, const double* k, const double* v,
                        int64_t N, int64_t d, int64_t prefix_len, double tau, int mode,
                        const uint8_t* mask_override, const int64_t* qblocks,
                        int64_t n_qblocks, double* out, uint8_t* mask_out,
                        double* score_out, double* thr_out, double* qbar_out,
                        double* kbar_out, double* vbar_out, int threads) {
    const int flags = mode & ~ORACLE_BASE_MASK;
    mode &= ORACLE_BASE_MASK;
    if (!q || !k || !v || N < 1 || d < 1 || prefix_len < 0 || prefix_len > N || isnan(tau) ||
        (mode != ORACLE_DENSE && mode != ORACLE_SPARSE && mode != ORACLE_TOPK))
        return -1;
    if (flags & ~(ORACLE_PREFIX_ROWS | ORACLE_VIDEO_STATS)) return -1;
    if ((flags & ORACLE_PREFIX_ROWS) && mode == ORACLE_DENSE) return -1;
    if ((flags & ORACLE_VIDEO_STATS) && mode != ORACLE_SPARSE) return -1;
    if (mode == ORACLE_TOPK && !(tau > 0.0 && tau <= 1.0)) return -1;
    int64_t Nb = (N + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    int64_t Pb = (prefix_len + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    double* qbar = (double*)malloc(sizeof(double) * Nb * d);
    double* kbar = (double*)malloc(sizeof(double) * Nb * d);
    double* vbar = (double*)malloc(sizeof(double) * Nb * d);
    if (!qbar || !kbar || !vbar) {
        free(qbar); free(kbar); free(vbar);
        return -2;
    }
    pool_blocks(q, N, d, qbar);
    pool_blocks(k, N, d, kbar);
    pool_blocks(v, N, d, vbar);
    if (qbar_out) memcpy(qbar_out, qbar, sizeof(double) * Nb * d);
    if (kbar_out) memcpy(kbar_out, kbar, sizeof(double) * Nb * d);
    if (vbar_out) memcpy(vbar_out, vbar, sizeof(double) * Nb * d);

    int64_t n_list = qblocks ? n_qblocks : Nb;
    double scale = 1.0 / sqrt((double)d);
    int err = 0;
#ifdef _OPENMP
    if (threads < 1) threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads)
#endif
    for (int64_t li = 0; li < n_list; ++li) {
        int64_t i = qblocks ? qblocks[li] : li;
        if (i < 0 || i >= Nb) { err = -1; continue; }
        uint8_t* keep = (uint8_t*)malloc(Nb);
        double* s = (double*)malloc(sizeof(double) * Nb);
        double* logit_buf = (double*)malloc(sizeof(double) * (N + Nb));
        double* sorted = (double*)malloc(sizeof(double) * Nb);
        if (!keep || !s || !logit_buf || !sorted) {
            free(keep); free(s); free(logit_buf); free(sorted);
            err = -2;
            continue;
        }
        /* step 3: one score per key block */
        for (int64_t j = 0; j < Nb; ++j) s[j] = dot(qbar + i * d, kbar + j * d, d) * scale;
        /* step 4: routing */
        double thr = -INFINITY;
        if (mask_override) {
            for (int64_t j = 0; j < Nb; ++j) keep[j] = mask_override[i * Nb + j] ? 1 : 0;
        } else if (mode == ORACLE_DENSE) {
            for (int64_t j = 0; j < Nb; ++j) keep[j] = 1;
        } else {
            if ((flags & ORACLE_PREFIX_ROWS) && i < Pb)
                thr = -INFINITY;  /* a prefix query block keeps every key block */
            else if (mode == ORACLE_TOPK)
                thr = kth_largest(s, Pb, Nb, topk_count(tau, Pb, Nb), sorted);
            else
                thr = row_threshold(s, (flags & ORACLE_VIDEO_STATS) ? Pb : 0, Nb, tau);
            for (int64_t j = 0; j < Nb; ++j) keep[j] = (j < Pb) || (s[j] >= thr);
        }
        if (mask_out) memcpy(mask_out + i * Nb, keep, Nb);
        if (score_out) memcpy(score_out + i * Nb, s, sizeof(double) * Nb);
        if (thr_out) thr_out[i] = thr;
        /* step 5: output rows of this query block */
        if (out) {
            for (int64_t r = i * ORACLE_BLOCK; r < i * ORACLE_BLOCK + block_len(N, i); ++r)
                attend_row(q + r * d, k, v, kbar, vbar, keep, mode != ORACLE_TOPK, N, d,
                           logit_buf, out + r * d);
        }
        free(keep); free(s); free(logit_buf); free(sorted);
    }
    free(qbar); free(kbar); free(vbar);
    return err;
}

/*
 * Whole tensors [B][H][N][d]; per-slice arrays are laid out the same way with
 * the slice index b*H + h leading (mask [B][H][Nb][Nb], thr [B][H][Nb], ...).
 */
int solattn_oracle_forward(const double* q, const double* k, const double* v, double* out,
                           int64_t B, int64_t H, int64_t N, int64_t d, int64_t prefix_len,
                           double tau, int mode, const uint8_t* mask_override,
                           uint8_t* mask_out, double* score_out, double* thr_out, int threads) {
    if (B < 1 || H < 1 || N < 1 || d < 1) return -1;
    int64_t Nb = (N + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    for (int64_t bh = 0; bh < B * H; ++bh) {
        int rc = solattn_oracle_head(
            q + bh * N * d, k + bh * N * d, v + bh * N * d, N, d, prefix_len, tau, mode,
            mask_override ? mask_override + bh * Nb * Nb : NULL, NULL, 0,
            out ? out + bh * N * d : NULL, mask_out ? mask_out + bh * Nb * Nb : NULL,
            score_out ? score_out + bh * Nb * Nb : NULL, thr_out ? thr_out + bh * Nb : NULL,
            NULL, NULL, NULL, threads);
        if (rc) return rc;
    }
    return 0;
}
