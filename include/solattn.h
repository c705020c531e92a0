/*
 * solattn.h -- C interface of the Sol-Attn block-sparse attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (forward only, non-causal, one scale 1/sqrt(d)):
 *
 *   Tokens of every (batch, head) slice are cut into 64-token blocks on the
 *   query and on the key side (page "英伟达开源 Sol-H3，给 MiniMax-H3 加速，
 *   5 秒视频 1.4 秒出", section 2.2; page "MiniMax 官宣 NVIDIA Sol 团队 H3
 *   加速:5 秒视频 1.653 秒生成并开源", section "提速来自流水线每一段的叠加").
 *   Nb = ceil(N/64); block j has n_j = min(64, N - 64j) tokens.
 *
 *   1. Pooling: qbar_j, kbar_j, vbar_j are the means of each block's rows
 *      (page "NVIDIA 团队开源 Sol-H3 的 DGX Spark 版本", section "119.68 GiB
 *      的内存池", Sol-Attn item: pooled K/V summaries).
 *   2. Routing: s_ij = qbar_i . kbar_j / sqrt(d).  Query block i keeps key
 *      block j when j < ceil(prefix_len/64) (the always-exact prefix of the
 *      packed sequence) or s_ij >= mu_i + tau*sigma_i, where mu_i and sigma_i
 *      are the mean and population standard deviation of row i over all Nb
 *      key blocks.  tau = -inf keeps everything, tau = +inf only the prefix,
 *      and sigma_i = 0 uses the threshold mu_i.
 *   3. Kept blocks contribute exact softmax terms exp(q_r.k_t/sqrt(d)) v_t.
 *   4. Each skipped block contributes one pooled term
 *      n_j exp(q_r.kbar_j/sqrt(d)) vbar_j to the numerator and
 *      n_j exp(q_r.kbar_j/sqrt(d)) to the denominator (the pages' pooled
 *      correction, taken at zeroth order).
 *   5. Routing, exact terms and pooled terms share one online softmax per
 *      query row; no score map and no routing index is written to device
 *      memory (only the debug entry point exports them).
 *
 * Conventions shared by every entry point:
 *   - q, k, v, out: caller-owned device pointers to contiguous row-major
 *     [B][H][N][d] tensors, all of element type `dtype`, 16-byte aligned.
 *     Inputs are read only; `out` must not overlap any input.
 *   - B, H, N >= 1; d is 64 or 128; 0 <= prefix_len <= N; N <= 262144.
 *   - tau may be +-infinity; NaN is rejected.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *     work on it and return without synchronising; completion is observed
 *     through the stream.
 *   - Every argument is checked on the host before any device call; a
 *     rejected call enqueues nothing and returns a nonzero code whose text
 *     solattn_last_error() gives.
 *   - Calls on different streams may run concurrently.  The entry points
 *     without a `ws` argument (solattn_forward, solattn_forward_debug,
 *     solattn_pool, solattn_route) keep one internal workspace per (device,
 *     stream), grown on demand (a growth allocates once; a buffer once
 *     handed out is kept, not freed, until the process ends), so their calls
 *     on different streams never share memory; calls on one stream are
 *     ordered by the stream.  Because they may allocate, they refuse a
 *     stream that is being captured into a graph (SOLATTN_EUNSUPPORTED,
 *     nothing enqueued); under capture use the _ws entry points or
 *     solattn_forward_noalloc.
 *   - Every pointer the kernels will read or write must be device memory
 *     HIP knows (hipMalloc / torch device tensors; managed memory is
 *     accepted): host pointers are rejected with SOLATTN_EINVAL before any
 *     launch.
 */
#ifndef SOLATTN_H
#define SOLATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define SOLATTN_OK 0
#define SOLATTN_EINVAL 1       /* argument outside the documented domain */
#define SOLATTN_EUNSUPPORTED 2 /* valid but not built (e.g. N > 262144) */
#define SOLATTN_EHIP 3         /* HIP runtime or launch error */
#define SOLATTN_ENOMEM 4       /* workspace allocation failed */

/* mode */
#define SOLATTN_DENSE 0  /* every key block exact (plain softmax attention) */
#define SOLATTN_SPARSE 1 /* Sol-Attn routing */
/*
 * Fixed-ratio block-sparse attention, the draft stage's scheme (page "NVIDIA
 * 团队开源 Sol-H3 的 DGX Spark 版本", section "潜空间直传：384p 草稿到 768p
 * 精修": a fixed 90 % video sparsity with 64-token blocks on a block-sparse
 * attention backend).  tau is then the kept fraction f of the video
 * (non-prefix) key blocks, 0 < f <= 1: with Nv = Nb - ceil(prefix_len/64)
 * and k = ceil(f * Nv) (evaluated in double from the float f), query block i
 * keeps the prefix blocks and every video block whose score s_ij (as above)
 * is at least the k-th largest video score of row i (ties all kept).  Skipped
 * blocks contribute nothing: no pooled term.
 */
#define SOLATTN_TOPK 2

/*
 * Routing variants, OR-ed into mode (the base mode is mode & SOLATTN_MODE_MASK).
 * Each takes the other reading of a passage the default routing reads one
 * way; a flag outside the modes named here is SOLATTN_EINVAL.
 *   SOLATTN_PREFIX_ROWS (SPARSE or TOPK): the packed prefix's exact attention
 *     (page "英伟达开源 Sol-H3", section 2.2) read on the query side too:
 *     query blocks i < ceil(prefix_len/64) keep every key block (their rows
 *     are plain dense attention; threshold -inf in the debug export).
 *   SOLATTN_VIDEO_STATS (SPARSE): the mean and standard deviation of the
 *     threshold (page "MiniMax 官宣 NVIDIA Sol 团队 H3 加速:5 秒视频 1.653
 *     秒生成并开源", section "提速来自流水线每一段的叠加") are taken over the
 *     video key blocks j >= ceil(prefix_len/64) only; a row with no video
 *     block has threshold +inf (only the prefix is kept).
 */
#define SOLATTN_MODE_MASK 0x0f
#define SOLATTN_PREFIX_ROWS 0x10
#define SOLATTN_VIDEO_STATS 0x20
/*
 * SOLATTN_TAYLOR1 (SPARSE, bf16; may be combined with the two flags above):
 * the skipped blocks' pooled term taken to first order (page "MiniMax 官推
 * 背书 Sol Engine：H3 的 10 秒 768p 生成从 414s 压到 14.93s", section "同一项目
 * 页上的另一种口径：3.95× 近无损", which calls the compensation a Taylor
 * approximation).  Skipped block j's value vbar_j becomes, for query row r,
 * vbar_j + c C_j^T q_r with C_j = (1/n_j) sum_t (k_t - kbar_j)(v_t - vbar_j)^T,
 * c = 1/sqrt(d); its weight n_j exp(c q_r.kbar_j) and the denominator are
 * unchanged (their first-order term is zero).  An accuracy mode: every
 * skipped block's key and value tiles are read and multiplied, about the
 * cost of dense attention.  With fp32 data: SOLATTN_EUNSUPPORTED.
 */
#define SOLATTN_TAYLOR1 0x40

/* dtype */
#define SOLATTN_F32 0
#define SOLATTN_BF16 1

/*
 * Full forward pass: pooling (step 1) then steps 2-5 -- for launches of
 * B*H*ceil(N/64) >= 2048 query blocks in bf16 SPARSE / TOPK the routing
 * plan and the attention that follows it (solattn_plan_ws and
 * solattn_attend_plan_ws below), otherwise one kernel that routes each
 * query block and attends.  In DENSE mode tau and prefix_len are ignored and no
 * pooling is done; in TOPK mode tau is the kept fraction (outside (0, 1]:
 * SOLATTN_EINVAL).  Uses the internal workspace of (current device,
 * stream), allocated or grown on first need.
 */
int solattn_forward(const void* q, const void* k, const void* v, void* out, int64_t B,
                    int64_t H, int64_t N, int64_t d, int64_t prefix_len, float tau, int mode,
                    int dtype, void* stream);

/* Bytes of workspace solattn_forward_ws needs for this shape and dtype. */
size_t solattn_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype);

/*
 * solattn_forward with a caller-owned device workspace `ws` of `ws_bytes`
 * bytes (at least solattn_workspace_bytes(), 256-byte aligned).  Allocates
 * nothing.  `ws` must not be used by another call until this one completes
 * on `stream`.
 */
int solattn_forward_ws(const void* q, const void* k, const void* v, void* out, int64_t B,
                       int64_t H, int64_t N, int64_t d, int64_t prefix_len, float tau, int mode,
                       int dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * solattn_forward for callers that cannot allocate device memory at call
 * time: code being captured into a HIP graph, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments, modes, results and
 * errors as solattn_forward (the same kernels run), but the workspace is a
 * fixed array of SOLATTN_NOALLOC_SCRATCH_BYTES bytes in the library's device
 * code, one copy per GPU held until the process ends, so the call
 * allocates nothing and enqueues only kernels on `stream`.  Shapes whose
 * workspace (solattn_workspace_bytes) exceeds it -- e.g. B=1, H=32,
 * N=16384, d=128 in bf16 -- are rejected with SOLATTN_EUNSUPPORTED before
 * any device call; 64 MiB covers, for instance, one GPU's four heads of
 * that shape (H=4).  Every call on one GPU uses the same array: calls that
 * overlap in time on one GPU (two streams, two host threads) race and must
 * be serialised by the caller.  The first call on each GPU resolves the
 * array's device address (a runtime query that may load the library's
 * device code): make it once before capturing.
 */
#define SOLATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
int solattn_forward_noalloc(const void* q, const void* k, const void* v, void* out,
                            int64_t B, int64_t H, int64_t N, int64_t d, int64_t prefix_len,
                            float tau, int mode, int dtype, void* stream);

/*
 * The two stages of solattn_forward_ws as separate launches, so that each
 * can be timed on its own.  solattn_prepare_ws runs step 1 (pooling into the
 * workspace; in DENSE mode only the value-tile relayout the attention kernel
 * reads).  solattn_attend_ws runs steps 2-5 and reads what prepare left in
 * the same workspace for the same q, k, v, shape, dtype and mode.  For bf16,
 * solattn_attend_ws reads only q and the workspace (keys and values come
 * from the tiles prepare wrote): k and v may then be NULL.
 */
int solattn_prepare_ws(const void* q, const void* k, const void* v, int64_t B, int64_t H,
                       int64_t N, int64_t d, int mode, int dtype, void* ws, size_t ws_bytes,
                       void* stream);
int solattn_attend_ws(const void* q, const void* k, const void* v, void* out, int64_t B,
                      int64_t H, int64_t N, int64_t d, int64_t prefix_len, float tau, int mode,
                      int dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * solattn_attend_ws split in two for bf16 SPARSE and TOPK (with either
 * routing flag; not SOLATTN_TAYLOR1): the routing plan, then the attention
 * that follows it.  For launches of B*H*ceil(N/64) >= 2048 query blocks
 * solattn_attend_ws runs exactly these two steps; below that it routes
 * inside the attention kernel.  The output is the same either way, bit for
 * bit: the routing arithmetic is shared and each query block's attention
 * does not depend on the order the blocks run in.
 *
 * solattn_plan_ws: step 2 (page "MiniMax 官宣 NVIDIA Sol 团队 H3 加速:5 秒
 * 视频 1.653 秒生成并开源", section "提速来自流水线每一段的叠加": block scores,
 * mean + tau * std threshold, keep mask) for every query block, on a
 * workspace solattn_prepare_ws filled for the same q, shape, dtype and mode.
 * Writes into ws each block's keep bits and the number of 64-key tiles its
 * attention will run, then the dispatch order of the attention launch:
 * within each (head, XCD) share of the launch, longest first.
 * solattn_attend_plan_ws: steps 3-5 (exact kept tiles, pooled correction,
 * one online softmax; page "NVIDIA 团队开源 Sol-H3 的 DGX Spark 版本",
 * section "119.68 GiB 的内存池") from the plan and tiles in ws into out
 * ([B][H][N][d] bf16); mode must be the one the plan was made with.  Both
 * allocate nothing, enqueue kernels on `stream`, and return
 * SOLATTN_EUNSUPPORTED for fp32, DENSE or SOLATTN_TAYLOR1.
 */
int solattn_plan_ws(const void* q, int64_t B, int64_t H, int64_t N, int64_t d,
                    int64_t prefix_len, float tau, int mode, int dtype, void* ws, size_t ws_bytes,
                    void* stream);
int solattn_attend_plan_ws(const void* q, void* out, int64_t B, int64_t H, int64_t N, int64_t d,
                           int mode, int dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * solattn_forward plus an export of the routing each query block used, from
 * the same device code: mask_out [B][H][Nb][ceil(Nb/32)] uint32 words (bit
 * j%32 of word j/32 in row i is keep_ij), score_out [B][H][Nb][Nb] fp32
 * scores s_ij, thr_out [B][H][Nb] fp32 thresholds (-inf / +inf for tau =
 * -inf / +inf; -inf in DENSE mode, where the mask is all ones; in TOPK mode
 * the k-th largest video score, +inf when k = 0).  Any export pointer may be
 * NULL.  For tests and measurement only.
 */
int solattn_forward_debug(const void* q, const void* k, const void* v, void* out, int64_t B,
                          int64_t H, int64_t N, int64_t d, int64_t prefix_len, float tau,
                          int mode, int dtype, uint32_t* mask_out, float* score_out,
                          float* thr_out, void* stream);

/*
 * Step 1 alone: block means as fp32 [B][H][Nb][d] into caller buffers
 * (any may be NULL).
 */
int solattn_pool(const void* q, const void* k, const void* v, float* qbar, float* kbar,
                 float* vbar, int64_t B, int64_t H, int64_t N, int64_t d, int dtype,
                 void* stream);

/*
 * Steps 1-2 alone (the routing "setup": pooling and scoring, no attention),
 * with the exports of solattn_forward_debug.  Uses the internal workspace.
 */
int solattn_route(const void* q, const void* k, const void* v, int64_t B, int64_t H,
                  int64_t N, int64_t d, int64_t prefix_len, float tau, int dtype,
                  uint32_t* mask_out, float* score_out, float* thr_out, void* stream);

/*
 * Step 2 alone on a workspace that solattn_prepare_ws (SPARSE or TOPK mode,
 * same shape and dtype) has filled: the block scores, thresholds and keep
 * bits of every query block, with the exports of solattn_forward_debug (any
 * may be NULL).  The scoring pass on its own (page "Sol-H3" news, kocpc,
 * section "技術組成", reports the routing setup time on its own).  Reads the
 * pooled key means in ws and the query means: for fp32 the ones prepare
 * wrote to ws, for bf16 formed from the query rows of q (the bf16 kernels
 * form each query block's mean from its rows; prepare writes none).
 * Allocates nothing.
 */
int solattn_route_ws(const void* q, int64_t B, int64_t H, int64_t N, int64_t d,
                     int64_t prefix_len, float tau, int dtype, const void* ws, size_t ws_bytes,
                     uint32_t* mask_out, float* score_out, float* thr_out, void* stream);

/* Static text of a return code. */
const char* solattn_strerror(int code);

/* Text of the last error raised on the calling thread ("" if none). */
const char* solattn_last_error(void);

/* Library version string. */
const char* solattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SOLATTN_H */
