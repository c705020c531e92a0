// Step 1 of Sol-Attn: 64-token block pooling (page "NVIDIA 团队开源 Sol-H3 的
// DGX Spark 版本", section "119.68 GiB 的内存池", Sol-Attn item: the pooled
// K/V summaries; page "MiniMax 官宣 NVIDIA Sol 团队 H3 加速", section
// "提速来自流水线每一段的叠加": 64-token query blocks and pooled K/V).
//
// One workgroup (256 threads) per (head slice, 64-token block).  Rows are read
// with fully coalesced 16-byte loads, summed in fp32 in a fixed order, and the
// means written in the layouts the routing and attention kernels read.  For
// bf16 inputs the same pass relays the block's V rows out into the MFMA
// operand order of the attention kernel (a transpose through LDS), so the PV
// contraction reads whole 1 KiB runs per load instruction.
//
// Bound: HBM bandwidth (reads 3 x 64 x d elements per block, writes the value
// tile once more for bf16).
//
// The same file holds produce_pool_kernel, the Q/K producer (QKNorm then
// partial RoPE) fused with this pass, and the launches of both, which put
// the (batch, head) slices on grid y in ranges within its limit.
#include "common.h"
#include "launch.h"
#include "producer.h"

namespace solattn {

template <typename T>
struct Vec16;  // 16 bytes of T
template <>
struct Vec16<float> {
    static constexpr int n = 4;
    typedef f32x4 type;
};
template <>
struct Vec16<bf16> {
    static constexpr int n = 8;
    typedef bf16x8 type;
};

template <typename T, int D>
__device__ inline void load_rows(const T* __restrict__ base, int n, int tid,
                                 float (&acc)[Vec16<T>::n], typename Vec16<T>::type* keep) {
    constexpr int VEC = Vec16<T>::n;
    constexpr int CPR = D / VEC;           // 16-byte chunks per row
    constexpr int RPP = 256 / CPR;         // rows per pass
    constexpr int PASSES = 64 / RPP;
    const int c = tid % CPR, r0 = tid / CPR;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = r0 + p * RPP;
        typename Vec16<T>::type x;
        if (r < n) {
            // (non-temporal: the pass reads each row once; see write_key_tile)
            x = __builtin_nontemporal_load(
                reinterpret_cast<const typename Vec16<T>::type*>(base + (int64_t)r * D + c * VEC));
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) x[e] = (T)0.f;
        }
        if (keep) keep[p] = x;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += (float)x[e];
    }
}

// Column sums of the per-thread partials -> block mean in red[0..D) (LDS).
template <typename T, int D>
__device__ inline void reduce_mean(const float (&acc)[Vec16<T>::n], int n, int tid, float* red,
                                   float* mean) {
    constexpr int VEC = Vec16<T>::n;
    constexpr int CPR = D / VEC;
    constexpr int RPP = 256 / CPR;
    const int c = tid % CPR, g = tid / CPR;
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[g * D + c * VEC + e] = acc[e];
    __syncthreads();
    if (tid < D) {
        float s = 0.f;
        for (int gg = 0; gg < RPP; ++gg) s += red[gg * D + tid];
        mean[tid] = s / (float)n;
    }
    __syncthreads();
}

// Relayout of one staged 64-row tile (LDS, row-major, zero rows past the
// block) into MFMA operand order; consecutive threads write consecutive
// 16-byte groups.
// The operand-ordered tiles are written, and the rows they come from read,
// with non-temporal hints: the pass streams twice the size of K and V
// through the caches, and with ordinary accesses the next kernels of a call
// (the routing, whose query rows come cold from HBM) pay for evicting it --
// the routing plan measured 73.5 -> 56.1 us at the refine shape, the call
// 2.5 % shorter, the attention kernel that later reads the tiles unchanged.
template <int D>
__device__ inline void write_key_tile(const bf16 (*tile)[D + 8], bf16* dst, int tid) {
    constexpr int KS = D / 16;
    for (int g = tid; g < D * 8; g += 256) {
        const int lane = g & 63, us = g >> 6;
        const int u = us / KS, s = us % KS;
        const int row = 32 * u + (lane & 31), col = 16 * s + 8 * (lane >> 5);
        __builtin_nontemporal_store(*reinterpret_cast<const bf16x8*>(&tile[row][col]),
                                    reinterpret_cast<bf16x8*>(dst + g * 8));
    }
}

template <int D>
__device__ inline void write_value_tile(const bf16 (*tile)[D + 8], bf16* dst, int tid) {
    for (int g = tid; g < D * 8; g += 256) {
        const int lane = g & 63, ms = g >> 6;
        const int mt = ms >> 2, s = ms & 3;
        const int dcol = 32 * mt + (lane & 31), half = lane >> 5;
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = tile[vtile_key(s, half, e)][dcol];
        __builtin_nontemporal_store(o, reinterpret_cast<bf16x8*>(dst + g * 8));
    }
}

// Pooled key `kk` of a 64-key tile, channel dcol, into the operand-ordered
// pooled key and value tiles.
template <int D>
__device__ inline void put_pooled_kv(bf16* kbarP, bf16* vbarP, int kk, int dcol, float km,
                                     float vm) {
    constexpr int KS = D / 16;
    // key: row kk of the tile, column dcol
    const int s = dcol / 16, half = (dcol / 8) & 1, e = dcol & 7;
    kbarP[ktile_offset(KS, kk / 32, s, 32 * half + (kk & 31), e)] = to_bf16(km);
    int vs, vh, ve;
    vtile_slot(kk, &vs, &vh, &ve);
    vbarP[vtile_offset(dcol / 32, vs, 32 * vh + (dcol & 31), ve)] = to_bf16(vm);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
    constexpr int VEC = Vec16<T>::n;
    constexpr int CPR = D / VEC;
    constexpr int RPP = 256 / CPR;
    constexpr int PASSES = 64 / RPP;
    __shared__ float red[RPP * D];
    __shared__ float mean[D];
    __shared__ bf16 tile[64][D + 8];  // staging for the operand relayout (bf16 only)

    const int tid = threadIdx.x;
    const int64_t j = blockIdx.x, bh = blockIdx.y;
    const int64_t Nb = a.Nb, Nbp = a.Nbp, N = a.N;
    const bool bf = a.dtype == kBF16;

    // pooled-operand slot of pooled key j (tile j/64, key j%64 of that tile)
    const int kk = (int)(j & 63);
    bf16* kbarP = bf ? reinterpret_cast<bf16*>(a.kbarP) + (bh * (Nbp / 64) + j / 64) * D * 64 : nullptr;
    bf16* vbarP = bf ? reinterpret_cast<bf16*>(a.vbarP) + (bh * (Nbp / 64) + j / 64) * D * 64 : nullptr;
    auto put_pooled = [&](int dcol, float km, float vm) {
        put_pooled_kv<D>(kbarP, vbarP, kk, dcol, km, vm);
    };

    if (j >= Nb) {
        // padding of the pooled tiles: zero keys and values (their logits are
        // masked to -inf; zeros keep 0 * value finite)
        if (!a.pooled) return;
        if (tid < D) {
            a.kbarT[(bh * D + tid) * Nbp + j] = 0.f;
            if (bf) put_pooled(tid, 0.f, 0.f);
        }
        return;
    }

    const int n = (int)((j + 1) * 64 <= N ? 64 : N - j * 64);
    const int64_t row0 = bh * N + j * 64;
    const bool pack = bf && a.pack;
    float acc[VEC];
    typename Vec16<T>::type keep[PASSES];
    auto stage = [&]() {
        const int c = tid % CPR, r0 = tid / CPR;
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
#pragma unroll
            for (int e = 0; e < VEC; ++e) tile[r0 + p * RPP][c * VEC + e] = (bf16)keep[p][e];
    };

    if (a.pooled && a.qmeans) {
        load_rows<T, D>(reinterpret_cast<const T*>(a.q) + row0 * D, n, tid, acc, nullptr);
        reduce_mean<T, D>(acc, n, tid, red, mean);
        if (tid < D) a.qbar[(bh * Nb + j) * D + tid] = mean[tid];
    }
    // K: means, and the operand-ordered key tile
    if (a.pooled || pack) {
        load_rows<T, D>(reinterpret_cast<const T*>(a.k) + row0 * D, n, tid, acc, keep);
        if (a.pooled) {
            reduce_mean<T, D>(acc, n, tid, red, mean);
            if (tid < D) {
                a.kbar[(bh * Nb + j) * D + tid] = mean[tid];
                a.kbarT[(bh * D + tid) * Nbp + j] = mean[tid];
            }
        }
        if (pack) {
            stage();
            __syncthreads();
            write_key_tile<D>(tile, reinterpret_cast<bf16*>(a.kP) + (bh * Nb + j) * (int64_t)D * 64, tid);
            __syncthreads();
        }
    }
    // V: means, and the operand-ordered value tile
    load_rows<T, D>(reinterpret_cast<const T*>(a.v) + row0 * D, n, tid, acc, keep);
    if (a.pooled) {
        const float km = tid < D ? mean[tid] : 0.f;  // K mean, still in LDS
        __syncthreads();
        reduce_mean<T, D>(acc, n, tid, red, mean);
        if (tid < D) {
            a.vbar[(bh * Nb + j) * D + tid] = mean[tid];
            if (bf) put_pooled(tid, km, mean[tid]);
        }
    }
    if (pack) {
        stage();
        __syncthreads();
        write_value_tile<D>(tile, reinterpret_cast<bf16*>(a.vP) + (bh * Nb + j) * (int64_t)D * 64, tid);
    }
}

// ---------------------------------------------------------------------------
// Pooling from received INT8 records: the receive side of the sequence-
// parallel exchange (page "MiniMax 官宣 NVIDIA Sol 团队 H3 加速:5 秒视频 1.653
// 秒生成并开源", section "提速来自流水线每一段的叠加", multi-GPU item: INT8
// Q/K/V; page "英伟达开源 Sol-H3，给 MiniMax-H3 加速，5 秒视频 1.4 秒出",
// section "2.2 剩下三层加速": 144-byte records) fused with step 1, so that
// the dequantized K and V never reach device memory as bf16 rows.  A thread
// takes the same 16-byte chunk of the same rows as pool_kernel<bf16, D>:
// 8 codes (one 8-byte load) and the record's scale, code * s in fp32
// rounded to bf16 -- the unpack kernel's arithmetic -- then sums, means and
// operand-ordered tiles exactly as pool_kernel computes them from loaded
// rows, so the workspace is bit for bit what unpacking and then pooling
// leaves.  Q rows also go to q_out (the attention reads its queries from
// there); in dense mode only q_out and the key and value tiles are written.
template <int D>
__device__ inline bf16x8 decode_chunk(const UnpackPoolArgs& u, int64_t bh, int64_t N,
                                      int64_t tok, int which, int c) {
    constexpr int REC = (D + 4 + 15) / 16 * 16;
    const int64_t src = tok / u.Ns, t = tok % u.Ns;
    const int64_t b = bh / u.Hp, hp = bh % u.Hp;
    const uint8_t* in = u.recv + ((((src * u.B + b) * u.Hp + hp) * u.Ns + t) * 3 + which) * REC;
    const uint2 w = *reinterpret_cast<const uint2*>(in + c * 8);
    const float sc = *reinterpret_cast<const float*>(in + D);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t word = e < 4 ? w.x : w.y;
        const int code = (int)(int8_t)((word >> (8 * (e & 3))) & 0xffu);
        o[e] = to_bf16((float)code * sc);
    }
    return o;
}

template <int D>
__device__ inline void decode_rows(const UnpackPoolArgs& u, int64_t bh, int64_t N, int64_t tok0,
                                   int which, int n, int tid, float (&acc)[8], bf16x8* keep,
                                   bf16* q_out) {
    constexpr int CPR = D / 8, RPP = 256 / CPR, PASSES = 64 / RPP;
    const int c = tid % CPR, r0 = tid / CPR;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = r0 + p * RPP;
        bf16x8 x;
        if (r < n) {
            x = decode_chunk<D>(u, bh, N, tok0 + r, which, c);
            if (q_out) *reinterpret_cast<bf16x8*>(q_out + (bh * N + tok0 + r) * D + c * 8) = x;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (bf16)0.f;
        }
        if (keep) keep[p] = x;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (float)x[e];
    }
}

template <int D>
__global__ __launch_bounds__(256) void unpack_pool_kernel(PoolArgs a, UnpackPoolArgs u) {
    constexpr int CPR = D / 8;
    constexpr int RPP = 256 / CPR;
    constexpr int PASSES = 64 / RPP;
    __shared__ float red[RPP * D];
    __shared__ float mean[D];
    __shared__ bf16 tile[64][D + 8];

    const int tid = threadIdx.x;
    const int64_t j = blockIdx.x, bh = blockIdx.y;
    const int64_t Nb = a.Nb, Nbp = a.Nbp, N = a.N;
    const int kk = (int)(j & 63);
    bf16* kbarP = reinterpret_cast<bf16*>(a.kbarP) + (bh * (Nbp / 64) + j / 64) * D * 64;
    bf16* vbarP = reinterpret_cast<bf16*>(a.vbarP) + (bh * (Nbp / 64) + j / 64) * D * 64;
    if (j >= Nb) {
        // padding of the pooled tiles (sparse and top-k modes only)
        if (!a.pooled) return;
        if (tid < D) {
            a.kbarT[(bh * D + tid) * Nbp + j] = 0.f;
            put_pooled_kv<D>(kbarP, vbarP, kk, tid, 0.f, 0.f);
        }
        return;
    }
    const int n = (int)((j + 1) * 64 <= N ? 64 : N - j * 64);
    const int64_t tok0 = j * 64;
    float acc[8];
    bf16x8 keep[PASSES];
    auto stage = [&]() {
        const int c = tid % CPR, r0 = tid / CPR;
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
#pragma unroll
            for (int e = 0; e < 8; ++e) tile[r0 + p * RPP][c * 8 + e] = keep[p][e];
    };
    decode_rows<D>(u, bh, N, tok0, 0, n, tid, acc, nullptr, reinterpret_cast<bf16*>(u.q_out));
    if (a.pooled && a.qmeans) {
        reduce_mean<bf16, D>(acc, n, tid, red, mean);
        if (tid < D) a.qbar[(bh * Nb + j) * D + tid] = mean[tid];
    }
    decode_rows<D>(u, bh, N, tok0, 1, n, tid, acc, keep, nullptr);
    if (a.pooled) {
        reduce_mean<bf16, D>(acc, n, tid, red, mean);
        if (tid < D) {
            a.kbar[(bh * Nb + j) * D + tid] = mean[tid];
            a.kbarT[(bh * D + tid) * Nbp + j] = mean[tid];
        }
    }
    stage();
    __syncthreads();
    write_key_tile<D>(tile, reinterpret_cast<bf16*>(a.kP) + (bh * Nb + j) * (int64_t)D * 64, tid);
    __syncthreads();
    decode_rows<D>(u, bh, N, tok0, 2, n, tid, acc, keep, nullptr);
    if (a.pooled) {
        const float km = tid < D ? mean[tid] : 0.f;  // K mean, still in LDS
        __syncthreads();
        reduce_mean<bf16, D>(acc, n, tid, red, mean);
        if (tid < D) {
            a.vbar[(bh * Nb + j) * D + tid] = mean[tid];
            put_pooled_kv<D>(kbarP, vbarP, kk, tid, km, mean[tid]);
        }
    }
    stage();
    __syncthreads();
    write_value_tile<D>(tile, reinterpret_cast<bf16*>(a.vP) + (bh * Nb + j) * (int64_t)D * 64, tid);
}

// ---------------------------------------------------------------------------
// Fused Q/K producer: QKNorm then partial RoPE on each Q and K row, the
// results stored in the input's element type, and the block pooling of the
// same workgroup taken from those stored values (page "MiniMax 官宣 NVIDIA Sol
// 团队 H3 加速:5 秒视频 1.653 秒生成并开源", section "提速来自流水线每一段的
// 叠加", fused-operator item: QKNorm + partial RoPE with the intermediates
// kept on chip; page "NVIDIA 與 SANA Sol-Engine" news, section "技術組成").
//
// Per row of d channels: y = x / sqrt(mean(x^2) + eps) * gamma, then channel
// pairs (2i, 2i+1) with i < rope_half turn by the tabulated angle of the
// row's token: (y0, y1) -> (y0 c - y1 s, y0 s + y1 c).  Arithmetic in fp32,
// one rounding to the element type at the end.  A row is held by CPR
// consecutive lanes (16 bytes each); its sum of squares is an xor butterfly
// over those lanes, so every lane normalises with the same bits.  Pooling
// then sums the rounded values in the order pool_kernel sums loaded ones, so
// the workspace equals the one pool_kernel leaves for the stored q', k'.

template <typename T, int D>
struct RowProducer {
    static constexpr int VEC = Vec16<T>::n;
    static constexpr int CPR = D / VEC;
    static constexpr int PAIRS = VEC / 2;
    float g[VEC];  // norm weight of this thread's channels
    const float* cosp;
    const float* sinp;
    int rope_half, vec_tables, c;
    float eps;

    __device__ RowProducer(const float* gamma, const ProducerArgs& p, int tid) {
        c = tid % CPR;
#pragma unroll
        for (int e = 0; e < VEC; ++e) g[e] = gamma ? gamma[c * VEC + e] : 1.f;
        cosp = p.rope_cos;
        sinp = p.rope_sin;
        rope_half = p.rope_half;
        vec_tables = p.vec_tables;
        eps = p.eps;
    }

    // Rotation angles of this thread's pairs in the row of token t: table
    // entries where the row lies inside the sequence (valid) and the pair is
    // rotated, else cos 1, sin 0 (an exact identity).
    __device__ void load_angles(int64_t t, bool valid, float (&cs)[PAIRS],
                                float (&sn)[PAIRS]) const {
        const int p0 = c * PAIRS;  // first pair of this thread
#pragma unroll
        for (int i = 0; i < PAIRS; ++i) cs[i] = 1.f, sn[i] = 0.f;
        if (!valid || p0 >= rope_half) return;
        const int64_t o = t * rope_half + p0;
        if (vec_tables) {
            // rope_half is a multiple of PAIRS and the tables are aligned to
            // PAIRS floats: this thread's pairs are one vector each
            if constexpr (PAIRS == 4) {
                const f32x4 cv = *reinterpret_cast<const f32x4*>(cosp + o);
                const f32x4 sv = *reinterpret_cast<const f32x4*>(sinp + o);
#pragma unroll
                for (int i = 0; i < 4; ++i) cs[i] = cv[i], sn[i] = sv[i];
            } else {
                const f32x2 cv = *reinterpret_cast<const f32x2*>(cosp + o);
                const f32x2 sv = *reinterpret_cast<const f32x2*>(sinp + o);
#pragma unroll
                for (int i = 0; i < 2; ++i) cs[i] = cv[i], sn[i] = sv[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < PAIRS; ++i) {
                if (p0 + i < rope_half) {
                    cs[i] = cosp[o + i];
                    sn[i] = sinp[o + i];
                }
            }
        }
    }

    // x: this thread's chunk of one row (zeros past the sequence end); cs,
    // sn: its angles.  Leaves the rounded result in x.
    __device__ void apply(typename Vec16<T>::type& x, const float (&cs)[PAIRS],
                          const float (&sn)[PAIRS]) const {
        float y[VEC];
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            y[e] = (float)x[e];
            ss = __builtin_fmaf(y[e], y[e], ss);
        }
#pragma unroll
        for (int m = 1; m < CPR; m <<= 1) ss += __shfl_xor(ss, m);
        const float rinv = 1.f / sqrtf(ss * (1.f / (float)D) + eps);
#pragma unroll
        for (int e = 0; e < VEC; ++e) y[e] = y[e] * rinv * g[e];
        const int p0 = c * PAIRS;
#pragma unroll
        for (int i = 0; i < PAIRS; ++i) {
            if (p0 + i < rope_half) {
                const float a0 = y[2 * i], a1 = y[2 * i + 1];
                y[2 * i] = a0 * cs[i] - a1 * sn[i];
                y[2 * i + 1] = a0 * sn[i] + a1 * cs[i];
            }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[e] = (T)y[e];
    }
};

// load_rows with the producer applied to every row before it is summed and
// kept; the produced rows inside the sequence are stored to `out` (if any).
// All of the thread's row chunks and angles are loaded before the first row
// is produced, so their latencies overlap.
template <typename T, int D>
__device__ inline void produce_rows(const T* __restrict__ base, T* __restrict__ out, int n,
                                    int64_t t0, int tid, const RowProducer<T, D>& prod,
                                    float (&acc)[Vec16<T>::n], typename Vec16<T>::type* keep) {
    constexpr int VEC = Vec16<T>::n;
    constexpr int CPR = D / VEC;
    constexpr int RPP = 256 / CPR;
    constexpr int PASSES = 64 / RPP;
    constexpr int PAIRS = RowProducer<T, D>::PAIRS;
    const int c = tid % CPR, r0 = tid / CPR;
    typename Vec16<T>::type xs[PASSES];
    float cs[PASSES][PAIRS], sn[PASSES][PAIRS];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = r0 + p * RPP;
        if (r < n) {
            // (non-temporal, as in load_rows: each pre-norm row is read once)
            xs[p] = __builtin_nontemporal_load(
                reinterpret_cast<const typename Vec16<T>::type*>(base + (int64_t)r * D + c * VEC));
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) xs[p][e] = (T)0.f;
        }
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) prod.load_angles(t0 + r0 + p * RPP, r0 + p * RPP < n, cs[p], sn[p]);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = r0 + p * RPP;
        typename Vec16<T>::type x = xs[p];
        prod.apply(x, cs[p], sn[p]);
        if (out && r < n)
            *reinterpret_cast<typename Vec16<T>::type*>(out + (int64_t)r * D + c * VEC) = x;
        if (keep) keep[p] = x;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += (float)x[e];
    }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void produce_pool_kernel(PoolArgs a, ProducerArgs pr) {
    constexpr int VEC = Vec16<T>::n;
    constexpr int CPR = D / VEC;
    constexpr int RPP = 256 / CPR;
    constexpr int PASSES = 64 / RPP;
    __shared__ float red[RPP * D];
    __shared__ float mean[D];
    __shared__ bf16 tile[64][D + 8];

    const int tid = threadIdx.x;
    // token blocks run fastest through the grid, as in pool_kernel: one head
    // streams through contiguous memory at a time, and with the block count a
    // multiple of eight each XCD serves the same eighth of the blocks -- and
    // of the rotary table rows -- for every head, so those rows stay in its L2
    // from one head to the next (measured 15 % faster than heads-fastest)
    const int64_t j = blockIdx.x, bh = blockIdx.y;
    const int64_t Nb = a.Nb, Nbp = a.Nbp, N = a.N;
    const bool bf = a.dtype == kBF16;
    const int kk = (int)(j & 63);
    const bool pooled_tiles = bf && a.pooled;
    bf16* kbarP = pooled_tiles ? reinterpret_cast<bf16*>(a.kbarP) + (bh * (Nbp / 64) + j / 64) * D * 64 : nullptr;
    bf16* vbarP = pooled_tiles ? reinterpret_cast<bf16*>(a.vbarP) + (bh * (Nbp / 64) + j / 64) * D * 64 : nullptr;

    if (j >= Nb) {
        // padding of the pooled tiles, as in pool_kernel
        if (!a.pooled) return;
        if (tid < D) {
            a.kbarT[(bh * D + tid) * Nbp + j] = 0.f;
            if (bf) put_pooled_kv<D>(kbarP, vbarP, kk, tid, 0.f, 0.f);
        }
        return;
    }

    const int n = (int)((j + 1) * 64 <= N ? 64 : N - j * 64);
    const int64_t row0 = bh * N + j * 64;
    const bool pack = bf && a.pack;
    float acc[VEC];
    typename Vec16<T>::type keep[PASSES];
    auto stage = [&]() {
        const int c = tid % CPR, r0 = tid / CPR;
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
#pragma unroll
            for (int e = 0; e < VEC; ++e) tile[r0 + p * RPP][c * VEC + e] = (bf16)keep[p][e];
    };

    // Q': stored; its block mean
    {
        const RowProducer<T, D> prod(pr.gamma_q, pr, tid);
        produce_rows<T, D>(reinterpret_cast<const T*>(a.q) + row0 * D,
                           reinterpret_cast<T*>(pr.q_out) + row0 * D, n, j * 64, tid, prod, acc,
                           nullptr);
    }
    if (a.pooled && a.qmeans) {
        reduce_mean<T, D>(acc, n, tid, red, mean);
        if (tid < D) a.qbar[(bh * Nb + j) * D + tid] = mean[tid];
    }
    // K': stored if asked; means and the operand-ordered key tile
    {
        const RowProducer<T, D> prod(pr.gamma_k, pr, tid);
        T* ko = pr.k_out ? reinterpret_cast<T*>(pr.k_out) + row0 * D : nullptr;
        produce_rows<T, D>(reinterpret_cast<const T*>(a.k) + row0 * D, ko, n, j * 64, tid, prod,
                           acc, keep);
    }
    if (a.pooled) {
        reduce_mean<T, D>(acc, n, tid, red, mean);
        if (tid < D) {
            a.kbar[(bh * Nb + j) * D + tid] = mean[tid];
            a.kbarT[(bh * D + tid) * Nbp + j] = mean[tid];
        }
    }
    if (pack) {
        stage();
        __syncthreads();
        write_key_tile<D>(tile, reinterpret_cast<bf16*>(a.kP) + (bh * Nb + j) * (int64_t)D * 64, tid);
        __syncthreads();
    }
    if (!a.pooled && !pack) return;  // the producer alone
    // V: as pool_kernel
    load_rows<T, D>(reinterpret_cast<const T*>(a.v) + row0 * D, n, tid, acc, keep);
    if (a.pooled) {
        const float km = tid < D ? mean[tid] : 0.f;  // K mean, still in LDS
        __syncthreads();
        reduce_mean<T, D>(acc, n, tid, red, mean);
        if (tid < D) {
            a.vbar[(bh * Nb + j) * D + tid] = mean[tid];
            if (bf) put_pooled_kv<D>(kbarP, vbarP, kk, tid, km, mean[tid]);
        }
    }
    if (pack) {
        stage();
        __syncthreads();
        write_value_tile<D>(tile, reinterpret_cast<bf16*>(a.vP) + (bh * Nb + j) * (int64_t)D * 64, tid);
    }
}

// The pooling grids put the (batch, head) slices on grid y, whose documented
// limit is 65536: larger counts are launched in ranges of heads, each a
// launch of its own over pointers advanced to its first head (every per-head
// region of the inputs and the workspace is contiguous in the slice index).
constexpr int64_t kMaxGridY = 65535;

template <typename P>
P* advance(P* p, int64_t bytes) {
    return p ? reinterpret_cast<P*>(reinterpret_cast<uintptr_t>(p) + bytes) : p;
}

PoolArgs heads_from(const PoolArgs& a, int64_t h0) {
    const int64_t es = a.dtype == kBF16 ? 2 : 4, D = a.d;
    PoolArgs b = a;
    b.q = advance(a.q, h0 * a.N * D * es);
    b.k = advance(a.k, h0 * a.N * D * es);
    b.v = advance(a.v, h0 * a.N * D * es);
    b.qbar = advance(a.qbar, h0 * a.Nb * D * 4);
    b.kbar = advance(a.kbar, h0 * a.Nb * D * 4);
    b.vbar = advance(a.vbar, h0 * a.Nb * D * 4);
    b.kbarT = advance(a.kbarT, h0 * D * a.Nbp * 4);
    b.kbarP = advance(a.kbarP, h0 * a.Nbp * D * 2);
    b.vbarP = advance(a.vbarP, h0 * a.Nbp * D * 2);
    b.kP = advance(a.kP, h0 * a.Nb * 64 * D * 2);
    b.vP = advance(a.vP, h0 * a.Nb * 64 * D * 2);
    return b;
}

ProducerArgs heads_from(const ProducerArgs& p, const PoolArgs& a, int64_t h0) {
    const int64_t es = a.dtype == kBF16 ? 2 : 4;
    ProducerArgs b = p;
    b.q_out = advance(p.q_out, h0 * a.N * a.d * es);
    b.k_out = advance(p.k_out, h0 * a.N * a.d * es);
    return b;
}

hipError_t launch_produce_pool_heads(const PoolArgs& a, const ProducerArgs& p, int64_t BH,
                                     hipStream_t s) {
    const dim3 grid((unsigned)(a.pooled ? a.Nbp : a.Nb), (unsigned)BH);
    if (a.dtype == kBF16) {
        if (a.d == 128)
            hipLaunchKernelGGL((produce_pool_kernel<bf16, 128>), grid, dim3(256), 0, s, a, p);
        else
            hipLaunchKernelGGL((produce_pool_kernel<bf16, 64>), grid, dim3(256), 0, s, a, p);
    } else {
        if (a.d == 128)
            hipLaunchKernelGGL((produce_pool_kernel<float, 128>), grid, dim3(256), 0, s, a, p);
        else
            hipLaunchKernelGGL((produce_pool_kernel<float, 64>), grid, dim3(256), 0, s, a, p);
    }
    return hipGetLastError();
}

hipError_t launch_pool_heads(const PoolArgs& a, int64_t BH, hipStream_t s) {
    const dim3 grid((unsigned)(a.pooled ? a.Nbp : a.Nb), (unsigned)BH);
    if (a.dtype == kBF16) {
        if (a.d == 128)
            hipLaunchKernelGGL((pool_kernel<bf16, 128>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((pool_kernel<bf16, 64>), grid, dim3(256), 0, s, a);
    } else {
        if (a.d == 128)
            hipLaunchKernelGGL((pool_kernel<float, 128>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((pool_kernel<float, 64>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_unpack_pool(const PoolArgs& a, const UnpackPoolArgs& u, hipStream_t s) {
    // (the caller keeps B * Hp within the grid's y limit)
    const dim3 grid((unsigned)(a.pooled ? a.Nbp : a.Nb), (unsigned)(u.B * u.Hp));
    if (a.d == 128)
        hipLaunchKernelGGL((unpack_pool_kernel<128>), grid, dim3(256), 0, s, a, u);
    else
        hipLaunchKernelGGL((unpack_pool_kernel<64>), grid, dim3(256), 0, s, a, u);
    return hipGetLastError();
}

hipError_t launch_produce_pool(const PoolArgs& a, const ProducerArgs& p, int64_t BH,
                               hipStream_t s) {
    for (int64_t h0 = 0; h0 < BH; h0 += kMaxGridY) {
        const int64_t n = BH - h0 < kMaxGridY ? BH - h0 : kMaxGridY;
        const hipError_t e = launch_produce_pool_heads(heads_from(a, h0), heads_from(p, a, h0), n, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_pool(const PoolArgs& a, int64_t BH, hipStream_t s) {
    if (a.dtype != kBF16 && !a.pooled) return hipSuccess;
    for (int64_t h0 = 0; h0 < BH; h0 += kMaxGridY) {
        const int64_t n = BH - h0 < kMaxGridY ? BH - h0 : kMaxGridY;
        const hipError_t e = launch_pool_heads(heads_from(a, h0), n, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace solattn
