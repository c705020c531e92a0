// Internal host <-> kernel interface of the Sol-Attn library: workspace layout,
// kernel argument blocks and launch functions.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace solattn {

enum Dtype { kF32 = 0, kBF16 = 1 };
enum Mode { kDense = 0, kSparse = 1, kTopk = 2 };

// Workspace regions (byte offsets, each 256-byte aligned).  BH = B*H,
// Nb = ceil(N/64), Nbp = Nb rounded up to a multiple of 64.
//   qbar, kbar, vbar  fp32 [BH][Nb][d]     block means (qbar: fp32 inputs and the
//                                          pooled-means export only)
//   kbarT             fp32 [BH][d][Nbp]    block means of K, transposed for the
//                                          coalesced score pass; zero padded
//   kbarP             bf16 [BH][Nbp/64][64*d] pooled keys, MFMA operand order (bf16 only)
//   vbarP             bf16 [BH][Nbp/64][d*64] pooled values, MFMA operand order
//   kP                bf16 [BH][Nb][64*d]  key tiles, MFMA operand order
//   vP                bf16 [BH][Nb][d*64]  value tiles, MFMA operand order
//   plan_mask         u32  [BH][Nb][ceil(Nb/32)] routed keep bits (bf16 only;
//                                          bit j%32 of word j/32 in row i)
//   plan_cost         i32  [BH*Nb]         tiles each query block will run
//   plan_perm         i32  [BH*Nb]         dispatch order: work item of each
//                                          launch position
struct WsLayout {
    size_t qbar, kbar, vbar, kbarT, kbarP, vbarP, kP, vP, plan_mask, plan_cost, plan_perm, total;
};

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

inline WsLayout ws_layout(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
    const int64_t BH = B * H, Nb = (N + 63) / 64, Nbp = (Nb + 63) / 64 * 64;
    WsLayout w;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    w.qbar = take(sizeof(float) * BH * Nb * d);
    w.kbar = take(sizeof(float) * BH * Nb * d);
    w.vbar = take(sizeof(float) * BH * Nb * d);
    w.kbarT = take(sizeof(float) * BH * d * Nbp);
    if (dtype == kBF16) {
        w.kbarP = take(2 * BH * Nbp * d);
        w.vbarP = take(2 * BH * Nbp * d);
        w.kP = take(2 * BH * Nb * 64 * d);
        w.vP = take(2 * BH * Nb * 64 * d);
        w.plan_mask = take(sizeof(uint32_t) * BH * Nb * ((Nb + 31) / 32));
        w.plan_cost = take(sizeof(int32_t) * BH * Nb);
        w.plan_perm = take(sizeof(int32_t) * BH * Nb);
    } else {
        w.kbarP = w.vbarP = w.kP = w.vP = w.plan_mask = w.plan_cost = w.plan_perm = 0;
    }
    w.total = off;
    return w;
}

struct PoolArgs {
    const void* q;
    const void* k;
    const void* v;
    float* qbar;
    float* kbar;
    float* vbar;
    float* kbarT;
    void* kbarP;
    void* vbarP;
    void* kP;
    void* vP;
    int64_t N, Nb, Nbp;
    int d, dtype;
    int pooled;   // compute block means (sparse and topk modes)
    int qmeans;   // with pooled: the query means too (fp32 inputs, and the
                  // pooled-means export; the bf16 attention and routing
                  // kernels form each query block's mean from its rows)
    int pack;     // write the operand-ordered key and value tiles (bf16)
};

struct AttnArgs {
    const void* q;
    const void* k;
    const void* kP;       // bf16: key tiles in operand order; f32: unused
    const void* vP;       // bf16: value tiles in operand order; f32: unused
    const void* v;        // f32 path reads V directly
    const void* kbarP;
    const void* vbarP;
    const float* kbar;    // f32 path pooled operands
    const float* vbar;
    const float* qbar;
    const float* kbarT;
    void* out;
    uint32_t* mask_out;   // debug exports (NULL in production)
    float* score_out;
    float* thr_out;
    int64_t BH, N, Nb, Nbp;
    int64_t Pb;
    float tau;
    int64_t topk;         // kTopk: video key blocks kept per query block
    int d, dtype, mode;   // mode: kDense, kSparse or kTopk (the flags below apart)
    int prefix_rows;      // query blocks i < Pb keep every key block
    int video_stats;      // kSparse: threshold statistics over key blocks j >= Pb
    // Routing plan (bf16 kSparse / kTopk).  The routing kernel writes the keep
    // bits and tile counts when plan_mask / plan_cost are set; the order
    // kernel writes plan_perm from plan_cost; the attention kernel, given
    // plan_perm, takes its work item from it and its routing from plan_mask
    // instead of routing the query block itself.  NULL: no plan.
    uint32_t* plan_mask;
    int32_t* plan_cost;
    int32_t* plan_perm;
};

// Sequence-parallel transport (transport.hip); record = d codes + fp32 scale,
// padded to a multiple of 16 bytes.
struct QkvPackArgs {        // q, k, v [B][H][Ns][d] bf16 -> send [P][B][Hp][Ns][3][rec]
    const void* q;
    const void* k;
    const void* v;
    uint8_t* send;
    int64_t B, H, Hp, Ns, P;
};
struct QkvUnpackArgs {      // recv [P][B][Hp][Ns][3][rec] -> q, k, v [B][Hp][P*Ns][d] bf16
    const uint8_t* recv;
    void* q;
    void* k;
    void* v;
    int64_t B, Hp, Ns, P;
};
struct OutPackArgs {        // o [B][Hp][P*Ns][d] bf16 -> send [P][B][Hp][Ns][rec]
    const void* o;
    uint8_t* send;
    int64_t B, Hp, Ns, P;
};
struct OutUnpackArgs {      // recv [P][B][Hp][Ns][rec] -> o [B][P*Hp][Ns][d] bf16
    const uint8_t* recv;
    void* o;
    int64_t B, Hp, Ns, P;
};
hipError_t launch_pack_qkv_int8(const QkvPackArgs& a, int d, hipStream_t s);
hipError_t launch_unpack_qkv_int8(const QkvUnpackArgs& a, int d, hipStream_t s);
hipError_t launch_pack_out_fp8(const OutPackArgs& a, int d, hipStream_t s);
hipError_t launch_unpack_out_fp8(const OutUnpackArgs& a, int d, hipStream_t s);

// Pooling straight from received INT8 Q/K/V records (transport layout
// [P][B][Hp][Ns][3][rec]; the slice bh = b * Hp + hp covers N = P * Ns
// tokens): the rows are dequantized in registers as the unpack kernel
// dequantizes them, Q rows are written to q_out, and the workspace of a is
// filled as pool_kernel fills it from the unpacked tensors (bf16 only).
struct UnpackPoolArgs {
    const uint8_t* recv;
    void* q_out;
    int64_t B, Hp, Ns, P;
};
hipError_t launch_unpack_pool(const PoolArgs& a, const UnpackPoolArgs& u, hipStream_t s);

hipError_t launch_pool(const PoolArgs& a, int64_t BH, hipStream_t s);
hipError_t launch_route(const AttnArgs& a, hipStream_t s);
hipError_t launch_order(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);

// bf16 MFMA peak probe: `waves` wavefronts x `iters` x 16 MFMAs 32x32x16.
hipError_t launch_probe_mfma(float* sink, int64_t waves, int64_t iters, hipStream_t s);

}  // namespace solattn
