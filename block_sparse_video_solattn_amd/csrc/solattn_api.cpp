// Host side of the Sol-Attn C ABI: argument checks, the internal workspaces
// (one per device and stream), and the launch sequence (pool, then fused
// route + attention).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/solattn.h"
#include "../../include/solattn_probe.h"
#include "../../include/solattn_producer.h"
#include "../../include/solattn_transport.h"
#include "launch.h"
#include "producer.h"
#include "taylor.h"

using namespace solattn;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(SOLATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxN = 64LL * 4096;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Every check happens here, on the host, before any device call.
int validate(const void* q, const void* k, const void* v, const void* out, bool need_out,
             int64_t B, int64_t H, int64_t N, int64_t d, int64_t prefix_len, float tau, int mode,
             int dtype, bool kv_optional = false) {
    g_last_error.clear();
    if (!q) return fail(SOLATTN_EINVAL, "q must be non-NULL");
    if (!kv_optional && (!k || !v)) return fail(SOLATTN_EINVAL, "q, k and v must be non-NULL");
    if (need_out && !out) return fail(SOLATTN_EINVAL, "out must be non-NULL");
    if (B < 1 || H < 1 || N < 1)
        return fail(SOLATTN_EINVAL, "B, H, N must be >= 1 (got %lld, %lld, %lld)", (long long)B,
                    (long long)H, (long long)N);
    if (d != 64 && d != 128) return fail(SOLATTN_EINVAL, "d must be 64 or 128 (got %lld)", (long long)d);
    if (prefix_len < 0 || prefix_len > N)
        return fail(SOLATTN_EINVAL, "prefix_len must lie in [0, N] (got %lld)", (long long)prefix_len);
    if (std::isnan(tau)) return fail(SOLATTN_EINVAL, "tau must not be NaN");
    const int base = mode & SOLATTN_MODE_MASK, flags = mode & ~SOLATTN_MODE_MASK;
    if (base != SOLATTN_DENSE && base != SOLATTN_SPARSE && base != SOLATTN_TOPK)
        return fail(SOLATTN_EINVAL, "unknown mode %d", mode);
    if (flags & ~(SOLATTN_PREFIX_ROWS | SOLATTN_VIDEO_STATS | SOLATTN_TAYLOR1))
        return fail(SOLATTN_EINVAL, "unknown mode flags 0x%x", flags);
    if ((flags & SOLATTN_TAYLOR1) && base != SOLATTN_SPARSE)
        return fail(SOLATTN_EINVAL, "SOLATTN_TAYLOR1 needs SPARSE");
    if ((flags & SOLATTN_PREFIX_ROWS) && base == SOLATTN_DENSE)
        return fail(SOLATTN_EINVAL, "SOLATTN_PREFIX_ROWS needs SPARSE or TOPK");
    if ((flags & SOLATTN_VIDEO_STATS) && base != SOLATTN_SPARSE)
        return fail(SOLATTN_EINVAL, "SOLATTN_VIDEO_STATS needs SPARSE");
    if (base == SOLATTN_TOPK && need_out && !(tau > 0.f && tau <= 1.f))
        return fail(SOLATTN_EINVAL, "topk mode: tau is the kept fraction, in (0, 1] (got %g)",
                    (double)tau);
    if (dtype != SOLATTN_F32 && dtype != SOLATTN_BF16)
        return fail(SOLATTN_EINVAL, "unknown dtype %d", dtype);
    if ((flags & SOLATTN_TAYLOR1) && dtype != SOLATTN_BF16)
        return fail(SOLATTN_EUNSUPPORTED, "SOLATTN_TAYLOR1 is built for bf16 only");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (out && !aligned16(out)))
        return fail(SOLATTN_EINVAL, "tensor pointers must be 16-byte aligned");
    if (N > kMaxN)
        return fail(SOLATTN_EUNSUPPORTED, "N = %lld exceeds the supported maximum %lld",
                    (long long)N, (long long)kMaxN);
    if (B > (int64_t(1) << 40) / H || B * H > (int64_t(1) << 31) / ((N + 63) / 64))
        return fail(SOLATTN_EUNSUPPORTED, "B*H*ceil(N/64) exceeds 2^31 workgroups");
    if (out) {
        const size_t bytes = (size_t)B * H * N * d * (dtype == SOLATTN_BF16 ? 2 : 4);
        if (overlaps(out, bytes, q, bytes) || (k && overlaps(out, bytes, k, bytes)) ||
            (v && overlaps(out, bytes, v, bytes)))
            return fail(SOLATTN_EINVAL, "out must not overlap q, k or v");
    }
    return SOLATTN_OK;
}

// Transport calls: shapes (each factor >= 1, d 64 or 128, every launch's
// rows well inside the grid limits).
int check_transport(int64_t B, int64_t H, int64_t Ns, int64_t d, int64_t P) {
    if (B < 1 || H < 1 || Ns < 1 || P < 1)
        return fail(SOLATTN_EINVAL, "B, H, Ns, P must be >= 1 (got %lld, %lld, %lld, %lld)",
                    (long long)B, (long long)H, (long long)Ns, (long long)P);
    if (d != 64 && d != 128) return fail(SOLATTN_EINVAL, "d must be 64 or 128 (got %lld)", (long long)d);
    const int64_t lim = int64_t(1) << 34;
    if (B > lim / H || B * H > lim / Ns || B * H * Ns > lim / (3 * P))
        return fail(SOLATTN_EUNSUPPORTED, "B*H*Ns*P too large");
    return SOLATTN_OK;
}

// Transport calls: non-NULL, 16-byte aligned buffers, outputs not
// overlapping inputs.
int check_buffers(std::initializer_list<const void*> in, size_t in_bytes,
                  std::initializer_list<const void*> out, size_t out_bytes) {
    for (const void* p : in)
        if (!p || !aligned16(p)) return fail(SOLATTN_EINVAL, "input buffers must be non-NULL and 16-byte aligned");
    for (const void* p : out)
        if (!p || !aligned16(p)) return fail(SOLATTN_EINVAL, "output buffers must be non-NULL and 16-byte aligned");
    size_t a = 0;
    for (const void* o : out) {
        for (const void* i : in)
            if (overlaps(o, out_bytes, i, in_bytes))
                return fail(SOLATTN_EINVAL, "output buffers must not overlap the inputs");
        size_t b = 0;
        for (const void* o2 : out)
            if (b++ > a && overlaps(o, out_bytes, o2, out_bytes))
                return fail(SOLATTN_EINVAL, "output buffers must not overlap each other");
        ++a;
    }
    return SOLATTN_OK;
}

// Every pointer the kernels will dereference must be GPU memory: a host
// pointer reaching a kernel faults the device.  Checked last, after the
// pure host-side checks, with one runtime query per distinct pointer
// (NULL entries are skipped; they were checked above where they matter).
int check_device_ptrs(std::initializer_list<const void*> ptrs) {
    const void* seen[16];
    int n = 0;
    for (const void* p : ptrs) {
        if (!p) continue;
        bool dup = false;
        for (int i = 0; i < n; ++i) dup = dup || seen[i] == p;
        if (dup) continue;
        if (n < 16) seen[n++] = p;
        hipPointerAttribute_t attr;
        const hipError_t e = hipPointerGetAttributes(&attr, p);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(SOLATTN_EINVAL, "pointer %p is not memory HIP knows (%s): pass device memory",
                        p, hipGetErrorString(e));
        }
        if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged &&
            attr.type != hipMemoryTypeUnified)
            return fail(SOLATTN_EINVAL, "pointer %p is not device memory (memory type %d)", p,
                        (int)attr.type);
    }
    return SOLATTN_OK;
}

// Internal workspaces of the plain entry points: one buffer per (device,
// stream), so that plain calls on different streams never share memory.
// A buffer handed out is never freed while the library is loaded: when a
// slot must grow, the old buffer moves to a retired list (work already
// enqueued, or a host thread that holds the pointer but has not launched
// yet, may still use it).  Growth is at least 2x, so the retired buffers of
// a slot never total more than its current one.  Everything is held until
// the process ends.
struct WsSlot {
    int dev;
    hipStream_t stream;
    void* ptr;
    size_t bytes;
};
std::mutex g_ws_mutex;
std::vector<WsSlot> g_ws;
std::vector<void*> g_ws_retired;

// The plain entry points may allocate, so they cannot be recorded into a
// graph (a captured call would also bake in a buffer a later growth
// retires).  Checked before any other runtime call of such an entry point.
int reject_capture(hipStream_t stream) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cap != hipStreamCaptureStatusNone)
        return fail(SOLATTN_EUNSUPPORTED,
                    "the stream is being captured: the entry points without a workspace argument "
                    "may allocate; use the _ws entry points under capture");
    return SOLATTN_OK;
}

int internal_ws(size_t need, hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    WsSlot* w = nullptr;
    for (WsSlot& x : g_ws)
        if (x.dev == dev && x.stream == stream) w = &x;
    if (!w) {
        g_ws.push_back(WsSlot{dev, stream, nullptr, 0});
        w = &g_ws.back();
    }
    if (w->bytes < need) {
        const size_t grow = need > 2 * w->bytes ? need : 2 * w->bytes;
        void* p = nullptr;
        e = hipMalloc(&p, grow);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(SOLATTN_ENOMEM, "workspace allocation of %zu bytes failed: %s", grow,
                        hipGetErrorString(e));
        }
        if (w->ptr) g_ws_retired.push_back(w->ptr);
        w->ptr = p;
        w->bytes = grow;
    }
    *out = w->ptr;
    return SOLATTN_OK;
}

// Workspace of solattn_forward_noalloc: a fixed device array, so that the
// call allocates nothing.  Each device holds its own copy (from the load of
// the library's device code until the process ends); host code must not use
// the array's name as an address -- it is a host-side stand-in -- but the
// per-device address from hipGetSymbolAddress, resolved on the first call
// on each device.  Nothing in it needs to start at zero: every byte the
// attention kernel reads is written earlier in the same call by the
// pooling pass (padding included).
__device__ __align__(256) unsigned char scratch[SOLATTN_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mutex;
std::vector<void*> g_scratch_ptr;  // per device; NULL until resolved

int scratch_ptr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(SOLATTN_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SOLATTN_OK;
}

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

PoolArgs pool_args(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t N,
                   int64_t d, int mode, int dtype, void* ws, bool pack, bool export_qmeans = false) {
    const WsLayout L = ws_layout(B, H, N, d, dtype);
    PoolArgs p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.qbar = reinterpret_cast<float*>(at(ws, L.qbar));
    p.kbar = reinterpret_cast<float*>(at(ws, L.kbar));
    p.vbar = reinterpret_cast<float*>(at(ws, L.vbar));
    p.kbarT = reinterpret_cast<float*>(at(ws, L.kbarT));
    p.kbarP = dtype == kBF16 ? at(ws, L.kbarP) : nullptr;
    p.vbarP = dtype == kBF16 ? at(ws, L.vbarP) : nullptr;
    p.kP = dtype == kBF16 ? at(ws, L.kP) : nullptr;
    p.vP = dtype == kBF16 ? at(ws, L.vP) : nullptr;
    p.N = N;
    p.Nb = (N + 63) / 64;
    p.Nbp = (p.Nb + 63) / 64 * 64;
    p.d = (int)d;
    p.dtype = dtype;
    p.pooled = (mode & SOLATTN_MODE_MASK) != SOLATTN_DENSE;
    p.qmeans = dtype != kBF16 || export_qmeans;
    p.pack = pack && dtype == kBF16;
    return p;
}

int run_prepare(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t N,
                int64_t d, int mode, int dtype, void* ws, hipStream_t s, bool pack,
                bool export_qmeans = false) {
    const PoolArgs p = pool_args(q, k, v, B, H, N, d, mode, dtype, ws, pack, export_qmeans);
    if (!p.pooled && !p.pack) return SOLATTN_OK;  // fp32 dense: nothing to prepare
    hipError_t e = launch_pool(p, B * H, s);
    if (e != hipSuccess) return hip_fail(e, "pool kernel launch");
    return SOLATTN_OK;
}

// Steps of run_attend: all of steps 2-5 (kStageAll), the routing alone with
// its exports (kStageRouteOnly), the routing plan alone (kStagePlan: keep
// bits, tile counts and the dispatch order into the workspace) and the
// attention from a plan already in the workspace (kStageAttendPlan).
enum Stage { kStageAll = 0, kStageRouteOnly = 1, kStagePlan = 2, kStageAttendPlan = 3 };

// Launches of B*H*Nb work items from this many on take the planned route in
// kStageAll: routing kernel, order kernel, then attention in the planned
// order.  Below it the launch is at most ~2 dispatch rounds of the chip's
// 1024 wave slots, where the order cannot shorten the last round and the
// two extra launches cost more than the routing they take out of the
// attention kernel.
constexpr int64_t kPlanMinItems = 2048;

bool plannable(int mode, int dtype) {
    const int base = mode & SOLATTN_MODE_MASK;
    return dtype == SOLATTN_BF16 && base != SOLATTN_DENSE && !(mode & SOLATTN_TAYLOR1);
}

int run_attend(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t H,
               int64_t N, int64_t d, int64_t prefix_len, float tau, int mode, int dtype, void* ws,
               hipStream_t s, uint32_t* mask_out, float* score_out, float* thr_out,
               int stage) {
    const int route_only = stage == kStageRouteOnly;
    const WsLayout L = ws_layout(B, H, N, d, dtype);
    AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.kP = dtype == kBF16 ? at(ws, L.kP) : nullptr;
    a.vP = dtype == kBF16 ? at(ws, L.vP) : nullptr;
    a.kbarP = dtype == kBF16 ? at(ws, L.kbarP) : nullptr;
    a.vbarP = dtype == kBF16 ? at(ws, L.vbarP) : nullptr;
    a.kbar = reinterpret_cast<const float*>(at(ws, L.kbar));
    a.vbar = reinterpret_cast<const float*>(at(ws, L.vbar));
    a.qbar = reinterpret_cast<const float*>(at(ws, L.qbar));
    a.kbarT = reinterpret_cast<const float*>(at(ws, L.kbarT));
    a.out = out;
    a.mask_out = mask_out;
    const int base = mode & SOLATTN_MODE_MASK;
    a.score_out = base != SOLATTN_DENSE ? score_out : nullptr;
    a.thr_out = thr_out;
    a.BH = B * H;
    a.N = N;
    a.Nb = (N + 63) / 64;
    a.Nbp = (a.Nb + 63) / 64 * 64;
    a.Pb = (prefix_len + 63) / 64;
    a.tau = tau;
    a.d = (int)d;
    a.dtype = dtype;
    a.mode = base;
    a.prefix_rows = (mode & SOLATTN_PREFIX_ROWS) != 0;
    a.video_stats = (mode & SOLATTN_VIDEO_STATS) != 0;
    // topk: k = ceil(tau * video key blocks), evaluated in double on the host
    // so that every query block (and any reference) uses the same count
    {
        const int64_t nv = a.Nb - a.Pb;
        int64_t kk = base == SOLATTN_TOPK ? (int64_t)std::ceil((double)tau * (double)nv) : 0;
        a.topk = kk > nv ? nv : kk;
    }
    a.plan_mask = nullptr;
    a.plan_cost = nullptr;
    a.plan_perm = nullptr;
    const bool plan = stage == kStagePlan || stage == kStageAttendPlan ||
                      (stage == kStageAll && plannable(mode, dtype) && a.BH * a.Nb >= kPlanMinItems);
    if (plan) {
        uint32_t* pm = reinterpret_cast<uint32_t*>(at(ws, L.plan_mask));
        int32_t* pc = reinterpret_cast<int32_t*>(at(ws, L.plan_cost));
        int32_t* pp = reinterpret_cast<int32_t*>(at(ws, L.plan_perm));
        if (stage != kStageAttendPlan) {
            // routing with the debug exports, keep bits and tile counts; then
            // the dispatch order from the counts
            a.plan_mask = pm;
            a.plan_cost = pc;
            hipError_t e = launch_route(a, s);
            if (e != hipSuccess) return hip_fail(e, "route kernel launch");
            a.plan_perm = pp;
            e = launch_order(a, s);
            if (e != hipSuccess) return hip_fail(e, "order kernel launch");
            if (stage == kStagePlan) return SOLATTN_OK;
        }
        // attention in the planned order, its routing from the keep bits
        a.plan_mask = pm;
        a.plan_cost = nullptr;
        a.plan_perm = pp;
        a.mask_out = nullptr;
        a.score_out = nullptr;
        a.thr_out = nullptr;
        const hipError_t e = launch_attn_bf16(a, s);
        if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
        return SOLATTN_OK;
    }
    hipError_t e = route_only                  ? launch_route(a, s)
                   : (mode & SOLATTN_TAYLOR1) ? launch_attn_bf16_taylor(a, s)
                   : dtype == kBF16           ? launch_attn_bf16(a, s)
                                              : launch_attn_f32(a, s);
    if (e != hipSuccess) return hip_fail(e, route_only ? "route kernel launch" : "attention kernel launch");
    return SOLATTN_OK;
}

int check_ws(void* ws, size_t ws_bytes, int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
    const size_t need = ws_layout(B, H, N, d, dtype).total;
    if (!ws) return fail(SOLATTN_EINVAL, "ws must be non-NULL");
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(SOLATTN_EINVAL, "ws must be 256-byte aligned");
    if (ws_bytes < need)
        return fail(SOLATTN_EINVAL, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    return SOLATTN_OK;
}

// Producer arguments (shapes were checked by validate()): weights, eps,
// rotary tables, the outputs and their overlaps.
int check_producer(const void* q, const void* k, const void* v, const float* gq,
                   const float* gk, float eps, int64_t rope_dim, const float* rc,
                   const float* rs, void* q_out, void* k_out, bool k_out_optional,
                   int64_t B, int64_t H, int64_t N, int64_t d, int dtype, ProducerArgs* pa) {
    if (!(eps > 0.f) || std::isinf(eps))
        return fail(SOLATTN_EINVAL, "eps must be finite and > 0 (got %g)", (double)eps);
    if (rope_dim < 0 || rope_dim > d || (rope_dim & 1))
        return fail(SOLATTN_EINVAL, "rope_dim must be even and in [0, d] (got %lld)",
                    (long long)rope_dim);
    if (rope_dim > 0 && (!rc || !rs))
        return fail(SOLATTN_EINVAL, "rope_cos and rope_sin must be non-NULL when rope_dim > 0");
    auto al4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
    if (!al4(gq) || !al4(gk) || (rope_dim > 0 && (!al4(rc) || !al4(rs))))
        return fail(SOLATTN_EINVAL, "norm weights and rotary tables must be 4-byte aligned");
    if (!q_out || (!k_out && !k_out_optional))
        return fail(SOLATTN_EINVAL, k_out_optional ? "q_out must be non-NULL"
                                                   : "q_out and k_out must be non-NULL");
    if (!aligned16(q_out) || !aligned16(k_out))
        return fail(SOLATTN_EINVAL, "q_out and k_out must be 16-byte aligned");
    const size_t tb = (size_t)B * H * N * d * (dtype == SOLATTN_BF16 ? 2 : 4);
    const size_t gb = (size_t)d * 4, tab = (size_t)N * (size_t)(rope_dim / 2) * 4;
    for (const void* o : {q_out, k_out}) {
        if (!o) continue;
        for (const void* i : {q, k, v})
            if (i && overlaps(o, tb, i, tb))
                return fail(SOLATTN_EINVAL, "q_out and k_out must not overlap q, k or v");
        if ((gq && overlaps(o, tb, gq, gb)) || (gk && overlaps(o, tb, gk, gb)) ||
            (tab && (overlaps(o, tb, rc, tab) || overlaps(o, tb, rs, tab))))
            return fail(SOLATTN_EINVAL, "q_out and k_out must not overlap the weights or tables");
    }
    if (k_out && overlaps(q_out, tb, k_out, tb))
        return fail(SOLATTN_EINVAL, "q_out and k_out must not overlap each other");
    const int pairs = dtype == SOLATTN_BF16 ? 4 : 2;  // rotary pairs per thread chunk
    const uintptr_t vmask = (uintptr_t)pairs * 4 - 1;
    pa->gamma_q = gq;
    pa->gamma_k = gk;
    pa->rope_cos = rope_dim > 0 ? rc : nullptr;
    pa->rope_sin = rope_dim > 0 ? rs : nullptr;
    pa->q_out = q_out;
    pa->k_out = k_out;
    pa->eps = eps;
    pa->rope_half = (int)(rope_dim / 2);
    pa->vec_tables = rope_dim > 0 && (rope_dim / 2) % pairs == 0 &&
                     (reinterpret_cast<uintptr_t>(rc) & vmask) == 0 &&
                     (reinterpret_cast<uintptr_t>(rs) & vmask) == 0;
    return SOLATTN_OK;
}

}  // namespace

extern "C" {

int solattn_qknorm_rope(const void* q, const void* k, const float* gamma_q,
                        const float* gamma_k, float eps, int64_t rope_dim,
                        const float* rope_cos, const float* rope_sin, void* q_out, void* k_out,
                        int64_t B, int64_t H, int64_t N, int64_t d, int dtype, void* stream) {
    // v is not read: q stands in for it in the shared shape checks
    int rc = validate(q, k, q, nullptr, false, B, H, N, d, 0, 0.f, SOLATTN_DENSE, dtype);
    if (rc) return rc;
    ProducerArgs pa;
    if ((rc = check_producer(q, k, nullptr, gamma_q, gamma_k, eps, rope_dim, rope_cos, rope_sin,
                             q_out, k_out, false, B, H, N, d, dtype, &pa)))
        return rc;
    if ((rc = check_device_ptrs({q, k, q_out, k_out, gamma_q, gamma_k, pa.rope_cos, pa.rope_sin})))
        return rc;
    PoolArgs p = {};
    p.q = q;
    p.k = k;
    p.N = N;
    p.Nb = (N + 63) / 64;
    p.Nbp = (p.Nb + 63) / 64 * 64;
    p.d = (int)d;
    p.dtype = dtype;
    p.pooled = 0;
    p.pack = 0;
    hipError_t e = launch_produce_pool(p, pa, B * H, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "producer kernel launch");
    return SOLATTN_OK;
}

int solattn_prepare_qknorm_rope_ws(const void* q, const void* k, const void* v,
                                   const float* gamma_q, const float* gamma_k, float eps,
                                   int64_t rope_dim, const float* rope_cos,
                                   const float* rope_sin, void* q_out, void* k_out, int64_t B,
                                   int64_t H, int64_t N, int64_t d, int mode, int dtype,
                                   void* ws, size_t ws_bytes, void* stream) {
    int rc = validate(q, k, v, nullptr, false, B, H, N, d, 0, 0.f, mode, dtype);
    if (rc) return rc;
    if ((rc = check_ws(ws, ws_bytes, B, H, N, d, dtype))) return rc;
    ProducerArgs pa;
    if ((rc = check_producer(q, k, v, gamma_q, gamma_k, eps, rope_dim, rope_cos, rope_sin, q_out,
                             k_out, dtype == SOLATTN_BF16, B, H, N, d, dtype, &pa)))
        return rc;
    if ((rc = check_device_ptrs({q, k, v, q_out, k_out, gamma_q, gamma_k, pa.rope_cos, pa.rope_sin,
                                 ws})))
        return rc;
    const PoolArgs p = pool_args(q, k, v, B, H, N, d, mode, dtype, ws, true);
    hipError_t e = launch_produce_pool(p, pa, B * H, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "producer kernel launch");
    return SOLATTN_OK;
}

size_t solattn_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
    if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128) || (dtype != 0 && dtype != 1)) return 0;
    return ws_layout(B, H, N, d, dtype).total;
}

int solattn_forward_ws(const void* q, const void* k, const void* v, void* out, int64_t B,
                       int64_t H, int64_t N, int64_t d, int64_t prefix_len, float tau, int mode,
                       int dtype, void* ws, size_t ws_bytes, void* stream) {
    int rc = validate(q, k, v, out, true, B, H, N, d, prefix_len, tau, mode, dtype);
    if (rc) return rc;
    if ((rc = check_ws(ws, ws_bytes, B, H, N, d, dtype))) return rc;
    if ((rc = check_device_ptrs({q, k, v, out, ws}))) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = run_prepare(q, k, v, B, H, N, d, mode, dtype, ws, s, true))) return rc;
    return run_attend(q, k, v, out, B, H, N, d, prefix_len, tau, mode, dtype, ws, s, nullptr,
                      nullptr, nullptr, 0);
}

int solattn_forward(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t H,
                    int64_t N, int64_t d, int64_t prefix_len, float tau, int mode, int dtype,
                    void* stream) {
    int rc = validate(q, k, v, out, true, B, H, N, d, prefix_len, tau, mode, dtype);
    if (rc) return rc;
    if ((rc = reject_capture(static_cast<hipStream_t>(stream)))) return rc;
    if ((rc = check_device_ptrs({q, k, v, out}))) return rc;
    void* ws = nullptr;
    const size_t need = ws_layout(B, H, N, d, dtype).total;
    if ((rc = internal_ws(need, static_cast<hipStream_t>(stream), &ws))) return rc;
    return solattn_forward_ws(q, k, v, out, B, H, N, d, prefix_len, tau, mode, dtype, ws, need,
                              stream);
}

int solattn_forward_noalloc(const void* q, const void* k, const void* v, void* out, int64_t B,
                            int64_t H, int64_t N, int64_t d, int64_t prefix_len, float tau,
                            int mode, int dtype, void* stream) {
    int rc = validate(q, k, v, out, true, B, H, N, d, prefix_len, tau, mode, dtype);
    if (rc) return rc;
    const size_t need = ws_layout(B, H, N, d, dtype).total;
    if (need > (size_t)SOLATTN_NOALLOC_SCRATCH_BYTES)
        return fail(SOLATTN_EUNSUPPORTED,
                    "this shape needs %zu bytes of workspace; solattn_forward_noalloc holds %zu "
                    "(use solattn_forward_ws)",
                    need, (size_t)SOLATTN_NOALLOC_SCRATCH_BYTES);
    if ((rc = check_device_ptrs({q, k, v, out}))) return rc;
    void* ws = nullptr;
    if ((rc = scratch_ptr(&ws))) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = run_prepare(q, k, v, B, H, N, d, mode, dtype, ws, s, true))) return rc;
    return run_attend(q, k, v, out, B, H, N, d, prefix_len, tau, mode, dtype, ws, s, nullptr,
                      nullptr, nullptr, 0);
}

int solattn_prepare_ws(const void* q, const void* k, const void* v, int64_t B, int64_t H,
                       int64_t N, int64_t d, int mode, int dtype, void* ws, size_t ws_bytes,
                       void* stream) {
    int rc = validate(q, k, v, nullptr, false, B, H, N, d, 0, 0.f, mode, dtype);
    if (rc) return rc;
    if ((rc = check_ws(ws, ws_bytes, B, H, N, d, dtype))) return rc;
    if ((rc = check_device_ptrs({q, k, v, ws}))) return rc;
    return run_prepare(q, k, v, B, H, N, d, mode, dtype, ws, static_cast<hipStream_t>(stream), true);
}

int solattn_attend_ws(const void* q, const void* k, const void* v, void* out, int64_t B,
                      int64_t H, int64_t N, int64_t d, int64_t prefix_len, float tau, int mode,
                      int dtype, void* ws, size_t ws_bytes, void* stream) {
    // the bf16 attention reads keys and values from the workspace only
    int rc = validate(q, k, v, out, true, B, H, N, d, prefix_len, tau, mode, dtype,
                      dtype == SOLATTN_BF16);
    if (rc) return rc;
    if ((rc = check_ws(ws, ws_bytes, B, H, N, d, dtype))) return rc;
    if ((rc = check_device_ptrs({q, k, v, out, ws}))) return rc;
    return run_attend(q, k, v, out, B, H, N, d, prefix_len, tau, mode, dtype, ws,
                      static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr, 0);
}

int solattn_plan_ws(const void* q, int64_t B, int64_t H, int64_t N, int64_t d,
                    int64_t prefix_len, float tau, int mode, int dtype, void* ws, size_t ws_bytes,
                    void* stream) {
    // q stands in for k and v in the checks (the routing reads q and ws)
    int rc = validate(q, q, q, nullptr, false, B, H, N, d, prefix_len, tau, mode, dtype);
    if (rc) return rc;
    if ((mode & SOLATTN_MODE_MASK) == SOLATTN_TOPK && !(tau > 0.f && tau <= 1.f))
        return fail(SOLATTN_EINVAL, "topk mode: tau is the kept fraction, in (0, 1] (got %g)",
                    (double)tau);
    if (!plannable(mode, dtype))
        return fail(SOLATTN_EUNSUPPORTED, "a routing plan is built for bf16 SPARSE or TOPK "
                                          "without SOLATTN_TAYLOR1 only");
    if ((rc = check_ws(ws, ws_bytes, B, H, N, d, dtype))) return rc;
    if ((rc = check_device_ptrs({q, ws}))) return rc;
    return run_attend(q, q, q, nullptr, B, H, N, d, prefix_len, tau, mode, dtype, ws,
                      static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr, kStagePlan);
}

int solattn_attend_plan_ws(const void* q, void* out, int64_t B, int64_t H, int64_t N, int64_t d,
                           int mode, int dtype, void* ws, size_t ws_bytes, void* stream) {
    // keys and values come from the workspace tiles; the routing from the
    // plan (prefix length and tau are in the keep bits already)
    int rc = validate(q, q, q, out, true, B, H, N, d, 0, 1.f, mode, dtype);
    if (rc) return rc;
    if (!plannable(mode, dtype))
        return fail(SOLATTN_EUNSUPPORTED, "a routing plan is built for bf16 SPARSE or TOPK "
                                          "without SOLATTN_TAYLOR1 only");
    if ((rc = check_ws(ws, ws_bytes, B, H, N, d, dtype))) return rc;
    if ((rc = check_device_ptrs({q, out, ws}))) return rc;
    return run_attend(q, nullptr, nullptr, out, B, H, N, d, 0, 1.f, mode, dtype, ws,
                      static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr,
                      kStageAttendPlan);
}

int solattn_forward_debug(const void* q, const void* k, const void* v, void* out, int64_t B,
                          int64_t H, int64_t N, int64_t d, int64_t prefix_len, float tau,
                          int mode, int dtype, uint32_t* mask_out, float* score_out,
                          float* thr_out, void* stream) {
    int rc = validate(q, k, v, out, true, B, H, N, d, prefix_len, tau, mode, dtype);
    if (rc) return rc;
    if ((rc = reject_capture(static_cast<hipStream_t>(stream)))) return rc;
    if ((rc = check_device_ptrs({q, k, v, out, mask_out, score_out, thr_out}))) return rc;
    void* ws = nullptr;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = internal_ws(ws_layout(B, H, N, d, dtype).total, s, &ws))) return rc;
    if ((rc = run_prepare(q, k, v, B, H, N, d, mode, dtype, ws, s, true))) return rc;
    return run_attend(q, k, v, out, B, H, N, d, prefix_len, tau, mode, dtype, ws, s, mask_out,
                      score_out, thr_out, 0);
}

int solattn_pool(const void* q, const void* k, const void* v, float* qbar, float* kbar,
                 float* vbar, int64_t B, int64_t H, int64_t N, int64_t d, int dtype,
                 void* stream) {
    int rc = validate(q, k, v, nullptr, false, B, H, N, d, 0, 0.f, SOLATTN_SPARSE, dtype);
    if (rc) return rc;
    if ((rc = reject_capture(static_cast<hipStream_t>(stream)))) return rc;
    if ((rc = check_device_ptrs({q, k, v, qbar, kbar, vbar}))) return rc;
    void* ws = nullptr;
    const WsLayout L = ws_layout(B, H, N, d, dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = internal_ws(L.total, s, &ws))) return rc;
    if ((rc = run_prepare(q, k, v, B, H, N, d, SOLATTN_SPARSE, dtype, ws, s, false, true)))
        return rc;
    const size_t bytes = sizeof(float) * B * H * ((N + 63) / 64) * d;
    const struct { float* dst; size_t off; } outs[3] = {{qbar, L.qbar}, {kbar, L.kbar}, {vbar, L.vbar}};
    for (const auto& o : outs) {
        if (!o.dst) continue;
        hipError_t e = hipMemcpyAsync(o.dst, at(ws, o.off), bytes, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    }
    return SOLATTN_OK;
}

int solattn_route(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t N,
                  int64_t d, int64_t prefix_len, float tau, int dtype, uint32_t* mask_out,
                  float* score_out, float* thr_out, void* stream) {
    int rc = validate(q, k, v, nullptr, false, B, H, N, d, prefix_len, tau, SOLATTN_SPARSE, dtype);
    if (rc) return rc;
    if ((rc = reject_capture(static_cast<hipStream_t>(stream)))) return rc;
    if ((rc = check_device_ptrs({q, k, v, mask_out, score_out, thr_out}))) return rc;
    void* ws = nullptr;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = internal_ws(ws_layout(B, H, N, d, dtype).total, s, &ws))) return rc;
    if ((rc = run_prepare(q, k, v, B, H, N, d, SOLATTN_SPARSE, dtype, ws, s, false))) return rc;
    return run_attend(q, k, v, nullptr, B, H, N, d, prefix_len, tau, SOLATTN_SPARSE, dtype, ws, s,
                      mask_out, score_out, thr_out, kStageRouteOnly);
}

int solattn_route_ws(const void* q, int64_t B, int64_t H, int64_t N, int64_t d,
                     int64_t prefix_len, float tau, int dtype, const void* ws, size_t ws_bytes,
                     uint32_t* mask_out, float* score_out, float* thr_out, void* stream) {
    // reads the pooled key means in ws and the query means: for fp32 from ws,
    // for bf16 formed from the query rows of q; q stands in for k and v in
    // the checks
    int rc = validate(q, q, q, nullptr, false, B, H, N, d, prefix_len, tau, SOLATTN_SPARSE, dtype);
    if (rc) return rc;
    if ((rc = check_ws(const_cast<void*>(ws), ws_bytes, B, H, N, d, dtype))) return rc;
    if ((rc = check_device_ptrs({q, ws, mask_out, score_out, thr_out}))) return rc;
    return run_attend(q, q, q, nullptr, B, H, N, d, prefix_len, tau, SOLATTN_SPARSE, dtype,
                      const_cast<void*>(ws), static_cast<hipStream_t>(stream), mask_out, score_out,
                      thr_out, kStageRouteOnly);
}

const char* solattn_strerror(int code) {
    switch (code) {
        case SOLATTN_OK: return "ok";
        case SOLATTN_EINVAL: return "invalid argument";
        case SOLATTN_EUNSUPPORTED: return "unsupported configuration";
        case SOLATTN_EHIP: return "HIP runtime error";
        case SOLATTN_ENOMEM: return "out of device memory";
        default: return "unknown error code";
    }
}

const char* solattn_last_error(void) { return g_last_error.c_str(); }

int solattn_probe_mfma_bf16(float* sink, int64_t waves, int64_t iters, void* stream) {
    g_last_error.clear();
    if (!sink) return fail(SOLATTN_EINVAL, "sink must be non-NULL");
    if (!aligned16(sink)) return fail(SOLATTN_EINVAL, "sink must be 16-byte aligned");
    if (waves < 1 || waves > (1LL << 20))
        return fail(SOLATTN_EINVAL, "waves must be in [1, 2^20] (got %lld)", (long long)waves);
    if (iters < 1 || iters > (1LL << 20))
        return fail(SOLATTN_EINVAL, "iters must be in [1, 2^20] (got %lld)", (long long)iters);
    if (int rc = check_device_ptrs({sink})) return rc;
    const hipError_t e = launch_probe_mfma(sink, waves, iters, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "probe launch");
    return SOLATTN_OK;
}

size_t solattn_transport_record_bytes(int64_t d) {
    return (d == 64 || d == 128) ? (size_t)((d + 4 + 15) / 16 * 16) : 0;
}

int solattn_pack_qkv_int8(const void* q, const void* k, const void* v, int64_t B, int64_t H,
                          int64_t Ns, int64_t d, int64_t P, void* send, void* stream) {
    g_last_error.clear();
    int rc = check_transport(B, H, Ns, d, P);
    if (rc) return rc;
    if (H % P) return fail(SOLATTN_EINVAL, "H (%lld) must be a multiple of P (%lld)", (long long)H,
                           (long long)P);
    const size_t tb = (size_t)B * H * Ns * d * 2, sb = (size_t)B * H * Ns * 3 *
                                                         solattn_transport_record_bytes(d);
    if ((rc = check_buffers({q, k, v}, tb, {send}, sb))) return rc;
    if ((rc = check_device_ptrs({q, k, v, send}))) return rc;
    QkvPackArgs a{q, k, v, static_cast<uint8_t*>(send), B, H, H / P, Ns, P};
    const hipError_t e = launch_pack_qkv_int8(a, (int)d, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOLATTN_OK : hip_fail(e, "pack kernel launch");
}

int solattn_unpack_qkv_int8(const void* recv, int64_t B, int64_t Hp, int64_t Ns, int64_t d,
                            int64_t P, void* q, void* k, void* v, void* stream) {
    g_last_error.clear();
    int rc = check_transport(B, Hp, Ns, d, P);
    if (rc) return rc;
    const size_t rb = (size_t)P * B * Hp * Ns * 3 * solattn_transport_record_bytes(d),
                 tb = (size_t)B * Hp * P * Ns * d * 2;
    if ((rc = check_buffers({recv}, rb, {q, k, v}, tb))) return rc;
    if ((rc = check_device_ptrs({recv, q, k, v}))) return rc;
    QkvUnpackArgs a{static_cast<const uint8_t*>(recv), q, k, v, B, Hp, Ns, P};
    const hipError_t e = launch_unpack_qkv_int8(a, (int)d, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOLATTN_OK : hip_fail(e, "unpack kernel launch");
}

int solattn_prepare_int8_ws(const void* recv, int64_t B, int64_t Hp, int64_t Ns, int64_t d,
                            int64_t P, int mode, void* q_out, void* ws, size_t ws_bytes,
                            void* stream) {
    g_last_error.clear();
    int rc = check_transport(B, Hp, Ns, d, P);
    if (rc) return rc;
    const int64_t N = P * Ns;
    // shapes, mode and alignment as for solattn_prepare_ws on the unpacked
    // tensors (q_out stands in for q, k and v)
    if ((rc = validate(q_out, q_out, q_out, nullptr, false, B, Hp, N, d, 0, 0.f, mode,
                       SOLATTN_BF16)))
        return rc;
    if (B * Hp > 65535)
        return fail(SOLATTN_EUNSUPPORTED, "B*Hp = %lld exceeds 65535 slices", (long long)(B * Hp));
    if ((rc = check_ws(ws, ws_bytes, B, Hp, N, d, SOLATTN_BF16))) return rc;
    const size_t rb = (size_t)P * B * Hp * Ns * 3 * solattn_transport_record_bytes(d),
                 tb = (size_t)B * Hp * N * d * 2;
    if ((rc = check_buffers({recv}, rb, {q_out}, tb))) return rc;
    if (overlaps(ws, ws_bytes, recv, rb) || overlaps(ws, ws_bytes, q_out, tb))
        return fail(SOLATTN_EINVAL, "ws must not overlap recv or q_out");
    if ((rc = check_device_ptrs({recv, q_out, ws}))) return rc;
    const PoolArgs p = pool_args(nullptr, nullptr, nullptr, B, Hp, N, d, mode, SOLATTN_BF16, ws,
                                 true);
    UnpackPoolArgs u{static_cast<const uint8_t*>(recv), q_out, B, Hp, Ns, P};
    const hipError_t e = launch_unpack_pool(p, u, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOLATTN_OK : hip_fail(e, "unpack-pool kernel launch");
}

int solattn_pack_out_fp8(const void* o, int64_t B, int64_t Hp, int64_t Ns, int64_t d, int64_t P,
                         void* send, void* stream) {
    g_last_error.clear();
    int rc = check_transport(B, Hp, Ns, d, P);
    if (rc) return rc;
    const size_t tb = (size_t)B * Hp * P * Ns * d * 2,
                 sb = (size_t)P * B * Hp * Ns * solattn_transport_record_bytes(d);
    if ((rc = check_buffers({o}, tb, {send}, sb))) return rc;
    if ((rc = check_device_ptrs({o, send}))) return rc;
    OutPackArgs a{o, static_cast<uint8_t*>(send), B, Hp, Ns, P};
    const hipError_t e = launch_pack_out_fp8(a, (int)d, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOLATTN_OK : hip_fail(e, "pack kernel launch");
}

int solattn_unpack_out_fp8(const void* recv, int64_t B, int64_t Hp, int64_t Ns, int64_t d,
                           int64_t P, void* o, void* stream) {
    g_last_error.clear();
    int rc = check_transport(B, Hp, Ns, d, P);
    if (rc) return rc;
    const size_t rb = (size_t)P * B * Hp * Ns * solattn_transport_record_bytes(d),
                 tb = (size_t)B * P * Hp * Ns * d * 2;
    if ((rc = check_buffers({recv}, rb, {o}, tb))) return rc;
    if ((rc = check_device_ptrs({recv, o}))) return rc;
    OutUnpackArgs a{static_cast<const uint8_t*>(recv), o, B, Hp, Ns, P};
    const hipError_t e = launch_unpack_out_fp8(a, (int)d, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOLATTN_OK : hip_fail(e, "unpack kernel launch");
}

const char* solattn_version(void) { return "solattn-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
