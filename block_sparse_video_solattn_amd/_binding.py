"""Thin ctypes binding over libsolattn.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  Tensors are torch device tensors (used for device
memory and streams); shapes are read from q, which must be contiguous
[B, H, N, d].  A missing library raises at import time; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsolattn.so")

OK, EINVAL, EUNSUPPORTED, EHIP, ENOMEM = 0, 1, 2, 3, 4
DENSE, SPARSE, TOPK = 0, 1, 2
PREFIX_ROWS, VIDEO_STATS = 0x10, 0x20  # routing variant flags, OR-ed into the mode
TAYLOR1 = 0x40                          # first-order correction of skipped blocks (sparse, bf16)
F32, BF16 = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libsolattn.so is not built (expected at %s); run "
        "`python -m block_sparse_video_solattn_amd.build`" % LIB_PATH)

# Load torch first when it is present: the library then binds to the HIP
# runtime torch already mapped instead of pulling in a second copy, which
# could not share device state with torch's allocations and streams.
try:
    import torch  # noqa: F401
except ImportError:  # pragma: no cover - torch is the expected host
    torch = None

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGS = {
    "solattn_forward": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _I, _I, _P], _I),
    "solattn_workspace_bytes": ([_I64, _I64, _I64, _I64, _I], _SZ),
    "solattn_forward_noalloc": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _I, _I, _P], _I),
    "solattn_forward_ws": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _I, _I, _P, _SZ, _P], _I),
    "solattn_prepare_ws": ([_P, _P, _P, _I64, _I64, _I64, _I64, _I, _I, _P, _SZ, _P], _I),
    "solattn_attend_ws": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _I, _I, _P, _SZ, _P], _I),
    "solattn_plan_ws": ([_P, _I64, _I64, _I64, _I64, _I64, _F, _I, _I, _P, _SZ, _P], _I),
    "solattn_attend_plan_ws": ([_P, _P, _I64, _I64, _I64, _I64, _I, _I, _P, _SZ, _P], _I),
    "solattn_forward_debug": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _I, _I, _P, _P, _P, _P], _I),
    "solattn_pool": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I, _P], _I),
    "solattn_route": ([_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _I, _P, _P, _P, _P], _I),
    "solattn_route_ws": ([_P, _I64, _I64, _I64, _I64, _I64, _F, _I, _P, _SZ, _P, _P, _P, _P], _I),
    "solattn_probe_mfma_bf16": ([_P, _I64, _I64, _P], _I),
    "solattn_transport_record_bytes": ([_I64], _SZ),
    "solattn_pack_qkv_int8": ([_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P], _I),
    "solattn_unpack_qkv_int8": ([_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P], _I),
    "solattn_prepare_int8_ws": ([_P, _I64, _I64, _I64, _I64, _I64, _I, _P, _P, _SZ, _P], _I),
    "solattn_pack_out_fp8": ([_P, _I64, _I64, _I64, _I64, _I64, _P, _P], _I),
    "solattn_unpack_out_fp8": ([_P, _I64, _I64, _I64, _I64, _I64, _P, _P], _I),
    "solattn_qknorm_rope": ([_P, _P, _P, _P, _F, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I,
                             _P], _I),
    "solattn_prepare_qknorm_rope_ws": ([_P, _P, _P, _P, _P, _F, _I64, _P, _P, _P, _P, _I64, _I64,
                                        _I64, _I64, _I, _I, _P, _SZ, _P], _I),
    "solattn_strerror": ([_I], ctypes.c_char_p),
    "solattn_last_error": ([], ctypes.c_char_p),
    "solattn_version": ([], ctypes.c_char_p),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTS = tuple(_SIGS)


class SolAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("solattn error %d (%s): %s" % (code, solattn_strerror(code), msg))
        self.code = code


def solattn_strerror(code: int) -> str:
    return _lib.solattn_strerror(int(code)).decode()


def solattn_last_error() -> str:
    return _lib.solattn_last_error().decode()


def solattn_version() -> str:
    return _lib.solattn_version().decode()


def _check(rc: int):
    if rc != OK:
        raise SolAttnError(rc, solattn_last_error())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _dtype_code(t) -> int:
    """Element type code of a tensor or a torch.dtype."""
    import torch
    dt = t if isinstance(t, torch.dtype) else t.dtype
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float32:
        return F32
    raise TypeError("q/k/v must be float32 or bfloat16, got %s" % dt)


def _mode_code(mode) -> int:
    """"dense", "sparse", "topk", optionally followed by "+prefix_rows",
    "+video_stats" and/or "+taylor1" (e.g. "sparse+video_stats"), or the
    integer code."""
    if isinstance(mode, str):
        parts = mode.split("+")
        code = {"dense": DENSE, "sparse": SPARSE, "topk": TOPK}[parts[0]]
        for f in parts[1:]:
            code |= {"prefix_rows": PREFIX_ROWS, "video_stats": VIDEO_STATS, "taylor1": TAYLOR1}[f]
        return code
    return int(mode)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _on_gpu(t, name):
    """Every tensor handed to the library must live in GPU memory: a host
    pointer reaching a kernel would fault the device."""
    if not getattr(t, "is_cuda", False):
        raise ValueError("%s must be a GPU tensor (got device %s)" % (name, getattr(t, "device", "?")))


def _shape(q):
    _on_gpu(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    for t in (q,):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return tuple(int(x) for x in q.shape)


def _check_like(q, *ts):
    for t in ts:
        if t is None:
            continue
        _on_gpu(t, "k, v and out")
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError("q, k, v, out must share shape, dtype, device and be contiguous")


def _same_device(q, t, name):
    """Workspaces, exports and tables: a GPU tensor on q's device, contiguous."""
    if t is None:
        return
    _on_gpu(t, name)
    if t.device != q.device or not t.is_contiguous():
        raise ValueError("%s must be contiguous and on %s" % (name, q.device))


def _ws_bytes(q, ws):
    _same_device(q, ws, "ws")
    return ws.numel() * ws.element_size()


def solattn_workspace_bytes(B: int, H: int, N: int, d: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(_lib.solattn_workspace_bytes(B, H, N, d, code))


def solattn_forward(q, k, v, out=None, prefix_len: int = 0, tau: float = 1.0, mode="sparse",
                    stream=None):
    """out = Sol-Attn(q, k, v); returns out (allocated when not given)."""
    B, H, N, d = _shape(q)
    if out is None:
        out = q.new_empty(q.shape)
    _check_like(q, k, v, out)
    _check(_lib.solattn_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d, prefix_len,
                                float(tau), _mode_code(mode), _dtype_code(q), _stream(stream)))
    return out


def solattn_forward_noalloc(q, k, v, out, prefix_len: int, tau: float, mode="sparse",
                            stream=None):
    """solattn_forward with the library's fixed device workspace (no
    allocation in the call; shapes beyond SOLATTN_NOALLOC_SCRATCH_BYTES of
    workspace are rejected).  Calls that overlap on one GPU race."""
    B, H, N, d = _shape(q)
    _check_like(q, k, v, out)
    _check(_lib.solattn_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d,
                                        prefix_len, float(tau), _mode_code(mode),
                                        _dtype_code(q), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def solattn_forward_ws(q, k, v, out, prefix_len, tau, mode, ws, stream=None):
    B, H, N, d = _shape(q)
    _check_like(q, k, v, out)
    _check(_lib.solattn_forward_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d, prefix_len,
                                   float(tau), _mode_code(mode), _dtype_code(q), _ptr(ws),
                                   _ws_bytes(q, ws), _stream(stream)))
    return out


def solattn_prepare_ws(q, k, v, mode, ws, stream=None):
    B, H, N, d = _shape(q)
    _check_like(q, k, v)
    _check(_lib.solattn_prepare_ws(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, _mode_code(mode),
                                   _dtype_code(q), _ptr(ws), _ws_bytes(q, ws),
                                   _stream(stream)))


def solattn_attend_ws(q, k, v, out, prefix_len, tau, mode, ws, stream=None):
    B, H, N, d = _shape(q)
    _check_like(q, k, v, out)
    _check(_lib.solattn_attend_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d, prefix_len,
                                  float(tau), _mode_code(mode), _dtype_code(q), _ptr(ws),
                                  _ws_bytes(q, ws), _stream(stream)))
    return out


def solattn_plan_ws(q, prefix_len, tau, mode, ws, stream=None):
    """Routing plan (keep bits, tile counts, dispatch order) into ws, which
    solattn_prepare_ws filled for q's shape (bf16 sparse / topk)."""
    B, H, N, d = _shape(q)
    _check(_lib.solattn_plan_ws(_ptr(q), B, H, N, d, prefix_len, float(tau), _mode_code(mode),
                                _dtype_code(q), _ptr(ws), _ws_bytes(q, ws), _stream(stream)))


def solattn_attend_plan_ws(q, out, mode, ws, stream=None):
    """Attention in the order and with the routing solattn_plan_ws left in ws."""
    B, H, N, d = _shape(q)
    _check_like(q, out)
    _check(_lib.solattn_attend_plan_ws(_ptr(q), _ptr(out), B, H, N, d, _mode_code(mode),
                                       _dtype_code(q), _ptr(ws), _ws_bytes(q, ws),
                                       _stream(stream)))
    return out


def solattn_forward_debug(q, k, v, out=None, prefix_len: int = 0, tau: float = 1.0,
                          mode="sparse", stream=None, want_scores: bool = True):
    """Forward plus the routing exports.  Returns (out, mask_words, scores, thr)."""
    import torch
    B, H, N, d = _shape(q)
    nb = (N + 63) // 64
    if out is None:
        out = q.new_empty(q.shape)
    _check_like(q, k, v, out)
    mask = torch.zeros((B, H, nb, (nb + 31) // 32), dtype=torch.int32, device=q.device)
    scores = (torch.full((B, H, nb, nb), float("nan"), dtype=torch.float32, device=q.device)
              if want_scores else None)
    thr = torch.full((B, H, nb), float("nan"), dtype=torch.float32, device=q.device)
    _check(_lib.solattn_forward_debug(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d,
                                      prefix_len, float(tau), _mode_code(mode), _dtype_code(q),
                                      _ptr(mask), _ptr(scores), _ptr(thr), _stream(stream)))
    return out, mask, scores, thr


def solattn_pool(q, k, v, stream=None):
    """Block means (fp32 [B, H, Nb, d]) of q, k, v."""
    import torch
    B, H, N, d = _shape(q)
    _check_like(q, k, v)
    nb = (N + 63) // 64
    outs = [torch.empty((B, H, nb, d), dtype=torch.float32, device=q.device) for _ in range(3)]
    _check(_lib.solattn_pool(_ptr(q), _ptr(k), _ptr(v), _ptr(outs[0]), _ptr(outs[1]),
                             _ptr(outs[2]), B, H, N, d, _dtype_code(q), _stream(stream)))
    return tuple(outs)


def solattn_route(q, k, v, prefix_len: int, tau: float, stream=None, want_scores: bool = True,
                  mask=None, scores=None, thr=None):
    """Pooling + routing only.  Returns (mask_words, scores, thr)."""
    import torch
    B, H, N, d = _shape(q)
    _check_like(q, k, v)
    nb = (N + 63) // 64
    if mask is None:
        mask = torch.zeros((B, H, nb, (nb + 31) // 32), dtype=torch.int32, device=q.device)
    if scores is None and want_scores:
        scores = torch.full((B, H, nb, nb), float("nan"), dtype=torch.float32, device=q.device)
    if thr is None:
        thr = torch.full((B, H, nb), float("nan"), dtype=torch.float32, device=q.device)
    for t, name in ((mask, "mask"), (scores, "scores"), (thr, "thr")):
        _same_device(q, t, name)
    _check(_lib.solattn_route(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, prefix_len, float(tau),
                              _dtype_code(q), _ptr(mask), _ptr(scores), _ptr(thr), _stream(stream)))
    return mask, scores, thr


def solattn_route_ws(q, prefix_len: int, tau: float, ws, mask=None, scores=None, thr=None,
                     stream=None):
    """The scoring / threshold pass alone on a workspace solattn_prepare_ws
    filled (sparse mode) for q's shape; writes the given exports (any None)."""
    B, H, N, d = _shape(q)
    for t, name in ((mask, "mask"), (scores, "scores"), (thr, "thr")):
        _same_device(q, t, name)
    _check(_lib.solattn_route_ws(_ptr(q), B, H, N, d, prefix_len, float(tau), _dtype_code(q),
                                 _ptr(ws), _ws_bytes(q, ws), _ptr(mask), _ptr(scores), _ptr(thr),
                                 _stream(stream)))
    return mask, scores, thr


def solattn_probe_mfma_bf16(sink, waves: int, iters: int, stream=None):
    """Enqueue the bf16 MFMA peak probe (waves * iters * 16 * 32768 FLOP);
    sink: float32 device tensor of at least waves * 64 elements."""
    _on_gpu(sink, "sink")
    if sink.numel() < waves * 64:
        raise ValueError("sink needs waves * 64 floats")
    _check(_lib.solattn_probe_mfma_bf16(_ptr(sink), int(waves), int(iters), _stream(stream)))


def raw_call(name: str, *args) -> int:
    """Call an exported C function with raw integer/float arguments (for
    argument-validation tests)."""
    return getattr(_lib, name)(*args)


def unpack_mask(words, nb: int):
    """[..., ceil(nb/32)] int32 words -> [..., nb] bool keep mask (host numpy)."""
    import numpy as np
    w = words.cpu().numpy().astype(np.uint32) if hasattr(words, "cpu") else np.asarray(words, np.uint32)
    bits = (w[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(w.shape[:-1] + (-1,))[..., :nb].astype(bool)


def isinf_tau(tau: float) -> bool:
    return math.isinf(tau)


# ------------------------------------------------------- sequence-parallel transport
def solattn_transport_record_bytes(d: int) -> int:
    return int(_lib.solattn_transport_record_bytes(int(d)))


def _bf16_4d(t, name):
    import torch
    _on_gpu(t, name)
    if t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous():
        raise ValueError("%s must be a contiguous 4-d bfloat16 tensor" % name)
    return tuple(t.shape)


def solattn_pack_qkv_int8(q, k, v, P: int, send=None, stream=None):
    """This rank's sequence shard q, k, v [B][H][Ns][d] -> INT8 records
    [P][B][H/P][Ns][3][rec] (uint8), chunk p for rank p."""
    import torch
    B, H, Ns, d = _bf16_4d(q, "q")
    if _bf16_4d(k, "k") != (B, H, Ns, d) or _bf16_4d(v, "v") != (B, H, Ns, d):
        raise ValueError("q, k, v shapes differ")
    rec = solattn_transport_record_bytes(d)
    if send is None:
        send = torch.empty((P, B, H // max(P, 1), Ns, 3, rec), dtype=torch.uint8, device=q.device)
    _same_device(q, send, "send")
    _check(_lib.solattn_pack_qkv_int8(_ptr(q), _ptr(k), _ptr(v), B, H, Ns, d, int(P), _ptr(send),
                                      _stream(stream)))
    return send


def solattn_unpack_qkv_int8(recv, d: int, q=None, k=None, v=None, stream=None):
    """Received records [P][B][Hp][Ns][3][rec] -> q, k, v [B][Hp][P*Ns][d] bf16."""
    import torch
    _on_gpu(recv, "recv")
    P, B, Hp, Ns = (int(x) for x in recv.shape[:4])
    shape = (B, Hp, P * Ns, d)
    q = torch.empty(shape, dtype=torch.bfloat16, device=recv.device) if q is None else q
    k = torch.empty(shape, dtype=torch.bfloat16, device=recv.device) if k is None else k
    v = torch.empty(shape, dtype=torch.bfloat16, device=recv.device) if v is None else v
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _same_device(recv, t, name)
    _check(_lib.solattn_unpack_qkv_int8(_ptr(recv), B, Hp, Ns, int(d), P, _ptr(q), _ptr(k), _ptr(v),
                                        _stream(stream)))
    return q, k, v


def solattn_prepare_int8_ws(recv, d: int, mode, ws, q_out=None, stream=None):
    """Received INT8 records [P][B][Hp][Ns][3][rec] -> q_out [B][Hp][P*Ns][d]
    bf16 and the workspace of the unpacked Q/K/V (dequantize + pool in one
    pass).  Returns q_out."""
    import torch
    _on_gpu(recv, "recv")
    P, B, Hp, Ns = (int(x) for x in recv.shape[:4])
    if q_out is None:
        q_out = torch.empty((B, Hp, P * Ns, d), dtype=torch.bfloat16, device=recv.device)
    _same_device(recv, q_out, "q_out")
    _same_device(recv, ws, "ws")
    _check(_lib.solattn_prepare_int8_ws(_ptr(recv), B, Hp, Ns, int(d), P, _mode_code(mode),
                                        _ptr(q_out), _ptr(ws), ws.numel() * ws.element_size(),
                                        _stream(stream)))
    return q_out


def solattn_pack_out_fp8(o, P: int, send=None, stream=None):
    """Output of this rank's heads o [B][Hp][P*Ns][d] -> FP8 records
    [P][B][Hp][Ns][rec] (uint8), chunk r for rank r."""
    import torch
    B, Hp, N, d = _bf16_4d(o, "o")
    if N % P:
        raise ValueError("the sequence length must be a multiple of P")
    Ns = N // P
    if send is None:
        send = torch.empty((P, B, Hp, Ns, solattn_transport_record_bytes(d)), dtype=torch.uint8,
                           device=o.device)
    _same_device(o, send, "send")
    _check(_lib.solattn_pack_out_fp8(_ptr(o), B, Hp, Ns, d, int(P), _ptr(send), _stream(stream)))
    return send


def solattn_unpack_out_fp8(recv, d: int, o=None, stream=None):
    """Received records [P][B][Hp][Ns][rec] -> o [B][P*Hp][Ns][d] bf16."""
    import torch
    _on_gpu(recv, "recv")
    P, B, Hp, Ns = (int(x) for x in recv.shape[:4])
    if o is None:
        o = torch.empty((B, P * Hp, Ns, d), dtype=torch.bfloat16, device=recv.device)
    _same_device(recv, o, "o")
    _check(_lib.solattn_unpack_out_fp8(_ptr(recv), B, Hp, Ns, int(d), P, _ptr(o), _stream(stream)))
    return o


# ------------------------------------------------------------ fused Q/K producer
def _f32_vec(t, n, name):
    import torch
    if t is None:
        return None
    _on_gpu(t, name)
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
        raise ValueError("%s must be a contiguous float32 tensor of %d elements" % (name, n))
    return t


def _producer_ptrs(q, gamma_q, gamma_k, rope_dim, rope_cos, rope_sin):
    B, H, N, d = _shape(q)
    _f32_vec(gamma_q, d, "gamma_q")
    _f32_vec(gamma_k, d, "gamma_k")
    if rope_dim > 0:
        _f32_vec(rope_cos, N * (rope_dim // 2), "rope_cos")
        _f32_vec(rope_sin, N * (rope_dim // 2), "rope_sin")
    for t, name in ((gamma_q, "gamma_q"), (gamma_k, "gamma_k"), (rope_cos, "rope_cos"),
                    (rope_sin, "rope_sin")):
        if t is not None and (rope_dim > 0 or name.startswith("gamma")):
            _same_device(q, t, name)
    return B, H, N, d


def solattn_qknorm_rope(q, k, gamma_q, gamma_k, eps: float, rope_dim: int, rope_cos=None,
                        rope_sin=None, q_out=None, k_out=None, stream=None):
    """q', k' = partial RoPE of the RMS-normalised q, k (the producer alone).
    gamma_*: float32 [d] or None (ones); rope_cos / rope_sin: float32 [N, rope_dim/2]."""
    B, H, N, d = _producer_ptrs(q, gamma_q, gamma_k, rope_dim, rope_cos, rope_sin)
    q_out = q.new_empty(q.shape) if q_out is None else q_out
    k_out = q.new_empty(q.shape) if k_out is None else k_out
    _check_like(q, k, q_out, k_out)
    _check(_lib.solattn_qknorm_rope(_ptr(q), _ptr(k), _ptr(gamma_q), _ptr(gamma_k), float(eps),
                                    int(rope_dim), _ptr(rope_cos), _ptr(rope_sin), _ptr(q_out),
                                    _ptr(k_out), B, H, N, d, _dtype_code(q), _stream(stream)))
    return q_out, k_out


def solattn_prepare_qknorm_rope_ws(q, k, v, gamma_q, gamma_k, eps: float, rope_dim: int,
                                   rope_cos, rope_sin, mode, ws, q_out=None, k_out=None,
                                   want_k_out: bool = True, stream=None):
    """The producer fused with pooling: writes q' (and k' unless want_k_out
    is False and no k_out is given; bf16 only) and fills ws as
    solattn_prepare_ws(q', k', v) would.  Returns (q_out, k_out or None)."""
    B, H, N, d = _producer_ptrs(q, gamma_q, gamma_k, rope_dim, rope_cos, rope_sin)
    q_out = q.new_empty(q.shape) if q_out is None else q_out
    if k_out is None and want_k_out:
        k_out = q.new_empty(q.shape)
    _check_like(q, k, v, q_out, k_out)
    _check(_lib.solattn_prepare_qknorm_rope_ws(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gamma_q), _ptr(gamma_k), float(eps), int(rope_dim),
        _ptr(rope_cos), _ptr(rope_sin), _ptr(q_out), _ptr(k_out), B, H, N, d, _mode_code(mode),
        _dtype_code(q), _ptr(ws), _ws_bytes(q, ws), _stream(stream)))
    return q_out, k_out
