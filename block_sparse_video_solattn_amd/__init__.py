"""Sol-Attn block-sparse video attention for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library libsolattn.so (C ABI in include/solattn.h);
this package re-exports its thin Python binding on first use.  Using it without
the built library raises ImportError: there is no CPU fallback.  The input
generators in ``.inputs`` need no library.
"""
_BINDING_NAMES = (
    "BF16", "DENSE", "EXPORTS", "F32", "PREFIX_ROWS", "SPARSE", "TAYLOR1", "TOPK", "VIDEO_STATS",
    "OK", "EINVAL", "EUNSUPPORTED", "EHIP", "ENOMEM", "NOALLOC_SCRATCH_BYTES",
    "SolAttnError", "solattn_attend_ws", "solattn_forward_noalloc", "solattn_plan_ws",
    "solattn_attend_plan_ws",
    "solattn_forward", "solattn_forward_debug", "solattn_forward_ws", "solattn_last_error",
    "solattn_pool", "solattn_prepare_ws", "solattn_probe_mfma_bf16", "solattn_route", "solattn_route_ws",
    "solattn_strerror",
    "solattn_version", "solattn_workspace_bytes", "unpack_mask", "raw_call",
    "solattn_transport_record_bytes", "solattn_pack_qkv_int8", "solattn_unpack_qkv_int8",
    "solattn_pack_out_fp8", "solattn_unpack_out_fp8", "solattn_prepare_int8_ws",
    "solattn_qknorm_rope", "solattn_prepare_qknorm_rope_ws",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
