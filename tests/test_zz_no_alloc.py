"""solattn_forward_noalloc, the entry point for callers that cannot
allocate (graph capture, serving loops, harnesses that forbid hipMalloc):
through the C ABI it must give what solattn_forward_ws gives on the same
inputs -- the same kernels run, so bit for bit -- on two calls in a row, the
second with a smaller input (the fixed device workspace keeps the first
call's contents), also when recorded into a HIP graph and replayed, and it
must reject a shape whose workspace exceeds its fixed size on the host."""
import numpy as np
import pytest

from block_sparse_video_solattn_amd import inputs
from gpu_util import device_tensors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(B, H, N, d, dtype, seed, prefix=128):
    grid = (max(1, -(-(N - prefix) // (24 * 42))), 24, 42)
    q, k, v = inputs.custom(B, H, N, d, dtype, prefix_len=prefix, seed=seed, kind="field",
                            grid=grid)
    return device_tensors(q, k, v, dtype)


def _ws_ref(sa, qd, kd, vd, prefix, tau, mode):
    import torch
    B, H, N, d = qd.shape
    ws = torch.empty(sa.solattn_workspace_bytes(B, H, N, d, qd.dtype), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(qd)
    sa.solattn_forward_ws(qd, kd, vd, out, prefix, tau, mode, ws)
    return out


@pytest.mark.parametrize("dtype,mode,tau", [("bf16", "sparse", 1.25), ("bf16", "dense", 0.0),
                                            ("bf16", "topk", 0.2), ("f32", "sparse", 1.0)])
def test_matches_ws_entry_point_twice_shrinking(dtype, mode, tau):
    import torch
    import block_sparse_video_solattn_amd as sa
    big = (1, 4, 3000, 128) if dtype == "bf16" else (1, 2, 1500, 64)
    small = (1, 2, 700, 128) if dtype == "bf16" else (1, 1, 300, 64)
    for n, shape in enumerate((big, small)):
        qd, kd, vd = _case(*shape, dtype, seed=91 + n)
        ref = _ws_ref(sa, qd, kd, vd, 128, tau, mode)
        out = torch.full_like(qd, float("nan"))
        sa.solattn_forward_noalloc(qd, kd, vd, out, 128, tau, mode)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        assert torch.equal(out, ref), (shape, mode)


def test_at_the_size_limit_and_beyond():
    import torch
    import block_sparse_video_solattn_amd as sa
    # one GPU's share of an 8-way head-sharded refine step fits ...
    B, H, N, d = 1, 4, 16384, 128
    assert sa.solattn_workspace_bytes(B, H, N, d, torch.bfloat16) <= sa.NOALLOC_SCRATCH_BYTES
    qd, kd, vd = _case(B, H, N, d, "bf16", seed=95, prefix=256)
    ref = _ws_ref(sa, qd, kd, vd, 256, 1.25, "sparse")
    out = torch.empty_like(qd)
    sa.solattn_forward_noalloc(qd, kd, vd, out, 256, 1.25, "sparse")
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    # ... a whole refine step does not: rejected on the host, nothing enqueued
    big = torch.empty((1, 32, 16384, 128), dtype=torch.bfloat16, device="cuda")
    ob = torch.empty_like(big)
    with pytest.raises(sa.SolAttnError) as e:
        sa.solattn_forward_noalloc(big, big, big, ob, 256, 1.25, "sparse")
    assert e.value.code == sa.EUNSUPPORTED and "workspace" in str(e.value)


def test_graph_capture_and_replay():
    import torch
    import block_sparse_video_solattn_amd as sa
    qd, kd, vd = _case(1, 2, 2000, 128, "bf16", seed=96)
    out = torch.empty_like(qd)
    sa.solattn_forward_noalloc(qd, kd, vd, out, 128, 1.25, "sparse")  # resolves the address
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sa.solattn_forward_noalloc(qd, kd, vd, out, 128, 1.25, "sparse")
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float(rep + 1))
        # another call on a different input between replays leaves its own
        # contents in the shared workspace
        q2, k2, v2 = _case(1, 1, 900, 128, "bf16", seed=97 + rep)
        o2 = torch.empty_like(q2)
        sa.solattn_forward_noalloc(q2, k2, v2, o2, 128, 1.0, "sparse")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
