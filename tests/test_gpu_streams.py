"""The C ABI on streams other than the default one, concurrently on two
streams, and captured into a HIP graph: the workspace entry points allocate
nothing and enqueue only kernels on the caller's stream, so each of these
must reproduce the default-stream result bit for bit (the kernels are
deterministic).  The plain entry points keep one internal workspace per
(device, stream): concurrent plain calls on two streams must also reproduce
their single-stream results, and under graph capture they refuse to run."""
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


def _case(seed, N=3000, H=4):
    grid = (-(-(N - 128) // (24 * 60)), 24, 60)
    q, k, v = inputs.custom(1, H, N, 128, "bf16", prefix_len=128, seed=seed, kind="field",
                            grid=grid)
    return device_tensors(q, k, v, "bf16")


def _ws(sa, q):
    import torch
    B, H, N, d = q.shape
    return torch.empty(sa.solattn_workspace_bytes(B, H, N, d, q.dtype), dtype=torch.uint8,
                       device="cuda")


def test_side_stream_matches_default_stream():
    import torch
    import block_sparse_video_solattn_amd as sa
    qd, kd, vd = _case(81)
    ref = sa.solattn_forward(qd, kd, vd, None, 128, 1.25, "sparse")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()          # default priority
    ws = _ws(sa, qd)
    out = torch.empty_like(qd)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sa.solattn_forward_ws(qd, kd, vd, out, 128, 1.25, "sparse", ws)
    side.synchronize()
    assert torch.equal(out, ref)


def test_two_streams_concurrently():
    import torch
    import block_sparse_video_solattn_amd as sa
    cases = [_case(82), _case(83, N=2000)]
    refs = [sa.solattn_forward(*c, None, 128, 1.25, "sparse").clone() for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [_ws(sa, c[0]) for c in cases]
    outs = [torch.empty_like(c[0]) for c in cases]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for c, s, ws, o in zip(cases, streams, wss, outs):
            with torch.cuda.stream(s):
                sa.solattn_prepare_ws(*c, "sparse", ws)
                sa.solattn_attend_ws(*c, o, 128, 1.25, "sparse", ws)
    for s in streams:
        s.synchronize()
    for o, r in zip(outs, refs):
        assert torch.equal(o, r)


def test_graph_capture_and_replay():
    import torch
    import block_sparse_video_solattn_amd as sa
    qd, kd, vd = _case(84)
    ws = _ws(sa, qd)
    out = torch.empty_like(qd)
    # eager result on the same buffers
    sa.solattn_prepare_ws(qd, kd, vd, "sparse", ws)
    sa.solattn_attend_ws(qd, kd, vd, out, 128, 1.25, "sparse", ws)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sa.solattn_prepare_ws(qd, kd, vd, "sparse", ws)
            sa.solattn_attend_ws(qd, kd, vd, out, 128, 1.25, "sparse", ws)
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between replays: scribble over the output and the workspace
        out.fill_(float(rep + 1))
        ws.fill_(rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
    # the captured launches read the inputs at replay time: new inputs, new output
    q2, k2, v2 = _case(85)
    qd.copy_(q2)
    kd.copy_(k2)
    vd.copy_(v2)
    g.replay()
    ref2 = sa.solattn_forward(q2, k2, v2, None, 128, 1.25, "sparse")
    torch.cuda.synchronize()
    assert torch.equal(out, ref2)
    assert not torch.equal(out, eager)


def test_fused_producer_on_a_side_stream():
    import torch
    import block_sparse_video_solattn_amd as sa
    d = inputs.producer_inputs(1, 2, 1500, 128, "bf16", prefix_len=100, grid=(2, 20, 35), seed=86)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(d[n])).cuda().to(torch.bfloat16)
               for n in ("q", "k", "v"))
    gq, gk, cs, sn = (torch.from_numpy(d[n]).cuda().contiguous()
                      for n in ("gamma_q", "gamma_k", "cos", "sin"))
    ws0, ws1 = _ws(sa, q).zero_(), _ws(sa, q).zero_()   # (alignment gaps stay zero)
    q0, _ = sa.solattn_prepare_qknorm_rope_ws(q, k, v, gq, gk, 1e-6, 64, cs, sn, "sparse", ws0,
                                              want_k_out=False)
    o0 = torch.empty_like(q)
    sa.solattn_attend_ws(q0, None, None, o0, 100, 1.25, "sparse", ws0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q1, _ = sa.solattn_prepare_qknorm_rope_ws(q, k, v, gq, gk, 1e-6, 64, cs, sn, "sparse",
                                                  ws1, want_k_out=False)
        o1 = torch.empty_like(q)
        sa.solattn_attend_ws(q1, None, None, o1, 100, 1.25, "sparse", ws1)
    side.synchronize()
    assert torch.equal(q1, q0) and torch.equal(o1, o0)
    assert torch.equal(ws1, ws0)


def test_plain_forward_on_two_streams_concurrently():
    import torch
    import block_sparse_video_solattn_amd as sa
    cases = [_case(87, N=6000, H=8), _case(88, N=2500, H=8)]
    refs = [sa.solattn_forward(*c, None, 128, 1.25, "sparse").clone() for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full_like(c[0], float("nan")) for c in cases]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(4):
        for c, s, o in zip(cases, streams, outs):
            with torch.cuda.stream(s):
                sa.solattn_forward(*c, o, 128, 1.25, "sparse")
    for s in streams:
        s.synchronize()
    for o, r in zip(outs, refs):
        assert torch.equal(o, r)
    # the routing exports of the plain debug entry point, also on two streams
    dbg = [None, None]
    for n, (c, s) in enumerate(zip(cases, streams)):
        with torch.cuda.stream(s):
            dbg[n] = sa.solattn_forward_debug(*c, None, 128, 1.25, "sparse")
    for s in streams:
        s.synchronize()
    for (o, words, sc, th), r in zip(dbg, refs):
        assert torch.equal(o, r)


def test_plain_entry_points_refuse_capture():
    import torch
    import block_sparse_video_solattn_amd as sa
    qd, kd, vd = _case(89)
    out = torch.empty_like(qd)
    x = torch.zeros(16, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    codes = []
    calls = (lambda: sa.solattn_forward(qd, kd, vd, out, 128, 1.25, "sparse"),
             lambda: sa.solattn_pool(qd, kd, vd),
             lambda: sa.solattn_route(qd, kd, vd, 128, 1.25, want_scores=False))
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for call in calls:
                try:
                    call()
                except sa.SolAttnError as e:
                    codes.append(e.code)
            x.add_(1)
    torch.cuda.synchronize()
    assert codes == [sa.EUNSUPPORTED] * len(calls)
    g.replay()
    torch.cuda.synchronize()
    assert bool(x.eq(1).all())
