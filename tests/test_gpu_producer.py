"""GPU parity of the fused Q/K producer (QKNorm then partial RoPE) against the
oracle (oracle/producer.py), and of its pooling epilogue against the plain
pooling pass: the fused call must leave the workspace, q' and k' bit for bit
as the producer alone followed by solattn_prepare_ws does.

Bars: bf16 -- every element within half a bf16 step of the exact value plus
the fp32 arithmetic's error (2e-6 of the row's RMS, which covers the
cancellation inside a rotated pair), and at most 0.2 % of the elements off
the exact value's own rounding (a rounding decision can only flip when the
exact value lies within the fp32 error of a midpoint); fp32 -- 1e-5 of
(|exact| + the row's RMS)."""
import numpy as np
import pytest

from oracle import producer as P
from block_sparse_video_solattn_amd import inputs as I

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(x, dtype):
    import torch
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(td).contiguous()


def dev_f32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda").contiguous()


def tables(inp, misalign):
    """Device rotary tables; `misalign` offsets them by one float (4-byte
    aligned only), which takes the kernel's element-wise table path."""
    import torch
    out = []
    for name in ("cos", "sin"):
        t = inp[name].reshape(-1)
        if misalign:
            buf = torch.zeros(t.size + 4, dtype=torch.float32, device="cuda")
            buf[1:1 + t.size] = torch.from_numpy(t).cuda()
            out.append(buf[1:1 + t.size])
        else:
            out.append(dev_f32(t))
    return out


def check_against_oracle(got, exact, dtype):
    """got: float64 GPU values; exact: the oracle's float64 result."""
    rms = np.sqrt(np.mean(exact * exact, axis=-1, keepdims=True))
    if dtype == "bf16":
        ax = np.abs(exact)
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
        half_step = np.where(ax > 0, 2.0 ** (e - 8), 0.0)
        err = np.abs(got - exact)
        bad = err > half_step + 2e-6 * rms
        assert not bad.any(), (np.argwhere(bad)[:5].tolist(), got[bad][:5], exact[bad][:5])
        flips = np.mean(got != P.round_bf16(exact))
        assert flips <= 2e-3, flips
    else:
        bad = np.abs(got - exact) > 1e-5 * (np.abs(exact) + rms)
        assert not bad.any(), (np.argwhere(bad)[:5].tolist(), got[bad][:5], exact[bad][:5])


CASES = [
    # dtype, B, H, N, d, rope_dim, prefix, grid, gamma, misaligned tables
    ("bf16", 1, 3, 1000, 128, 64, 40, (2, 20, 24), True, False),    # ragged tail of 40 rows
    ("bf16", 2, 2, 300, 64, 64, 0, (3, 10, 10), True, False),       # full rotation, B > 1
    ("bf16", 1, 2, 130, 128, 0, 2, (2, 8, 8), True, False),         # no rotation
    ("bf16", 1, 1, 200, 128, 128, 8, (2, 8, 12), False, False),     # full rotation, weights NULL
    ("bf16", 1, 2, 64 * 5, 128, 64, 64, (1, 16, 16), True, True),   # element-wise table reads
    ("bf16", 1, 1, 77, 128, 36, 13, (1, 8, 8), True, False),        # 18 pairs: partial chunks
    ("bf16", 1, 1, 1, 64, 64, 0, (1, 1, 1), True, False),           # a single token
    ("f32", 1, 2, 333, 128, 64, 21, (2, 12, 13), True, False),
    ("f32", 1, 2, 100, 64, 6, 4, (1, 8, 12), True, False),          # 3 pairs over 2-pair chunks
    ("f32", 1, 1, 64, 64, 64, 0, (1, 8, 8), True, True),
]


def _run_alone(c, seed):
    import torch
    import block_sparse_video_solattn_amd as sa
    dtype, B, H, N, d, r, prefix, grid, use_g, mis = c
    inp = I.producer_inputs(B, H, N, d, dtype, prefix_len=prefix, grid=grid, rope_dim=r,
                            seed=seed)
    gq = dev_f32(inp["gamma_q"]) if use_g else None
    gk = dev_f32(inp["gamma_k"]) if use_g else None
    cos, sin = tables(inp, mis) if r else (None, None)
    qo, ko = sa.solattn_qknorm_rope(dev(inp["q"], dtype), dev(inp["k"], dtype), gq, gk, EPS, r,
                                    cos, sin)
    torch.cuda.synchronize()
    return inp, qo.double().cpu().numpy(), ko.double().cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}H{c[2]}N{c[3]}d{c[4]}r{c[5]}"
                                             + ("-mis" if c[9] else "") + ("" if c[8] else "-nog")
                                             for c in CASES])
def test_producer_matches_oracle(case):
    dtype, r, use_g = case[0], case[5], case[8]
    inp, qo, ko = _run_alone(case, seed=21)
    tab = (inp["cos"], inp["sin"]) if r else (None, None)
    for got, x, g in ((qo, inp["q"], inp["gamma_q"]), (ko, inp["k"], inp["gamma_k"])):
        exact = P.qknorm_rope(x, g if use_g else None, EPS, *tab)
        check_against_oracle(got, exact, dtype)


def test_eps_dominates_small_rows():
    # rows of magnitude ~1e-4: mean square 1e-8 against eps 1e-6, so eps sets the scale
    import torch
    import block_sparse_video_solattn_amd as sa
    rng = np.random.default_rng(7)
    N, d = 256, 128
    x = I.round_to_bf16((rng.standard_normal((1, 2, N, d)) * 1e-4).astype(np.float32))
    g = (1 + 0.2 * rng.standard_normal(d)).astype(np.float32)
    qo, ko = sa.solattn_qknorm_rope(dev(x, "bf16"), dev(x, "bf16"), dev_f32(g), None, EPS, 0)
    torch.cuda.synchronize()
    check_against_oracle(qo.double().cpu().numpy(), P.qknorm_rope(x, g, EPS), "bf16")
    check_against_oracle(ko.double().cpu().numpy(), P.qknorm_rope(x, None, EPS), "bf16")
    assert float(qo.abs().max()) < 1.5     # eps-free rows would have unit RMS, peaks near 5


def _fused_vs_unfused(dtype, B, H, N, d, r, prefix, grid, mode, seed, want_k=True):
    import torch
    import block_sparse_video_solattn_amd as sa
    inp = I.producer_inputs(B, H, N, d, dtype, prefix_len=prefix, grid=grid, rope_dim=r,
                            seed=seed)
    q, k, v = (dev(inp[n], dtype) for n in ("q", "k", "v"))
    gq, gk = dev_f32(inp["gamma_q"]), dev_f32(inp["gamma_k"])
    cos, sin = (dev_f32(inp["cos"]), dev_f32(inp["sin"])) if r else (None, None)
    nbytes = sa.solattn_workspace_bytes(B, H, N, d, q.dtype)
    ws1 = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ws2 = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    q1, k1 = sa.solattn_prepare_qknorm_rope_ws(q, k, v, gq, gk, EPS, r, cos, sin, mode, ws1,
                                               want_k_out=want_k)
    q2, k2 = sa.solattn_qknorm_rope(q, k, gq, gk, EPS, r, cos, sin)
    sa.solattn_prepare_ws(q2, k2, v, mode, ws2)
    torch.cuda.synchronize()
    assert torch.equal(q1.view(torch.int16) if dtype == "bf16" else q1.view(torch.int32),
                       q2.view(torch.int16) if dtype == "bf16" else q2.view(torch.int32))
    if want_k:
        assert torch.equal(k1.view(torch.uint8), k2.view(torch.uint8))
    else:
        assert k1 is None
    diff = (ws1 != ws2).nonzero()
    assert diff.numel() == 0, diff[:8].flatten().tolist()
    return inp, q1, k1, v, ws1, q2, k2


@pytest.mark.parametrize("dtype,B,H,N,d,r,prefix,grid,mode", [
    ("bf16", 1, 3, 1000, 128, 64, 40, (2, 20, 24), "sparse"),
    ("bf16", 2, 2, 64 * 65 + 7, 64, 64, 64, (3, 33, 42), "sparse"),   # pooled padding, > 64 blocks
    ("bf16", 1, 2, 700, 128, 64, 100, (2, 20, 15), "dense"),
    ("bf16", 1, 2, 700, 128, 64, 100, (2, 20, 15), "topk"),
    ("f32", 1, 2, 333, 128, 64, 21, (2, 12, 13), "sparse"),
    ("f32", 1, 2, 333, 64, 64, 21, (2, 12, 13), "dense"),
])
def test_fused_prepare_equals_producer_then_prepare(dtype, B, H, N, d, r, prefix, grid, mode):
    import torch
    import block_sparse_video_solattn_amd as sa
    inp, q1, k1, v, ws1, q2, k2 = _fused_vs_unfused(dtype, B, H, N, d, r, prefix, grid, mode,
                                                    seed=31)
    # the attention on the fused workspace equals the whole forward on q', k'
    tau = 0.2 if mode == "topk" else 1.25
    out1 = torch.empty_like(q1)
    if dtype == "bf16":
        sa.solattn_attend_ws(q1, None, None, out1, prefix, tau, mode, ws1)
    else:
        sa.solattn_attend_ws(q1, k1, v, out1, prefix, tau, mode, ws1)
    out2 = sa.solattn_forward(q2, k2, v, None, prefix, tau, mode)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


def test_fused_prepare_without_k_out():
    _fused_vs_unfused("bf16", 1, 2, 1000, 128, 64, 40, (2, 20, 24), "sparse", seed=41,
                      want_k=False)


def test_fp32_fused_needs_k_out():
    import torch
    import block_sparse_video_solattn_amd as sa
    q = torch.zeros((1, 1, 64, 64), dtype=torch.float32, device="cuda")
    ws = torch.zeros(sa.solattn_workspace_bytes(1, 1, 64, 64, q.dtype), dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(sa.SolAttnError):
        sa.solattn_prepare_qknorm_rope_ws(q, q, q, None, None, EPS, 0, None, None, "sparse", ws,
                                          want_k_out=False)


def test_refine_shape_sampled():
    # the bench workload's shape (B=1, H=32, N=16384, d=128, half the channels
    # rotated): producer rows of sampled heads against the oracle, and the
    # fused workspace against the unfused one in full
    w = I.WORKLOADS["refine"]
    inp, q1, k1, v, ws1, q2, k2 = _fused_vs_unfused("bf16", w.B, w.H, w.N, w.D, w.D // 2,
                                                    w.prefix_len, w.grid, "sparse", seed=51)
    for h in (0, 17, 31):
        rows = np.r_[0:70, w.N - 70:w.N]
        for got, x, g in ((q1, inp["q"], inp["gamma_q"]), (k1, inp["k"], inp["gamma_k"])):
            gv = got[0, h, rows].double().cpu().numpy()
            exact = P.qknorm_rope(x[0, h, rows], g, EPS, inp["cos"][rows], inp["sin"][rows])
            check_against_oracle(gv, exact, "bf16")
