"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
seeded inputs, plus the invariants the method guarantees, at sizes the oracle
finishes in seconds (several tiles and a ragged tail)."""
import math

import numpy as np
import pytest

import oracle
from block_sparse_video_solattn_amd import inputs
from gpu_util import (POOLED_GATE, TOL_BF16_ABS, TOL_F32_REL, block_rows, device_tensors,
                      gpu_debug, mask_compare, out_error, pooled_gate)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_video_solattn_amd  # noqa: F401  (raises when the library is missing)


def check_forward(q, k, v, dtype, prefix, tau, mode="sparse", rows_blocks=None):
    """GPU forward vs oracle recomputed with the GPU's mask; returns stats."""
    B, H, N, d = q.shape
    gout, gmask, gs, gthr = gpu_debug(q, k, v, dtype, prefix, tau, mode)
    parts = mode.split("+")
    omode = {"sparse": oracle.SPARSE, "dense": oracle.DENSE, "topk": oracle.TOPK}[parts[0]]
    for f in parts[1:]:
        omode |= {"prefix_rows": oracle.PREFIX_ROWS, "video_stats": oracle.VIDEO_STATS}[f]
    otau = float(np.float32(tau))  # the value the C ABI received
    n_diff = n_near = 0
    worst = 0.0
    for b in range(B):
        for h in range(H):
            ores = oracle.head(q[b, h], k[b, h], v[b, h], prefix, otau, mode=omode,
                               want_out=False)
            if mode != "dense":
                nd, nn = mask_compare(gmask, ores, b, h)
                n_diff += nd
                n_near += nn
                fin = np.isfinite(ores["score"])
                assert np.max(np.abs(gs[b, h][fin] - ores["score"][fin])) < 1e-4
                # the same infinite thresholds (tau = +-inf, rows with no video
                # block, prefix rows of the PREFIX_ROWS variant), the finite
                # ones within the score tolerance
                fin_t = np.isfinite(ores["thr"])
                assert np.array_equal(np.isfinite(gthr[b, h]), fin_t)
                assert np.array_equal(gthr[b, h][~fin_t], ores["thr"][~fin_t])
                assert np.max(np.abs(gthr[b, h][fin_t] - ores["thr"][fin_t]), initial=0) < 1e-4
            else:
                assert gmask[b, h].all()
            r = oracle.head(q[b, h], k[b, h], v[b, h], prefix, otau, mode=omode,
                            mask_override=gmask[b, h].astype(np.uint8), qblocks=rows_blocks)
            rows = None if rows_blocks is None else block_rows(rows_blocks, N)
            ab, rel = out_error(gout[b, h], r["out"], rows)
            worst = max(worst, rel if dtype == "f32" else ab)
    if dtype == "f32":
        assert worst <= TOL_F32_REL, worst
    else:
        assert worst <= TOL_BF16_ABS, worst
    return dict(worst=worst, n_diff=n_diff, n_near=n_near, mask=gmask, out=gout)


# ------------------------------------------------------------------ pooling
@pytest.mark.parametrize("dtype,N,d", [("f32", 1024, 64), ("bf16", 1000, 128), ("bf16", 37, 64),
                                       ("f32", 4100, 128)])
def test_pool_parity(dtype, N, d):
    import torch
    import block_sparse_video_solattn_amd as sa
    q, k, v = inputs.custom(1, 2, N, d, dtype, seed=11)
    qd, kd, vd = device_tensors(q, k, v, dtype)
    qb, kb, vb = sa.solattn_pool(qd, kd, vd)
    torch.cuda.synchronize()
    for h in range(2):
        r = oracle.head(q[0, h], k[0, h], v[0, h], 0, 1.0, want_out=False)
        for name, g in (("qbar", qb), ("kbar", kb), ("vbar", vb)):
            ref = r[name]
            err = np.max(np.abs(g[0, h].cpu().numpy() - ref)) / np.max(np.abs(ref))
            assert err < 1e-6, (name, err)


# ------------------------------------------------------------------ workloads
def test_tiny_workload_f32():
    w = inputs.WORKLOADS["tiny"]
    q, k, v = inputs.make_inputs(w, 1000)
    st = check_forward(q, k, v, "f32", w.prefix_len, 1.0)
    m = st["mask"][0, 0]
    assert m[:, :2].all() and 0 < m.mean() < 1


def test_tiny_workload_constant_key_block():
    w = inputs.WORKLOADS["tiny"]
    q, k, v = inputs.make_inputs(w, 1001, const_key_block=9)
    check_forward(q, k, v, "f32", w.prefix_len, 1.0)


@pytest.mark.parametrize("tau", [-math.inf, math.inf])
def test_tiny_workload_tau_limits(tau):
    w = inputs.WORKLOADS["tiny"]
    q, k, v = inputs.make_inputs(w, 1002)
    st = check_forward(q, k, v, "f32", w.prefix_len, tau)
    m = st["mask"][0, 0]
    if tau < 0:
        assert m.all()
    else:
        assert m[:, :2].all() and not m[:, 2:].any()


def test_small_workload_bf16():
    w = inputs.WORKLOADS["small"]
    q, k, v = inputs.make_inputs(w, 2000)
    st = check_forward(q, k, v, "bf16", w.prefix_len, 1.25)
    m = st["mask"]
    assert m[..., :4].all()
    assert 0.02 < 1 - m[..., 4:].mean() < 0.99


def test_dense_mode_bf16_and_f32():
    for dtype, d in (("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)):
        q, k, v = inputs.custom(1, 2, 700, d, dtype, seed=21)
        check_forward(q, k, v, dtype, 0, 0.0, mode="dense")


# ------------------------------------------------------------------ edges
@pytest.mark.parametrize("dtype,B,H,N,d,prefix,tau", [
    ("bf16", 1, 1, 37, 128, 0, 1.0),        # one partial block
    ("bf16", 1, 1, 64, 64, 64, 1.0),        # one full block, all prefix
    ("bf16", 2, 3, 1000, 128, 100, 0.5),    # ragged tail of 40 keys, B > 1
    ("bf16", 1, 2, 64 * 9 + 20, 128, 0, 1.0),  # tail of 20 keys (one half tile)
    ("bf16", 1, 1, 64 * 70 + 33, 64, 512, 1.5),  # tail of 33 keys, > 64 blocks
    ("f32", 1, 2, 64 * 9 + 20, 128, 0, 1.0),
    ("f32", 2, 1, 300, 64, 300, 2.0),       # prefix = N
    ("bf16", 1, 1, 64 * 130, 128, 0, math.inf),  # nothing kept: pooled terms only
    ("bf16", 1, 1, 64 * 130, 128, 128, math.inf),
    ("bf16", 1, 1, 64 * 130, 128, 0, -math.inf),
])
def test_edge_shapes(dtype, B, H, N, d, prefix, tau):
    q, k, v = inputs.custom(B, H, N, d, dtype, prefix_len=prefix, seed=N + H)
    check_forward(q, k, v, dtype, prefix, tau)


def test_field_inputs_bf16_d64():
    q, k, v = inputs.custom(1, 2, 5000, 64, "bf16", prefix_len=256, seed=5, kind="field",
                            grid=(4, 24, 50))
    check_forward(q, k, v, "bf16", 256, 1.25)


# ------------------------------------------------------------------ invariants
def test_tau_minus_inf_matches_dense():
    import torch
    import block_sparse_video_solattn_amd as sa
    q, k, v = inputs.custom(1, 2, 2000, 128, "bf16", seed=31)
    qd, kd, vd = device_tensors(q, k, v, "bf16")
    a = sa.solattn_forward(qd, kd, vd, None, 128, -math.inf, "sparse")
    b = sa.solattn_forward(qd, kd, vd, None, 128, 0.0, "dense")
    torch.cuda.synchronize()
    assert (a.float() - b.float()).abs().max().item() <= 1e-2


def test_constant_values_give_ones():
    import torch
    import block_sparse_video_solattn_amd as sa
    q, k, _ = inputs.custom(1, 2, 1500, 128, "bf16", seed=32)
    v = np.ones_like(q)
    qd, kd, vd = device_tensors(q, k, v, "bf16")
    for tau in (-math.inf, 0.5, 1.25, math.inf):
        o = sa.solattn_forward(qd, kd, vd, None, 64, tau, "sparse")
        torch.cuda.synchronize()
        assert (o.float() - 1).abs().max().item() <= 1e-2


def test_all_blocks_constant_tau_inf_equals_dense():
    # every key block constant: each pooled term equals its exact block, so
    # pooled-only routing (tau = +inf, no prefix) reproduces dense attention;
    # both GPU paths are held against the fp64 dense result
    import torch
    import block_sparse_video_solattn_amd as sa
    for dtype, N in (("f32", 1000), ("bf16", 2000)):
        q, k, v = inputs.custom(1, 2, N, 128, dtype, seed=33)
        # multiples of 1/16: block sums of 64 equal rows are exact in fp32, so
        # the pooled key/value equals the row and only summation order remains
        k = np.round(k * 16) / 16
        v = np.round(v * 16) / 16
        for j in range((N + 63) // 64):
            k[:, :, 64 * j:64 * j + 64] = k[:, :, 64 * j:64 * j + 1]
            v[:, :, 64 * j:64 * j + 64] = v[:, :, 64 * j:64 * j + 1]
        qd, kd, vd = device_tensors(q, k, v, dtype)
        a = sa.solattn_forward(qd, kd, vd, None, 0, math.inf, "sparse")
        b = sa.solattn_forward(qd, kd, vd, None, 0, 0.0, "dense")
        torch.cuda.synchronize()
        for h in range(2):
            ref = oracle.head(q[0, h], k[0, h], v[0, h], 0, 0.0, mode=oracle.DENSE)["out"]
            for name, g in (("pooled-only", a), ("dense", b)):
                ab, rel = out_error(g[0, h].double().cpu().numpy(), ref)
                if dtype == "f32":
                    assert rel <= TOL_F32_REL, (name, rel)
                else:
                    assert ab <= TOL_BF16_ABS, (name, ab)


@pytest.mark.parametrize("mode", ["sparse", "dense"])
@pytest.mark.parametrize("scale", [2.5, 10.0])
def test_steep_logit_rise_after_first_block(mode, scale):
    # Logits against key block 5 exceed block 0's (the first tile) by about
    # 30 (scale 2.5) or 125..150 (scale 10) log2 units.  A softmax reference
    # fixed at the first tile's maximum handles the first; the second would
    # overflow bf16/fp32 weights (> 2^128), so the GPU must rescale there.
    q, k, v = inputs.logit_jump(1, 2, 64 * 12 + 20, 128, "bf16", jump_block=5, scale=scale, seed=41)
    check_forward(q, k, v, "bf16", 64, 1.25, mode)


def test_steep_logit_rise_f32():
    q, k, v = inputs.logit_jump(1, 1, 64 * 9 + 7, 64, "f32", jump_block=3, scale=10.0, seed=42)
    check_forward(q, k, v, "f32", 64, 1.0)


# ------------------------------------------------- fixed-ratio (TOPK) mode
@pytest.mark.parametrize("dtype,N,d,prefix,f", [
    ("bf16", 2000, 128, 128, 0.1), ("bf16", 64 * 9 + 20, 64, 0, 0.25), ("f32", 1024, 64, 128, 0.3),
    ("bf16", 700, 128, 64, 1.0), ("bf16", 1500, 128, 1500, 0.1)])
def test_topk_mode(dtype, N, d, prefix, f):
    q, k, v = inputs.custom(1, 2, N, d, dtype, prefix_len=prefix, seed=51)
    st = check_forward(q, k, v, dtype, prefix, f, "topk")
    nb = (N + 63) // 64
    pb = (prefix + 63) // 64
    kk = min(nb - pb, math.ceil(float(np.float32(f)) * (nb - pb)))
    # every row keeps its prefix and (distinct scores) exactly k video blocks
    assert st["mask"][..., :pb].all()
    assert (st["mask"][..., pb:].sum(-1) == kk).all()


def test_topk_draft_fraction_field_inputs():
    # the draft stage's 90 % video sparsity on field inputs (ragged tail)
    q, k, v = inputs.custom(1, 2, 4000, 128, "bf16", prefix_len=256, seed=52, kind="field",
                            grid=(4, 24, 40))
    check_forward(q, k, v, "bf16", 256, 0.1, "topk")


def test_topk_fraction_one_matches_dense():
    import torch
    import block_sparse_video_solattn_amd as sa
    q, k, v = inputs.custom(1, 2, 1800, 128, "bf16", seed=53)
    qd, kd, vd = device_tensors(q, k, v, "bf16")
    a = sa.solattn_forward(qd, kd, vd, None, 64, 1.0, "topk")
    b = sa.solattn_forward(qd, kd, vd, None, 64, 0.0, "dense")
    torch.cuda.synchronize()
    assert (a.float() - b.float()).abs().max().item() <= 1e-2


# ------------------------------------------------------- routing variants
@pytest.mark.parametrize("mode,tau", [("sparse+prefix_rows", 1.0), ("sparse+prefix_rows", math.inf),
                                      ("sparse+video_stats", 1.25), ("topk+prefix_rows", 0.2),
                                      ("sparse+prefix_rows+video_stats", 0.75)])
@pytest.mark.parametrize("dtype,N,d", [("bf16", 64 * 20 + 17, 128), ("f32", 64 * 12 + 40, 64)])
def test_routing_variants(mode, tau, dtype, N, d):
    prefix = 150  # 3 prefix blocks, the third one partly prefix
    q, k, v = inputs.custom(1, 2, N, d, dtype, prefix_len=prefix, seed=71, kind="field",
                            grid=(2, 12, 50))
    st = check_forward(q, k, v, dtype, prefix, tau, mode)
    pb = 3
    assert st["mask"][..., :pb].all()
    if "prefix_rows" in mode:
        assert st["mask"][..., :pb, :].all()


def test_video_stats_without_video_blocks():
    # the whole sequence is prefix: every row keeps every block, thresholds +inf
    q, k, v = inputs.custom(1, 1, 700, 64, "bf16", prefix_len=700, seed=72)
    st = check_forward(q, k, v, "bf16", 700, 1.0, "sparse+video_stats")
    assert st["mask"].all()


@pytest.mark.parametrize("N,tau", [(64 * 30 + 8, math.inf), (64 * 30 + 8, 1.0),
                                   (64 * 130 + 8, 1.0), (64 * 130 + 8, math.inf)])
def test_pooled_terms_gate_ragged_tail(N, tau):
    # bf16 outputs, every row: the GPU must sit far closer to the full oracle
    # than the pooled terms move the rows (POOLED_GATE), with an 8-key tail
    # block skipped by some or all rows and one to three pooled tiles -- a
    # dropped pooled tile or the tail block weighted as a full one fails
    # here (measured with the oracle on the CPU), not only the absolute bound
    grid = (1, -(-(N - 64) // 64), 64)
    q, k, v = inputs.custom(1, 2, N, 128, "bf16", prefix_len=64, seed=N % 97 + 3, kind="field",
                            grid=grid)
    gout, gmask, _, _ = gpu_debug(q, k, v, "bf16", 64, tau)
    assert (~gmask[..., -1]).any()
    if math.isinf(tau):
        assert not gmask[..., 1:].any()
    for h in range(2):
        mo = gmask[0, h].astype(np.uint8)
        full = oracle.head(q[0, h], k[0, h], v[0, h], 64, float(np.float32(tau)),
                           mask_override=mo)["out"]
        nopool = oracle.head(q[0, h], k[0, h], v[0, h], 64, 0.5, mode=oracle.TOPK,
                             mask_override=mo)["out"]
        ab, _ = out_error(gout[0, h], full)
        sg, med = pooled_gate(gout[0, h], full, nopool)
        print("N=%d tau=%g head %d: max abs err %.3g, median pooled distance %.3g, gate %.4f"
              % (N, tau, h, ab, med, sg))
        assert ab <= TOL_BF16_ABS
        assert sg <= POOLED_GATE, sg


def test_pooled_only_path_f32():
    q, k, v = inputs.custom(1, 1, 1024, 64, "f32", seed=34)
    check_forward(q, k, v, "f32", 0, math.inf)


def test_deterministic():
    import torch
    import block_sparse_video_solattn_amd as sa
    q, k, v = inputs.custom(1, 4, 3000, 128, "bf16", prefix_len=128, seed=34)
    qd, kd, vd = device_tensors(q, k, v, "bf16")
    a = sa.solattn_forward(qd, kd, vd, None, 128, 1.0)
    b = sa.solattn_forward(qd, kd, vd, None, 128, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_workspace_entry_points_match_forward():
    import torch
    import block_sparse_video_solattn_amd as sa
    q, k, v = inputs.custom(1, 2, 2000, 128, "bf16", prefix_len=128, seed=35)
    qd, kd, vd = device_tensors(q, k, v, "bf16")
    ref = sa.solattn_forward(qd, kd, vd, None, 128, 1.0)
    nbytes = sa.solattn_workspace_bytes(1, 2, 2000, 128, sa.BF16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out1 = torch.empty_like(qd)
    sa.solattn_forward_ws(qd, kd, vd, out1, 128, 1.0, "sparse", ws)
    out2 = torch.empty_like(qd)
    sa.solattn_prepare_ws(qd, kd, vd, "sparse", ws)
    sa.solattn_attend_ws(qd, kd, vd, out2, 128, 1.0, "sparse", ws)
    torch.cuda.synchronize()
    assert torch.equal(ref, out1) and torch.equal(ref, out2)


@pytest.mark.parametrize("H,N,d,dtype", [(2, 3000, 128, "bf16"), (3, 64 * 9 + 5, 64, "f32"),
                                         (1, 64 * 4096, 128, "bf16")])
def test_route_only_matches_debug_forward(H, N, d, dtype):
    # the routing-only kernel (four query blocks per workgroup; at N = 262144
    # its LDS passes 64 KiB) gives the fused kernels' scores, thresholds and
    # masks bit for bit, also for a last group of fewer than four blocks
    import torch
    import block_sparse_video_solattn_amd as sa
    q, k, v = inputs.custom(1, H, N, d, dtype, prefix_len=128, seed=36)
    qd, kd, vd = device_tensors(q, k, v, dtype)
    _, w1, s1, t1 = sa.solattn_forward_debug(qd, kd, vd, None, 128, 1.25)
    w2, s2, t2 = sa.solattn_route(qd, kd, vd, 128, 1.25)
    # the scoring pass alone on a prepared workspace: the same exports
    ws = torch.empty(sa.solattn_workspace_bytes(1, H, N, d, qd.dtype), dtype=torch.uint8,
                     device="cuda")
    sa.solattn_prepare_ws(qd, kd, vd, "sparse", ws)
    w3, s3, t3 = (torch.zeros_like(w2), torch.full_like(s2, float("nan")),
                  torch.full_like(t2, float("nan")))
    sa.solattn_route_ws(qd, 128, 1.25, ws, w3, s3, t3)
    torch.cuda.synchronize()
    assert torch.equal(w1, w2) and torch.equal(s1, s2) and torch.equal(t1, t2)
    assert torch.equal(w3, w2) and torch.equal(s3, s2) and torch.equal(t3, t2)


def test_invalid_arguments_on_gpu_enqueue_nothing():
    import torch
    import block_sparse_video_solattn_amd as sa
    q, k, v = inputs.custom(1, 1, 128, 64, "bf16", seed=37)
    qd, kd, vd = device_tensors(q, k, v, "bf16")
    out = torch.zeros_like(qd)
    with pytest.raises(sa.SolAttnError) as e:
        sa.solattn_forward(qd, kd, vd, out, 129, 1.0)
    assert e.value.code == 1
    with pytest.raises(sa.SolAttnError):
        sa.solattn_forward(qd, kd, vd, out, 0, float("nan"))
    torch.cuda.synchronize()
    assert out.abs().max().item() == 0


def test_slices_beyond_one_grid_row():
    # more (batch, head) slices than the pooling grids' y limit (65536): the
    # pooling passes run in ranges of heads; heads on both sides of each range
    # boundary are held to the oracle (forward, pooled means, the fused
    # producer)
    import torch
    import block_sparse_video_solattn_amd as sa
    from oracle import producer as OP
    B, H, N, d = 1, 65600, 100, 64
    q, k, v = inputs.custom(B, H, N, d, "bf16", prefix_len=0, seed=77)
    qd, kd, vd = device_tensors(q, k, v, "bf16")
    out, words, scores, thr = sa.solattn_forward_debug(qd, kd, vd, None, 0, 0.5, "sparse",
                                                        want_scores=False)
    qbar, kbar, vbar = sa.solattn_pool(qd, kd, vd)
    torch.cuda.synchronize()
    heads = [0, 1, 65533, 65534, 65535, 65536, 65599]
    gmask = sa.unpack_mask(words[:, heads], 2)
    gout = out[0, heads].float().cpu().numpy().astype(np.float64)
    for n, h in enumerate(heads):
        r = oracle.head(q[0, h], k[0, h], v[0, h], 0, 0.5,
                        mask_override=gmask[0, n].astype(np.uint8))
        assert np.max(np.abs(gout[n] - r["out"])) <= TOL_BF16_ABS, h
        ro = oracle.head(q[0, h], k[0, h], v[0, h], 0, 0.5, want_out=False)
        near = np.abs(ro["score"] - ro["thr"][:, None]) <= 1e-4
        assert not ((gmask[0, n] != ro["mask"].astype(bool)) & ~near).any(), h
        for got, x in ((qbar, q), (kbar, k), (vbar, v)):
            ref = np.stack([x[0, h, :64].astype(np.float64).mean(0),
                            x[0, h, 64:].astype(np.float64).mean(0)])
            np.testing.assert_allclose(got[0, h].double().cpu().numpy(), ref, rtol=1e-6,
                                       atol=1e-6)
    del out, qbar, kbar, vbar
    # the fused producer over the same slice count (no rotation, weights NULL)
    ws = torch.empty(sa.solattn_workspace_bytes(B, H, N, d, qd.dtype), dtype=torch.uint8,
                     device="cuda")
    qo, _ = sa.solattn_prepare_qknorm_rope_ws(qd, kd, vd, None, None, 1e-6, 0, None, None,
                                              "sparse", ws, want_k_out=False)
    torch.cuda.synchronize()
    for h in heads:
        exact = OP.qknorm_rope(q[0, h], None, 1e-6)
        err = np.abs(qo[0, h].double().cpu().numpy() - exact)
        assert np.all(err <= np.abs(exact) * 2.0 ** -8 + 1e-6), h
