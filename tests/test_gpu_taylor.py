"""GPU parity of the first-order (Taylor) mode, SOLATTN_TAYLOR1, against the
oracle (oracle/taylor.py, explicit d x d cross-covariances in fp64).  Masks
are held to the C oracle's routing as in the other parity tests; outputs to
the Taylor oracle recomputed with the GPU's mask (bf16 bar: 2e-2 absolute).
Also on the GPU: constant key blocks leave the sparse result unchanged, and
on blocks whose keys sit eps from their mean the first-order mode is far
closer to dense attention than the zeroth-order one."""
import numpy as np
import pytest

import oracle
from oracle import taylor as OT
from block_sparse_video_solattn_amd import inputs
from gpu_util import TOL_BF16_ABS, device_tensors, mask_compare, max_abs_diff

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(q, k, v, prefix, tau, mode="sparse+taylor1"):
    import torch
    import block_sparse_video_solattn_amd as sa
    qd, kd, vd = device_tensors(q, k, v, "bf16")
    out, words, _, _ = sa.solattn_forward_debug(qd, kd, vd, None, prefix, tau, mode,
                                                want_scores=False)
    torch.cuda.synchronize()
    nb = (q.shape[2] + 63) // 64
    return out.float().cpu().numpy().astype(np.float64), sa.unpack_mask(words, nb)


@pytest.mark.parametrize("B,H,N,d,prefix,tau,kind", [
    (1, 2, 1000, 128, 64, 1.0, "iid_qk_offset"),    # ragged tail of 40 keys
    (2, 1, 64 * 9 + 5, 64, 0, 0.5, "iid_qk_offset"),  # tail of 5, B > 1, d = 64
    (1, 2, 2000, 128, 128, 1.25, "field"),
    (1, 1, 700, 128, 0, float("inf"), "iid_qk_offset"),     # every block skipped
    (1, 1, 700, 64, 0, float("-inf"), "iid_qk_offset"),     # none skipped: dense
])
def test_taylor_matches_oracle(B, H, N, d, prefix, tau, kind):
    grid = (2, 24, 40) if kind == "field" else None
    q, k, v = inputs.custom(B, H, N, d, "bf16", prefix_len=prefix, seed=N + 7, kind=kind,
                            grid=grid)
    g, gmask = _run(q, k, v, prefix, tau)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            ro = oracle.head(q[b, h], k[b, h], v[b, h], prefix, tau, want_out=False)
            mask_compare(gmask, ro, b, h)
            r = OT.head(q[b, h], k[b, h], v[b, h], prefix, tau, order=1,
                        mask_override=gmask[b, h])
            worst = max(worst, max_abs_diff(g[b, h], r["out"]))
    assert worst <= TOL_BF16_ABS, worst


def test_constant_key_blocks_leave_sparse_unchanged():
    q, k, v = inputs.custom(1, 2, 640, 128, "bf16", prefix_len=64, seed=91)
    for j in range(0, 640, 64):
        k[:, :, j:j + 64] = k[:, :, j:j + 1]
    g1, m1 = _run(q, k, v, 64, 0.5)
    g0, m0 = _run(q, k, v, 64, 0.5, mode="sparse")
    assert np.array_equal(m1, m0) and (~m1).any()
    assert np.abs(g1 - g0).max() <= 2e-3


def test_first_order_is_closer_to_dense():
    # keys = block base + eps * D (D of zero block mean): the mask does not
    # depend on eps and the skipped blocks' expansion is accurate
    rng = np.random.default_rng(92)
    N, d, nb = 64 * 16, 128, 16
    q = rng.standard_normal((1, 2, N, d))
    base = np.repeat(rng.standard_normal((1, 2, nb, d)) * 1.5, 64, axis=2)
    D = rng.standard_normal((1, 2, N, d))
    D -= np.repeat(D.reshape(1, 2, nb, 64, d).mean(3), 64, axis=2)
    v = rng.standard_normal((1, 2, N, d))
    k = base + 0.1 * D
    q, k, v = (inputs.round_to_bf16(x.astype(np.float32)) for x in (q, k, v))
    g1, m = _run(q, k, v, 0, 0.5)
    g0, _ = _run(q, k, v, 0, 0.5, mode="sparse")
    gd, _ = _run(q, k, v, 0, 0.0, mode="dense")
    assert (~m).mean() > 0.3
    e0, e1 = np.abs(g0 - gd).max(), np.abs(g1 - gd).max()
    assert e1 < e0 / 4, (e0, e1)


def test_refine_shape_sampled():
    # the refine workload at tau = 1.25: masks of two heads against the C
    # oracle, sampled query blocks' outputs against the Taylor oracle
    w = inputs.WORKLOADS["refine"]
    heads = [0, 31]
    q, k, v = inputs.make_inputs(w, 3000, heads=heads)
    g, gmask = _run(q, k, v, w.prefix_len, 1.25)
    blocks = [0, 5, 100, w.nb - 1]
    rows = np.concatenate([np.arange(64 * i, min(w.N, 64 * i + 64)) for i in blocks])
    for hi in range(len(heads)):
        ro = oracle.head(q[0, hi], k[0, hi], v[0, hi], w.prefix_len, 1.25, want_out=False)
        mask_compare(gmask, ro, 0, hi)
        r = OT.head(q[0, hi], k[0, hi], v[0, hi], w.prefix_len, 1.25, order=1,
                    mask_override=gmask[0, hi], rows=rows)
        assert np.abs(g[0, hi, rows] - r["out"]).max() <= TOL_BF16_ABS


@pytest.mark.parametrize("flags,omode", [("+video_stats", oracle.SPARSE | oracle.VIDEO_STATS),
                                         ("+prefix_rows", oracle.SPARSE | oracle.PREFIX_ROWS)])
def test_taylor_with_routing_variants(flags, omode):
    q, k, v = inputs.custom(1, 2, 1500, 128, "bf16", prefix_len=192, seed=93, kind="field",
                            grid=(2, 24, 28))
    g, gmask = _run(q, k, v, 192, 1.0, mode="sparse" + flags + "+taylor1")
    for h in range(2):
        ro = oracle.head(q[0, h], k[0, h], v[0, h], 192, 1.0, mode=omode, want_out=False)
        mask_compare(gmask, ro, 0, h)
        r = OT.head(q[0, h], k[0, h], v[0, h], 192, 1.0, order=1, mask_override=gmask[0, h],
                    mode=omode)
        assert np.abs(g[0, h] - r["out"]).max() <= TOL_BF16_ABS
