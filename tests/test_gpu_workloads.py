"""GPU parity at the full workload sizes (refine 16384 tokens, draft 32768,
long 48416 with a 32-token tail; 32 heads, d = 128, bf16), in the launch
configuration the benchmark times.  Keep masks are compared on every head;
outputs on sampled heads and query blocks, each recomputed by the oracle with
the GPU's mask (several masks are correct where scores sit within 1e-4 of the
threshold)."""
import json
import os

import numpy as np
import pytest

import oracle
from block_sparse_video_solattn_amd import inputs
from gpu_util import TOL_BF16_ABS, block_rows, device_tensors, mask_compare, out_error

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_cache = {}


def workload_inputs(name, seed):
    key = (name, seed)
    if key not in _cache:
        _cache.clear()
        w = inputs.WORKLOADS[name]
        q, k, v = inputs.make_inputs(w, seed)
        _cache[key] = (w, q, k, v, device_tensors(q, k, v, w.dtype))
    return _cache[key]


def run_workload(name, seed, tau, heads, block_step):
    import torch
    import block_sparse_video_solattn_amd as sa
    w, q, k, v, (qd, kd, vd) = workload_inputs(name, seed)
    nb = w.nb
    out, words, _, _ = sa.solattn_forward_debug(qd, kd, vd, None, w.prefix_len, tau, "sparse",
                                                want_scores=False)
    # the production entry point must give the same output as the debug one
    out2 = sa.solattn_forward(qd, kd, vd, None, w.prefix_len, tau, "sparse")
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    gmask = sa.unpack_mask(words, nb)
    n_diff = n_near = 0
    for h in range(w.H):
        r = oracle.head(q[0, h], k[0, h], v[0, h], w.prefix_len, tau, want_out=False)
        nd, nn = mask_compare(gmask, r, 0, h)
        n_diff += nd
        n_near += nn
    pb = (w.prefix_len + 63) // 64
    assert gmask[..., :pb].all()
    blocks = sorted(set(list(range(0, nb, block_step)) + [nb - 1]))
    g = out.float().cpu().numpy()
    worst = 0.0
    for h in heads:
        r = oracle.head(q[0, h], k[0, h], v[0, h], w.prefix_len, tau,
                        mask_override=gmask[0, h].astype(np.uint8), qblocks=blocks)
        ab, _ = out_error(g[0, h].astype(np.float64), r["out"], block_rows(blocks, w.N))
        worst = max(worst, ab)
    print("%s tau=%g: video skip %.4f, mask diffs %d (near-threshold %d), max abs err %.4g"
          % (name, tau, 1 - gmask[..., pb:].mean(), n_diff, n_near, worst))
    assert worst <= TOL_BF16_ABS
    return gmask


@pytest.mark.parametrize("tau", [1.0, 1.25, 1.5])
def test_refine_workload(tau):
    run_workload("refine", 3000, tau, heads=(0, 13, 31), block_step=8)


def test_draft_workload_calibrated_tau():
    with open(os.path.join(GOLDEN, "draft_tau.json")) as f:
        cal = json.load(f)
    m = run_workload("draft", cal["seed"], cal["tau"], heads=(0, 31), block_step=24)
    pb = 8
    assert abs((1 - m[..., pb:].mean()) - 0.90) < 0.01


def test_long_workload_ragged_tail():
    m = run_workload("long", 5000, 1.5, heads=(0, 31), block_step=40)
    assert m.shape[-1] == 757
