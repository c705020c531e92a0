"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C ABI (via the binding) and compare with the
fp64 oracle on the same inputs."""
import math

import numpy as np

BAND = 1e-4          # near-threshold band (scaled-logit units), both mask bits accepted
TOL_BF16_ABS = 2e-2  # bf16 outputs, unit-variance V
TOL_F32_REL = 1e-5   # fp32 outputs, max|g - o| / max|o|
# Pooled-term gate for bf16 outputs, on top of TOL_BF16_ABS: the largest
# row error against the full oracle must stay below this fraction of the
# median row distance between the full oracle and the same oracle with every
# pooled term dropped (pooled_gate).  A bf16-rounded oracle output scores
# 0.0003-0.009 on the gated cases; one dropped pooled tile or a tail block
# weighted with 64 instead of its own key count scores 0.14 or more (both
# measured on the CPU, tests/test_pooled_gate_cpu.py).
POOLED_GATE = 0.05


def device_tensors(q, k, v, dtype):
    import torch
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    return [torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(td).contiguous() for x in (q, k, v)]


def gpu_debug(q, k, v, dtype, prefix_len, tau, mode="sparse"):
    """Run solattn_forward_debug; returns numpy (out fp64, mask bool, scores, thr)."""
    import torch
    import block_sparse_video_solattn_amd as sa
    qd, kd, vd = device_tensors(q, k, v, dtype)
    out, words, scores, thr = sa.solattn_forward_debug(qd, kd, vd, None, prefix_len, tau, mode)
    torch.cuda.synchronize()
    nb = (q.shape[2] + 63) // 64
    return (out.float().cpu().numpy().astype(np.float64), sa.unpack_mask(words, nb),
            scores.cpu().numpy().astype(np.float64), thr.cpu().numpy().astype(np.float64))


def mask_compare(gmask, ores, b, h):
    """Compare the GPU keep mask of one slice with the oracle's.  Differences
    are allowed only where the oracle's fp64 score lies within BAND of its
    threshold.  Returns (n_diff, n_near)."""
    om = ores["mask"].astype(bool)
    s, thr = ores["score"], ores["thr"][:, None]
    near = np.abs(s - thr) <= BAND
    diff = gmask[b, h] != om
    bad = diff & ~near
    assert not bad.any(), "mask differs outside the near-threshold band at %s" % (
        np.argwhere(bad)[:5].tolist())
    return int(diff.sum()), int(near.sum())


def max_abs_diff(g, o):
    """max |g - o| over the elements, +inf as soon as g holds a non-finite
    value (NaN or inf), so that a caller folding errors with max() -- which
    drops NaN -- cannot pass on a broken output."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if g.size == 0:
        return 0.0
    if not np.isfinite(g).all():
        return float("inf")
    return float(np.max(np.abs(g - o)))


def out_error(gout, oout, rows=None):
    """(max abs error, max abs error / max |oracle|) over the rows the
    oracle produced; both +inf when the GPU rows hold NaN or inf."""
    g, o = gout, oout
    if rows is not None:
        g, o = g[rows], o[rows]
    ok = ~np.isnan(o).any(axis=-1)
    g, o = g[ok], o[ok]
    ab = max_abs_diff(g, o)
    return ab, ab / max(float(np.max(np.abs(o))) if o.size else 0.0, 1e-30)


def block_rows(blocks, N):
    rows = []
    for i in blocks:
        rows.extend(range(64 * i, min(N, 64 * i + 64)))
    return np.array(rows, dtype=np.int64)


def is_inf(tau):
    return math.isinf(tau)


def pooled_gate(g, full, nopool):
    """max_r max_c |g - full| / median_r max_c |full - nopool| over the rows
    given (all [R, d]): the GPU's worst row error as a fraction of how far
    the pooled terms move a typical row.  +inf for a non-finite g."""
    e = max_abs_diff(g, full)
    dist = np.abs(np.asarray(full, np.float64) - np.asarray(nopool, np.float64)).max(axis=1)
    return e / max(float(np.median(dist)), 1e-300), float(np.median(dist))
