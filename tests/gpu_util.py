"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C ABI (via the binding) and compare with the
fp64 oracle on the same inputs."""
import math

import numpy as np

BAND = 1e-4          # near-threshold band (scaled-logit units), both mask bits accepted
TOL_BF16_ABS = 2e-2  # bf16 outputs, unit-variance V
TOL_F32_REL = 1e-5   # fp32 outputs, max|g - o| / max|o|


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


def out_error(gout, oout, rows=None):
    g, o = gout, oout
    if rows is not None:
        g, o = g[rows], o[rows]
    ok = ~np.isnan(o).any(axis=-1)
    g, o = g[ok], o[ok]
    return float(np.max(np.abs(g - o))), float(np.max(np.abs(g - o)) / max(np.max(np.abs(o)), 1e-30))


def block_rows(blocks, N):
    rows = []
    for i in blocks:
        rows.extend(range(64 * i, min(N, 64 * i + 64)))
    return np.array(rows, dtype=np.int64)


def is_inf(tau):
    return math.isinf(tau)
