"""Oracle of Sol-Attn with the first-order (Taylor) correction of skipped
blocks.  TEST INFRASTRUCTURE ONLY.

Plain numpy, float64, one (batch, head) slice at a time; the routing (pooled
means, scores, thresholds, keep mask) comes from the C oracle's routing
(oracle.head with want_out=False), which tests/test_oracle_pins.py pins.
Shares no code with the GPU library; only the tests, the smoke check and the
benchmark's CPU leg may import it.

What the pages say: the skipped blocks' pooled compensation is called a
Taylor approximation (page "MiniMax 官推背书 Sol Engine：H3 的 10 秒 768p 生成
从 414s 压到 14.93s", section "同一项目页上的另一种口径：3.95× 近无损"); the
pooled correction is described on page "NVIDIA 团队开源 Sol-H3 的 DGX Spark 版
本", section "119.68 GiB 的内存池", Sol-Attn item.  No form is printed.  The
reading taken here expands each skipped block's exact contribution around its
pooled key k_bar_j (c = 1/sqrt(d), dk_t = k_t - k_bar_j, dv_t = v_t - v_bar_j,
n = n_j):

  sum_t exp(c q.k_t) v_t  = exp(c q.k_bar) sum_t exp(c q.dk_t) (v_bar + dv_t)
                          ~ exp(c q.k_bar) sum_t (1 + c q.dk_t) (v_bar + dv_t)
                          = n exp(c q.k_bar) (v_bar + c C_j^T q),
  C_j = (1/n) sum_t dk_t dv_t^T            (sum_t dk_t = sum_t dv_t = 0),

  sum_t exp(c q.k_t)      ~ n exp(c q.k_bar)   (its first-order term vanishes).

So the zeroth-order term (the default operator) keeps its weight and only the
skipped block's value moves from v_bar_j to v_bar_j + c C_j^T q_r.  Here C_j
is formed explicitly as a d x d matrix.

tests/test_taylor_oracle.py pins it: order 0 reproduces the C oracle's output,
constant blocks have C_j = 0, tau = -inf is dense attention, and on blocks
whose keys sit eps from their mean the error against exact attention falls
like eps at order 0 and like eps^2 at order 1.
"""
from typing import Optional

import numpy as np

import oracle

BLOCK = 64


def block_cov(k: np.ndarray, v: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """C_j = (1/n) sum_t (k_t - k_bar)(v_t - v_bar)^T over tokens [lo, hi)."""
    kb = k[lo:hi] - k[lo:hi].mean(0)
    vb = v[lo:hi] - v[lo:hi].mean(0)
    return kb.T @ vb / (hi - lo)


def head(q, k, v, prefix_len: int, tau: float, order: int = 1,
         mask_override: Optional[np.ndarray] = None, rows: Optional[np.ndarray] = None,
         mode: int = oracle.SPARSE) -> dict:
    """One slice: q, k, v [N, d].  Returns {"out": [len(rows), d], "mask"}.

    order 0: exact kept blocks plus the pooled zeroth-order term of every
    skipped block (the default operator); order 1: the skipped blocks'
    values also carry c C_j^T q_r.  mask_override replaces the routing
    (several masks are correct where a score sits on its threshold); mode
    is the C oracle's routing mode (SPARSE with its variant flags)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, d = q.shape
    nb = (N + BLOCK - 1) // BLOCK
    r = oracle.head(q, k, v, prefix_len, tau, mode=mode, want_out=False)
    mask = r["mask"].astype(bool) if mask_override is None else np.asarray(mask_override, bool)
    c = 1.0 / np.sqrt(d)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    lo = np.arange(nb) * BLOCK
    hi = np.minimum(lo + BLOCK, N)
    n = (hi - lo).astype(np.float64)
    kbar = np.stack([k[a:b].mean(0) for a, b in zip(lo, hi)])
    vbar = np.stack([v[a:b].mean(0) for a, b in zip(lo, hi)])
    cov = [block_cov(k, v, a, b) for a, b in zip(lo, hi)] if order >= 1 else None
    out = np.empty((len(rows), d))
    for x, rr in enumerate(rows):
        i = rr // BLOCK
        keep = mask[i]
        toks = np.concatenate([np.arange(lo[j], hi[j]) for j in np.flatnonzero(keep)]) \
            if keep.any() else np.zeros(0, np.int64)
        skip = np.flatnonzero(~keep)
        lk = c * (k[toks] @ q[rr])                            # exact logits
        lp = c * (kbar[skip] @ q[rr]) + np.log(n[skip])        # pooled logits (with ln n_j)
        m = max(lk.max(initial=-np.inf), lp.max(initial=-np.inf))
        wk = np.exp(lk - m)
        wp = np.exp(lp - m)
        val = vbar[skip].copy()
        if order >= 1:
            for a, j in enumerate(skip):
                val[a] += c * (cov[j].T @ q[rr])
        out[x] = (wk @ v[toks] + wp @ val) / (wk.sum() + wp.sum())
    return {"out": out, "mask": mask}
