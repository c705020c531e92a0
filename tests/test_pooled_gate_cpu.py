"""The pooled-term gate of the bf16 parity tests (gpu_util.POOLED_GATE),
checked on the CPU against what it is meant to separate: a correctly
computed output, rounded to bf16 as the GPU rounds it, must score well under
the gate; an output with one pooled tile dropped, or with the ragged tail
block's pooled term weighted by 64 instead of its own key count, must score
well over it -- while both mistakes can stay inside the absolute bf16 bound.
The mistakes are planted in a brute-force softmax over kept keys and pooled
keys written here (the augmented-key form of the pooled correction), never
in the oracle."""
import numpy as np
import pytest

import oracle
from block_sparse_video_solattn_amd import inputs
from gpu_util import POOLED_GATE, pooled_gate


def brute(q, k, v, keep, drop_tiles=(), tail_count=None):
    """Rows of q [R, d] against the keys of their query blocks' masks keep
    [R, Nb]: exact keys of kept blocks, one pooled key per skipped block
    with log-weight ln n_j (ln tail_count for the last block when given),
    skipped blocks whose pooled tile (64 blocks per tile) is in drop_tiles
    left out."""
    N, d = k.shape
    nb = (N + 63) // 64
    n = np.array([min(64, N - 64 * j) for j in range(nb)])
    kbar = np.stack([k[64 * j:64 * j + n[j]].mean(0) for j in range(nb)])
    vbar = np.stack([v[64 * j:64 * j + n[j]].mean(0) for j in range(nb)])
    out = np.empty((q.shape[0], d))
    for r in range(q.shape[0]):
        ks, vs, bs = [], [], []
        for j in range(nb):
            if keep[r, j]:
                ks.append(k[64 * j:64 * j + n[j]])
                vs.append(v[64 * j:64 * j + n[j]])
                bs.append(np.zeros(n[j]))
            elif j // 64 not in drop_tiles:
                cnt = tail_count if (tail_count is not None and j == nb - 1) else n[j]
                ks.append(kbar[j:j + 1])
                vs.append(vbar[j:j + 1])
                bs.append(np.array([np.log(cnt)]))
        K, V, b = np.concatenate(ks), np.concatenate(vs), np.concatenate(bs)
        lg = K @ q[r] / np.sqrt(d) + b
        p = np.exp(lg - lg.max())
        out[r] = p @ V / p.sum()
    return out


def to_bf16(x):
    torch = pytest.importorskip("torch")
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("N,tau", [(64 * 30 + 8, float("inf")), (64 * 30 + 8, 1.0),
                                   (64 * 130 + 8, 1.0)])
def test_gate_separates_correct_from_planted_mistakes(N, tau):
    grid = (1, -(-(N - 64) // 64), 64)
    q, k, v = inputs.custom(1, 1, N, 128, "bf16", prefix_len=64, seed=N % 97 + 3, kind="field",
                            grid=grid)
    q, k, v = (x[0, 0].astype(np.float64) for x in (q, k, v))
    r = oracle.head(q, k, v, 64, tau, want_out=False)
    mask = r["mask"]
    full = oracle.head(q, k, v, 64, tau, mask_override=mask)["out"]
    nopool = oracle.head(q, k, v, 64, 0.5, mode=oracle.TOPK, mask_override=mask)["out"]
    # a correct result rounded to bf16, as the GPU stores it
    good, _ = pooled_gate(to_bf16(full), full, nopool)
    assert good <= POOLED_GATE / 4, good
    # the brute force reproduces the oracle (so the planted variants differ
    # from it only by the planted mistake)
    rows = np.arange(0, N, 16)
    keep = mask[rows // 64].astype(bool)
    assert np.max(np.abs(brute(q[rows], k, v, keep) - full[rows])) < 1e-12
    nb = mask.shape[0]
    tail = N - 64 * (nb - 1)
    scores = {}
    for T in range((nb + 63) // 64):
        if T * 64 + 64 > nb and (nb - 64 * T) < 16:
            continue            # a tile holding only a few blocks moves the rows little
        scores["drop tile %d" % T] = brute(q[rows], k, v, keep, drop_tiles=(T,))
    scores["tail weighted as 64 keys"] = brute(q[rows], k, v, keep, tail_count=64)
    assert tail == 8
    for name, bad in scores.items():
        sg, _ = pooled_gate(bad, full[rows], nopool[rows])
        assert sg >= 2 * POOLED_GATE, (name, sg)
