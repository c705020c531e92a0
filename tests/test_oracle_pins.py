"""Pins of the fp64 oracle to things other than itself.

Each test checks one part of the oracle against a closed form, a textbook
routine (numpy / torch softmax attention), an invariant the method must obey,
or the hand-worked threshold examples in tests/golden.  Chosen so that a
plausible slip (a dropped n_j weight, the wrong std convention, a transposed
score, the wrong block for a pooled term, a missed prefix) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from block_sparse_video_solattn_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_dense(q, k, v):
    """Textbook softmax(q k^T / sqrt(d)) v in fp64, written independently."""
    d = q.shape[-1]
    s = (q.astype(np.float64) @ k.astype(np.float64).T) / math.sqrt(d)
    s -= s.max(axis=1, keepdims=True)
    w = np.exp(s)
    return (w @ v.astype(np.float64)) / w.sum(axis=1, keepdims=True)


def rand_head(N, d, seed, offset=1.5):
    rng = np.random.default_rng(seed)
    nb = (N + 63) // 64
    out = []
    for _ in range(3):
        x = rng.standard_normal((N, d)) + np.repeat(rng.standard_normal((nb, d)) * offset, 64, 0)[:N]
        out.append(x)
    return out


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------- pooling
@pytest.mark.parametrize("N", [64, 1000, 1024, 37])
def test_pooling_is_block_mean(N):
    q, k, v = rand_head(N, 16, 1)
    r = oracle.head(q, k, v, 0, 1.0, want_out=False)
    for name, x in (("qbar", q), ("kbar", k), ("vbar", v)):
        nb = (N + 63) // 64
        ref = np.stack([x[64 * j:min(N, 64 * j + 64)].mean(axis=0) for j in range(nb)])
        assert rel(r[name], ref) < 1e-14, name
    if N % 64:
        # the tail block averages only its own rows
        tail = N % 64
        assert np.allclose(r["kbar"][-1], k[N - tail:].sum(0) / tail, rtol=1e-14, atol=0)


def test_constant_block_pools_to_its_row():
    q, k, v = rand_head(256, 8, 2)
    k[64:128] = k[64]
    r = oracle.head(q, k, v, 0, 1.0, want_out=False)
    assert np.allclose(r["kbar"][1], k[64], rtol=1e-14, atol=0)
    # dyadic values make every partial sum exact: the mean is the row itself
    k[64:128] = np.round(k[64] * 8) / 8
    r = oracle.head(q, k, v, 0, 1.0, want_out=False)
    assert np.array_equal(r["kbar"][1], k[64])


# ---------------------------------------------------------------- scores
def test_scores_are_scaled_pooled_dot_products():
    q, k, v = rand_head(640, 32, 3)
    r = oracle.head(q, k, v, 0, 1.0, want_out=False)
    ref = (r["qbar"] @ r["kbar"].T) / math.sqrt(32)
    assert rel(r["score"], ref) < 1e-13
    # query-block index is the row, key-block index the column
    qb = q.reshape(10, 64, 32).mean(1)
    kb = k.reshape(10, 64, 32).mean(1)
    assert abs(r["score"][2, 7] - qb[2] @ kb[7] / math.sqrt(32)) < 1e-12


# ---------------------------------------------------------------- threshold
def _score_row_inputs(scores, d=64):
    """Inputs whose score row 0 equals `scores` exactly: query block 0 rows are
    8*e0 and key block j rows are scores[j]*e0, so s_0j = 8*scores[j]/sqrt(64)."""
    nb = len(scores)
    N = 64 * nb
    q = np.zeros((N, d))
    q[:, 0] = 8.0
    k = np.zeros((N, d))
    for j, s in enumerate(scores):
        k[64 * j:64 * j + 64, 0] = s
    v = np.random.default_rng(0).standard_normal((N, d))
    return q, k, v


def test_threshold_worked_examples():
    with open(os.path.join(GOLDEN, "threshold_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        tau = float(c["tau"])
        q, k, v = _score_row_inputs(c["scores"])
        mode = oracle.SPARSE | (oracle.VIDEO_STATS if c.get("video_stats") else 0)
        r = oracle.head(q, k, v, 64 * c["prefix_blocks"], tau, mode=mode, want_out=False)
        assert np.allclose(r["score"][0], c["scores"], atol=1e-15)
        thr = float(c["thr"])
        if math.isinf(thr):
            assert r["thr"][0] == thr
        else:
            assert abs(r["thr"][0] - thr) < 1e-12, c
        assert list(r["mask"][0]) == c["keep"], c


@pytest.mark.parametrize("base", [oracle.SPARSE, oracle.TOPK])
def test_prefix_rows_variant_keeps_every_block(base):
    # PREFIX_ROWS: query blocks inside the prefix keep every key block (their
    # rows are plain dense attention); the other rows route as without it
    rng = np.random.default_rng(41)
    N, d, prefix = 64 * 12 + 20, 32, 150   # Pb = 3, ragged last block
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    tau = math.inf if base == oracle.SPARSE else 0.25
    plain = oracle.head(q, k, v, prefix, tau, mode=base)
    var = oracle.head(q, k, v, prefix, tau, mode=base | oracle.PREFIX_ROWS)
    dense = oracle.head(q, k, v, prefix, 0.0, mode=oracle.DENSE)
    pb = 3
    assert var["mask"][:pb].all()
    assert np.all(var["thr"][:pb] == -math.inf)
    assert np.array_equal(var["mask"][pb:], plain["mask"][pb:])
    assert np.array_equal(var["thr"][pb:], plain["thr"][pb:])
    if base == oracle.SPARSE:
        assert not plain["mask"][:pb, pb:].any()   # tau = +inf: prefix only
    rows = slice(0, 64 * pb)
    assert np.array_equal(var["out"][rows], dense["out"][rows])
    assert np.array_equal(var["out"][64 * pb:], plain["out"][64 * pb:])


def test_video_stats_variant_on_random_rows():
    # VIDEO_STATS: the threshold of every row is mean + tau * population std
    # of its video scores, recomputed here with numpy from the oracle's scores
    rng = np.random.default_rng(42)
    N, d, prefix = 64 * 20, 32, 200   # Pb = 4
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    r = oracle.head(q, k, v, prefix, 0.8, mode=oracle.SPARSE | oracle.VIDEO_STATS, want_out=False)
    video = r["score"][:, 4:]
    thr = video.mean(1) + 0.8 * video.std(1)
    assert np.allclose(r["thr"], thr, rtol=0, atol=1e-12)
    keep = np.concatenate([np.ones((20, 4), bool), r["score"][:, 4:] >= r["thr"][:, None]], 1)
    assert np.array_equal(r["mask"].astype(bool), keep)
    whole = oracle.head(q, k, v, prefix, 0.8, want_out=False)
    assert not np.allclose(whole["thr"], r["thr"])


def test_variant_flags_rejected_where_they_do_not_apply():
    q = k = v = np.zeros((128, 8))
    for mode, tau in ((oracle.DENSE | oracle.PREFIX_ROWS, 0.0), (oracle.TOPK | oracle.VIDEO_STATS, 0.5),
                      (oracle.DENSE | oracle.VIDEO_STATS, 0.0), (oracle.SPARSE | 0x40, 1.0)):
        with pytest.raises(ValueError):
            oracle.head(q, k, v, 64, tau, mode=mode)


@pytest.mark.parametrize("tau", [-1.0, 0.0, 1.0, 2.5, math.inf])
def test_prefix_always_kept(tau):
    q, k, v = rand_head(1024, 16, 4)
    for prefix in (1, 64, 65, 300):
        r = oracle.head(q, k, v, prefix, tau, want_out=False)
        pb = (prefix + 63) // 64
        assert r["mask"][:, :pb].all()
        if tau == math.inf:
            assert not r["mask"][:, pb:].any()


def test_mask_invariances():
    q, k, v = rand_head(2048, 32, 5)
    base = oracle.head(q, k, v, 128, 1.0, want_out=False)["mask"]
    # positive scaling of Q scales every score row: mask unchanged
    assert np.array_equal(oracle.head(3.0 * q, k, v, 128, 1.0, want_out=False)["mask"], base)
    # adding one vector to every key shifts each score row by a constant
    u = np.random.default_rng(6).standard_normal(32)
    assert np.array_equal(oracle.head(q, k + u, v, 128, 1.0, want_out=False)["mask"], base)
    # permuting tokens inside a key block leaves the mask alone
    perm = np.arange(2048)
    perm[640:704] = perm[640:704][::-1]
    assert np.array_equal(oracle.head(q, k[perm], v[perm], 128, 1.0, want_out=False)["mask"], base)


@pytest.mark.parametrize("tau,expect", [(1.0, 0.159), (1.25, 0.106), (1.5, 0.067)])
def test_kept_fraction_gaussian_rows(tau, expect):
    # pooled vectors dominated by independent Gaussian offsets give near
    # Gaussian score rows; kept fraction ~ 1 - Phi(tau) (sanity band only)
    q, k, v = rand_head(64 * 512, 64, 7, offset=3.0)
    m = oracle.head(q, k, v, 0, tau, want_out=False)["mask"]
    assert abs(m.mean() - expect) < 0.03


# ---------------------------------------------------------------- exact part
def test_dense_matches_bruteforce_and_torch():
    q, k, v = rand_head(700, 32, 8)
    ref = brute_dense(q, k, v)
    r = oracle.head(q, k, v, 0, 0.0, mode=oracle.DENSE)
    assert rel(r["out"], ref) < 1e-12
    torch = pytest.importorskip("torch")
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None])[0, 0].numpy()
    assert rel(r["out"], t) < 1e-12


def test_tau_minus_inf_is_dense():
    q, k, v = rand_head(1000, 16, 9)
    r = oracle.head(q, k, v, 128, -math.inf)
    assert r["mask"].all()
    assert rel(r["out"], brute_dense(q, k, v)) < 1e-12


def test_all_ones_override_is_dense():
    q, k, v = rand_head(640, 16, 10)
    r = oracle.head(q, k, v, 0, 1.0, mask_override=np.ones((10, 10), np.uint8))
    assert rel(r["out"], brute_dense(q, k, v)) < 1e-12


def test_single_block_rows_keep_everything():
    # Nb = 1: sigma = 0, threshold = mean, the only block is kept -> dense
    for N in (10, 64):
        q, k, v = rand_head(N, 8, 11)
        r = oracle.head(q, k, v, 0, 2.0)
        assert r["mask"].all()
        assert rel(r["out"], brute_dense(q, k, v)) < 1e-12


# ---------------------------------------------------------------- correction
@pytest.mark.parametrize("N,j", [(1024, 9), (1000, 15), (1024, 0)])
def test_constant_block_correction_is_exact(N, j):
    q, k, v = rand_head(N, 32, 12)
    lo, hi = 64 * j, min(N, 64 * j + 64)
    k[lo:hi] = k[lo]
    v[lo:hi] = v[lo]
    nb = (N + 63) // 64
    keep_all = np.ones((nb, nb), np.uint8)
    skip_j = keep_all.copy()
    skip_j[:, j] = 0
    a = oracle.head(q, k, v, 0, 0.0, mask_override=keep_all)["out"]
    b = oracle.head(q, k, v, 0, 0.0, mask_override=skip_j)["out"]
    assert rel(b, a) < 1e-12


def test_constant_keys_alone_suffice():
    # identical keys but distinct values: the pooled value is the block mean
    # and every key gets the same weight, so the term is still exact
    q, k, v = rand_head(512, 16, 13)
    k[128:192] = k[128]
    keep = np.ones((8, 8), np.uint8)
    skip = keep.copy()
    skip[:, 2] = 0
    a = oracle.head(q, k, v, 0, 0.0, mask_override=keep)["out"]
    b = oracle.head(q, k, v, 0, 0.0, mask_override=skip)["out"]
    assert rel(b, a) < 1e-12


def test_all_blocks_constant_and_tau_inf_is_dense():
    q, k, v = rand_head(1000, 16, 14)
    for j in range(16):
        lo, hi = 64 * j, min(1000, 64 * j + 64)
        k[lo:hi] = k[lo]
        v[lo:hi] = v[lo]
    r = oracle.head(q, k, v, 0, math.inf)
    assert not r["mask"].any()
    assert rel(r["out"], brute_dense(q, k, v)) < 1e-12


def test_pooled_term_weight_is_block_length():
    # every block skipped: the output is softmax attention over the pooled keys
    # with log(n_j) added to each logit (tail block n = 40)
    q, k, v = rand_head(1000, 16, 15)
    r = oracle.head(q, k, v, 0, math.inf)
    n = np.array([64] * 15 + [40], np.float64)
    s = q @ r["kbar"].T / 4.0 + np.log(n)[None, :]
    s -= s.max(1, keepdims=True)
    w = np.exp(s)
    ref = w @ r["vbar"] / w.sum(1, keepdims=True)
    assert rel(r["out"], ref) < 1e-12


def test_mixed_routing_matches_augmented_key_softmax():
    q, k, v = rand_head(1000, 32, 16)
    r = oracle.head(q, k, v, 64, 0.5)
    m = r["mask"]
    assert 0 < m.mean() < 1
    N = 1000
    for i in (0, 7, 15):
        keys, vals, bias = [], [], []
        for j in range(16):
            lo, hi = 64 * j, min(N, 64 * j + 64)
            if m[i, j]:
                keys.append(k[lo:hi]); vals.append(v[lo:hi]); bias.append(np.zeros(hi - lo))
            else:
                keys.append(r["kbar"][j:j + 1]); vals.append(r["vbar"][j:j + 1])
                bias.append(np.array([math.log(hi - lo)]))
        K, V, b = np.concatenate(keys), np.concatenate(vals), np.concatenate(bias)
        rows = slice(64 * i, min(N, 64 * i + 64))
        s = q[rows] @ K.T / math.sqrt(32) + b[None, :]
        s -= s.max(1, keepdims=True)
        w = np.exp(s)
        assert rel(r["out"][rows], w @ V / w.sum(1, keepdims=True)) < 1e-12


def test_jensen_pooled_mass_below_exact_mass():
    # n_j exp(c q.kbar_j) <= sum_t exp(c q.k_t) for every row and block, so a
    # skipped block's pooled mass never exceeds its exact mass
    q, k, v = rand_head(512, 16, 17)
    r = oracle.head(q, k, v, 0, 1.0, want_out=False)
    c = 1.0 / 4.0
    for j in range(8):
        exact = np.exp(q @ k[64 * j:64 * j + 64].T * c).sum(1)
        pooled = 64 * np.exp(q @ r["kbar"][j] * c)
        assert np.all(pooled <= exact * (1 + 1e-12))


# ---------------------------------------------------------------- normalisation
@pytest.mark.parametrize("tau", [-math.inf, 0.0, 1.0, math.inf])
def test_constant_values_give_constant_output(tau):
    q, k, _ = rand_head(1000, 16, 18)
    v = np.ones((1000, 16))
    r = oracle.head(q, k, v, 128, tau)
    assert np.max(np.abs(r["out"] - 1.0)) < 1e-13


def test_affine_in_values():
    q, k, v = rand_head(1000, 16, 19)
    b = np.random.default_rng(20).standard_normal(16)
    r0 = oracle.head(q, k, v, 64, 1.0)
    r1 = oracle.head(q, k, 2.5 * v + b, 64, 1.0)
    assert np.array_equal(r0["mask"], r1["mask"])
    assert rel(r1["out"], 2.5 * r0["out"] + b) < 1e-13


def test_outputs_inside_value_hull():
    q, k, v = rand_head(1000, 16, 21)
    out = oracle.head(q, k, v, 0, 1.25)["out"]
    assert np.all(out >= v.min(0) - 1e-12) and np.all(out <= v.max(0) + 1e-12)


def test_permuting_non_prefix_key_blocks():
    q, k, v = rand_head(1024, 16, 22)
    r0 = oracle.head(q, k, v, 128, 1.0)
    order = [0, 1, 5, 3, 9, 2, 15, 7, 8, 4, 10, 11, 12, 13, 14, 6]
    perm = np.concatenate([np.arange(64 * j, 64 * j + 64) for j in order])
    r1 = oracle.head(q, k[perm], v[perm], 128, 1.0)
    assert np.array_equal(r1["mask"], r0["mask"][:, order])
    assert rel(r1["out"], r0["out"]) < 1e-12


def test_query_blocks_subset_matches_full():
    q, k, v = rand_head(1000, 16, 23)
    full = oracle.head(q, k, v, 64, 1.0)
    part = oracle.head(q, k, v, 64, 1.0, qblocks=[3, 15])
    rows = np.r_[192:256, 960:1000]
    assert np.array_equal(part["out"][rows], full["out"][rows])
    assert np.isnan(part["out"][0]).all()


# ---------------------------------------------------------------- arguments
def test_rejects_bad_arguments():
    q, k, v = rand_head(128, 8, 24)
    with pytest.raises(ValueError):
        oracle.head(q, k, v, 0, float("nan"))
    with pytest.raises(ValueError):
        oracle.head(q, k, v, 129, 1.0)
    with pytest.raises(ValueError):
        oracle.head(q, k, v, -1, 1.0)


def test_tiny_workload_end_to_end():
    w = inputs.WORKLOADS["tiny"]
    q, k, v = inputs.make_inputs(w, 1000)
    r = oracle.forward(q, k, v, w.prefix_len, 1.0)
    assert r["out"].shape == q.shape
    assert np.isfinite(r["out"]).all()
    m = r["mask"][0, 0]
    assert m[:, :2].all() and 0 < m.mean() < 1


# ------------------------------------------------- fixed-ratio (TOPK) routing
def brute_block_sparse(q, k, v, keep_row, nb):
    """softmax over the keys of the kept blocks only, written independently."""
    cols = np.concatenate([np.arange(64 * j, min(64 * j + 64, k.shape[0]))
                           for j in range(nb) if keep_row[j]])
    return brute_dense(q, k[cols], v[cols])


def test_topk_worked_examples():
    # prefix block 0, video scores [1, 4, 1, 5, 9, 2, 6]:
    #   f = 0.3 -> k = ceil(2.1) = 3 -> top three {9, 6, 5} -> threshold 5
    #   f = 1/7 -> k = ceil(1.0) = 1 -> {9}, threshold 9 (exact multiple)
    #   f = 0.5 -> k = ceil(3.5) = 4 -> {9, 6, 5, 4}, threshold 4
    #   f = 1   -> every block
    scores = [3.0, 1.0, 4.0, 1.0, 5.0, 9.0, 2.0, 6.0]
    q, k, v = _score_row_inputs(scores)
    for f, thr, keep in ((0.3, 5.0, [1, 0, 0, 0, 1, 1, 0, 1]),
                         (1.0 / 7.0, 9.0, [1, 0, 0, 0, 0, 1, 0, 0]),
                         (0.5, 4.0, [1, 0, 1, 0, 1, 1, 0, 1]),
                         (1.0, 1.0, [1] * 8)):
        r = oracle.head(q, k, v, 64, f, mode=oracle.TOPK, want_out=False)
        assert r["thr"][0] == thr, f
        assert list(r["mask"][0]) == keep, f


def test_topk_ties_at_the_threshold_are_all_kept():
    # video scores [2, 7, 7, 3], f = 0.25 -> k = 1 -> threshold 7, both 7s kept
    q, k, v = _score_row_inputs([0.0, 2.0, 7.0, 7.0, 3.0])
    r = oracle.head(q, k, v, 64, 0.25, mode=oracle.TOPK, want_out=False)
    assert list(r["mask"][0]) == [1, 0, 1, 1, 0]


def test_topk_no_video_blocks_keeps_the_prefix():
    q, k, v = rand_head(300, 16, 40)
    r = oracle.head(q, k, v, 300, 0.1, mode=oracle.TOPK)
    assert r["mask"].all()
    assert np.allclose(r["out"], brute_dense(q, k, v), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("N,prefix,f", [(1000, 128, 0.1), (777, 0, 0.25), (640, 64, 0.5)])
def test_topk_counts_and_ranking(N, prefix, f):
    q, k, v = rand_head(N, 32, 41)
    nb = (N + 63) // 64
    pb = (prefix + 63) // 64
    kk = min(nb - pb, math.ceil(f * (nb - pb)))
    r = oracle.head(q, k, v, prefix, f, mode=oracle.TOPK, want_out=False)
    for i in range(nb):
        s = r["score"][i]
        vid = np.arange(pb, nb)
        top = set(vid[np.argsort(-s[pb:], kind="stable")][:kk].tolist())
        kept = set(np.nonzero(r["mask"][i][pb:])[0] + pb)
        assert kept == top                                    # distinct scores: exactly the top k
        assert r["mask"][i][:pb].all()
        assert r["thr"][i] == np.sort(s[pb:])[::-1][kk - 1]


@pytest.mark.parametrize("N,prefix,f", [(700, 64, 0.2), (333, 0, 0.5)])
def test_topk_output_is_block_sparse_softmax(N, prefix, f):
    # skipped blocks contribute nothing: each row is a softmax over the kept
    # blocks' keys alone
    q, k, v = rand_head(N, 16, 42)
    nb = (N + 63) // 64
    r = oracle.head(q, k, v, prefix, f, mode=oracle.TOPK)
    for i in range(nb):
        rows = slice(64 * i, min(64 * i + 64, N))
        ref = brute_block_sparse(q[rows], k, v, r["mask"][i], nb)
        assert np.allclose(r["out"][rows], ref, rtol=1e-12, atol=1e-12)


def test_topk_fraction_one_is_dense():
    q, k, v = rand_head(500, 16, 43)
    a = oracle.head(q, k, v, 64, 1.0, mode=oracle.TOPK)
    b = oracle.head(q, k, v, 64, 0.0, mode=oracle.DENSE)
    assert a["mask"].all()
    assert np.array_equal(a["out"], b["out"])


def test_topk_rejects_fraction_outside_unit_interval():
    q, k, v = rand_head(128, 8, 44)
    for f in (0.0, -0.5, 1.5, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            oracle.head(q, k, v, 0, f, mode=oracle.TOPK)
