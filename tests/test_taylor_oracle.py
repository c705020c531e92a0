"""Pins of the first-order (Taylor) oracle (oracle/taylor.py): order 0 is the
C oracle's operator, constant blocks carry no correction, tau = -inf is
dense attention, the correction's token-sum form equals the covariance form,
and the error against exact attention falls like eps (order 0) and eps^2
(order 1) when skipped blocks' keys sit eps from their mean."""
import numpy as np

import oracle
from oracle import taylor as T


def _dense(q, k, v):
    s = q @ k.T / np.sqrt(q.shape[1])
    s -= s.max(1, keepdims=True)
    w = np.exp(s)
    return (w @ v) / w.sum(1, keepdims=True)


def _iid(N, d, seed):
    rng = np.random.default_rng(seed)
    nb = (N + 63) // 64
    x = [rng.standard_normal((N, d)) + np.repeat(rng.standard_normal((nb, d)) * 1.5, 64, 0)[:N]
         for _ in range(3)]
    return x


def test_order_zero_is_the_c_oracle():
    q, k, v = _iid(530, 64, 1)
    for tau, prefix in ((1.0, 64), (0.3, 0), (2.0, 100)):
        a = T.head(q, k, v, prefix, tau, order=0)["out"]
        b = oracle.head(q, k, v, prefix, tau)["out"]
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_constant_blocks_carry_no_correction():
    q, k, v = _iid(400, 32, 2)
    kc = k.copy()
    for j in range(0, 400, 64):
        kc[j:j + 64] = kc[j]                 # every key block constant: dk = 0
    a0 = T.head(q, kc, v, 0, 0.5, order=0)["out"]
    a1 = T.head(q, kc, v, 0, 0.5, order=1)["out"]
    np.testing.assert_allclose(a1, a0, rtol=0, atol=1e-14)
    vc = v.copy()
    for j in range(0, 400, 64):
        vc[j:j + 64] = vc[j]                 # every value block constant: dv = 0
    np.testing.assert_allclose(T.head(q, k, vc, 0, 0.5, order=1)["out"],
                               T.head(q, k, vc, 0, 0.5, order=0)["out"], rtol=0, atol=1e-14)


def test_tau_minus_inf_is_dense():
    q, k, v = _iid(300, 32, 3)
    np.testing.assert_allclose(T.head(q, k, v, 0, -np.inf, order=1)["out"], _dense(q, k, v),
                               rtol=0, atol=1e-12)


def test_correction_as_a_token_sum():
    # c C^T q = (1/n) sum_t c (q.k_t - q.k_bar) v_t  (sum_t dk_t = 0): the
    # form that needs no d x d matrix
    rng = np.random.default_rng(4)
    k, v = rng.standard_normal((50, 16)), rng.standard_normal((50, 16))
    q = rng.standard_normal(16)
    c = 0.25
    lhs = c * T.block_cov(k, v, 0, 50).T @ q
    rhs = (c * (k @ q - k.mean(0) @ q)) @ v / 50
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-14)


def test_error_falls_like_eps_and_eps_squared():
    # keys of every block = the block's base key + eps * D with D of zero
    # block mean, so the pooled means, the scores and the mask do not depend
    # on eps; values arbitrary
    rng = np.random.default_rng(5)
    N, d, nb = 64 * 8, 32, 8
    q = rng.standard_normal((N, d))
    base = np.repeat(rng.standard_normal((nb, d)) * 1.5, 64, 0)
    D = rng.standard_normal((N, d))
    D -= np.repeat(D.reshape(nb, 64, d).mean(1), 64, 0)
    v = rng.standard_normal((N, d))
    errs = {0: [], 1: []}
    masks = []
    for eps in (0.2, 0.1, 0.05):
        k = base + eps * D
        exact = _dense(q, k, v)
        for order in (0, 1):
            r = T.head(q, k, v, 0, 0.5, order=order)
            errs[order].append(np.abs(r["out"] - exact).max())
            masks.append(r["mask"])
    assert all(np.array_equal(m, masks[0]) for m in masks)
    assert (~masks[0]).sum() > 0.3 * nb * nb        # blocks are skipped
    r0 = [errs[0][a] / errs[0][a + 1] for a in range(2)]
    r1 = [errs[1][a] / errs[1][a + 1] for a in range(2)]
    assert all(1.7 < x < 2.3 for x in r0), r0        # first order in eps
    assert all(3.3 < x < 4.7 for x in r1), r1        # second order in eps
    assert errs[1][-1] < errs[0][-1] / 10
