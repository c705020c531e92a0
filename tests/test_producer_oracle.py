"""Pins of the Q/K producer oracle (oracle/producer.py): a hand-worked case
that fixes the order norm -> weight -> rotation, the RMS and scale invariants
of the norm, the rotation against complex multiplication, pass-through of the
unrotated channels, norm preservation, the relative-position property of
rotary tables, and the single rounding to bf16 against a brute-force search."""
import numpy as np
import pytest

from oracle import producer as P
from block_sparse_video_solattn_amd import inputs as I


def test_hand_worked_case():
    # x = (3, 4, 0, 0): mean square 25/4, rms 2.5 -> (1.2, 1.6, 0, 0);
    # weight (2, 0.5, 1, 1) -> (2.4, 0.8, 0, 0); the first pair turned by a
    # quarter turn (cos 0, sin 1) -> (-0.8, 2.4, 0, 0).  Weighting after the
    # rotation would give (-3.2, 0.6), rotating before the norm the same as
    # here only if the weight were uniform.
    x = np.array([[3.0, 4.0, 0.0, 0.0]])
    y = P.qknorm_rope(x, np.array([2.0, 0.5, 1.0, 1.0]), 1e-300,
                      np.array([[0.0]]), np.array([[1.0]]))
    np.testing.assert_allclose(y, [[-0.8, 2.4, 0.0, 0.0]], rtol=0, atol=1e-15)
    # eps enters under the root: mean square 6.25 + eps 3.75 -> rms sqrt(10)
    y = P.qknorm_rope(x, None, 3.75)
    np.testing.assert_allclose(y, x / np.sqrt(10.0), rtol=1e-15)


def test_rms_is_one_and_scale_invariant():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 50, 128)) * rng.uniform(0.01, 100, (3, 50, 1))
    y = P.qknorm_rope(x, None, 1e-300)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    y2 = P.qknorm_rope(7.25 * x, None, 1e-300)
    np.testing.assert_allclose(y2, y, rtol=1e-13, atol=1e-15)
    # the weight scales each channel linearly
    g = rng.uniform(0.5, 2.0, 128)
    np.testing.assert_allclose(P.qknorm_rope(x, g, 1e-300), y * g, rtol=1e-14)


def test_rotation_is_complex_multiplication_and_rest_passes_through():
    rng = np.random.default_rng(2)
    N, d, r = 40, 64, 24
    x = rng.standard_normal((2, N, d))
    ang = rng.uniform(-np.pi, np.pi, (N, r // 2))
    y = P.qknorm_rope(x, None, 1e-6, np.cos(ang), np.sin(ang))
    base = P.qknorm_rope(x, None, 1e-6)
    z = base[..., 0:r:2] + 1j * base[..., 1:r:2]
    zr = z * np.exp(1j * ang)
    np.testing.assert_allclose(y[..., 0:r:2], zr.real, atol=1e-14)
    np.testing.assert_allclose(y[..., 1:r:2], zr.imag, atol=1e-14)
    assert np.array_equal(y[..., r:], base[..., r:])
    # a rotation keeps every pair's length, so the row norm too
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(base, axis=-1),
                               rtol=1e-14)
    # zero angles are the identity
    y0 = P.qknorm_rope(x, None, 1e-6, np.ones((N, r // 2)), np.zeros((N, r // 2)))
    assert np.array_equal(y0, base)


def test_relative_position_property():
    # tables from angles t * omega_i: the dot product of a query at position
    # t with a key at position s depends on t - s only
    rng = np.random.default_rng(3)
    d, r, N = 64, 64, 40
    omega = 10000.0 ** (-np.arange(r // 2) / (r // 2))
    ang = np.arange(N)[:, None] * omega[None, :]
    c, s = np.cos(ang), np.sin(ang)
    q = np.repeat(rng.standard_normal((1, d)), N, axis=0)
    k = np.repeat(rng.standard_normal((1, d)), N, axis=0)
    qr = P.qknorm_rope(q, None, 1e-6, c, s)
    kr = P.qknorm_rope(k, None, 1e-6, c, s)
    for t, u, shift in [(5, 2, 11), (0, 17, 20), (30, 30, -25)]:
        np.testing.assert_allclose(qr[t] @ kr[u], qr[t + shift] @ kr[u + shift], rtol=1e-11)
    # and it does depend on the offset
    assert abs(qr[5] @ kr[2] - qr[5] @ kr[3]) > 1e-6


def test_round_bf16_single_rounding():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-30, 30, 20000),
                        [0.0, 1.0, -1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8,
                         # just above a tie: fp32 would round it onto the tie first
                         1 + 2 ** -8 + 2 ** -40, -(1 + 2 ** -8 + 2 ** -40)]])
    got = P.round_bf16(v)
    # brute force: the two bf16 neighbours of v from its binade's spacing
    e = np.floor(np.log2(np.abs(np.where(v == 0, 1, v))))
    step = 2.0 ** (e - 7)
    lo = np.floor(v / step) * step
    hi = lo + step
    dlo, dhi = np.abs(v - lo), np.abs(hi - v)
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi,
                    np.where(np.mod(lo / step, 2) == 0, lo, hi)))
    want = np.where(v == 0, 0.0, want)
    assert np.array_equal(got, want)
    assert got[-4] == 1.0 and got[-3] == 1 + 2 ** -6
    assert got[-2] == 1 + 2 ** -7 and got[-1] == -(1 + 2 ** -7)
    # on float32 inputs it agrees with torch's conversion
    torch = pytest.importorskip("torch")
    x = (rng.standard_normal(5000) * 100).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(P.round_bf16(x.astype(np.float64)), ref)


def test_produce_rounds_once():
    d = I.producer_inputs(1, 1, 130, 64, "bf16", prefix_len=2, grid=(2, 8, 8), seed=5)
    exact = P.qknorm_rope(d["q"], d["gamma_q"], 1e-6, d["cos"], d["sin"])
    got = P.produce(d["q"], d["gamma_q"], 1e-6, d["cos"], d["sin"], "bf16")
    assert got.dtype == np.float32
    assert np.array_equal(got.astype(np.float64), P.round_bf16(exact))
    assert np.all(np.abs(got - exact) <= np.abs(exact) * 2.0 ** -8)


def test_rope_tables_recipe():
    cos, sin = I.rope_tables(300, 44, (2, 8, 16), 64)
    assert cos.shape == (300, 32) and cos.dtype == np.float32
    # prefix tokens and the grid origin are unrotated
    assert np.all(cos[:45] == 1) and np.all(sin[:45] == 0)
    np.testing.assert_allclose(cos ** 2 + sin ** 2, 1.0, rtol=1e-6)
