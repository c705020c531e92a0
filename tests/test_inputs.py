"""The seeded input generators: shapes, determinism, bf16 rounding."""
import numpy as np

from block_sparse_video_solattn_amd import inputs


def test_workload_sizes():
    W = inputs.WORKLOADS
    assert (W["tiny"].N, W["tiny"].nb) == (1024, 16)
    assert (W["small"].N, W["small"].nb) == (8192, 128)
    assert (W["refine"].N, W["refine"].nb) == (16384, 256)
    assert (W["draft"].N, W["draft"].nb) == (32768, 512)
    assert (W["long"].N, W["long"].nb) == (48416, 757)
    assert W["long"].N % 64 == 32


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5], np.float32)
    r = inputs.round_to_bf16(x)
    assert list(r) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5]
    assert np.array_equal(inputs.round_to_bf16(r), r)
    assert inputs.bf16_bits(np.array([1.0], np.float32))[0] == 0x3F80


def test_heads_are_independent_streams():
    w = inputs.WORKLOADS["small"]
    q_all, k_all, v_all = inputs.make_inputs(w, 2000)
    q2, k2, v2 = inputs.make_inputs(w, 2000, heads=[2])
    assert np.array_equal(q_all[:, 2], q2[:, 0]) and np.array_equal(v_all[:, 2], v2[:, 0])
    q_b, _, _ = inputs.make_inputs(w, 2001, heads=[2])
    assert not np.array_equal(q_b, q2)


def test_values_are_bf16_and_unit_scale():
    w = inputs.WORKLOADS["small"]
    q, k, v = inputs.make_inputs(w, 2000, heads=[0])
    for x in (q, k, v):
        assert np.array_equal(inputs.round_to_bf16(x), x)
        assert 0.7 < x[0, 0, w.prefix_len:].std() < 1.5


def test_video_positions_fill_grid_in_order():
    p = inputs.video_positions(7936, (8, 24, 42))
    assert tuple(p[0]) == (0, 0, 0) and tuple(p[41]) == (0, 0, 41) and tuple(p[42]) == (0, 1, 0)
    assert tuple(p[-1]) == (7, 20, 39)


def test_constant_key_block_variant():
    w = inputs.WORKLOADS["tiny"]
    q, k, v = inputs.make_inputs(w, 1000, const_key_block=9)
    blk = k[0, 0, 576:640]
    assert (blk == blk[0]).all() and (v[0, 0, 576:640] == v[0, 0, 576]).all()
