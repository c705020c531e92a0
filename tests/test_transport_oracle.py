"""Pins of the transport oracle (oracle/transport.py): the record size the
pages state (132 -> 144 bytes at d = 128), closed-form quantization cases,
an exhaustive E4M3 round trip and a brute-force nearest-value search, bf16
rounding against torch, and the pack / exchange / unpack layouts against a
direct per-row quantization of the assembled tensors."""
import numpy as np
import pytest

from oracle import transport as T


def test_record_size_matches_the_pages():
    # 128 int8 codes + a 4-byte scale = 132 bytes, aligned to 144
    assert T.record_bytes(128) == 144
    assert T.record_bytes(64) == 80


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 100,
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0,
                                  3.0e38, 1e-40], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(T.to_bf16(x).view(np.uint32), ref.view(np.uint32))
    # ties to even: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    assert T.to_bf16(np.float32(1 + 2 ** -8)) == 1.0
    assert T.to_bf16(np.float32(1 + 3 * 2 ** -8)) == np.float32(1 + 2 ** -6)


def test_int8_closed_forms():
    c, s = T.quant_int8(np.array([[0.0, 63.5, -127.0, 1.0]], np.float32))
    assert s[0] == 1.0
    assert list(c[0]) == [0, 64, -127, 1]          # 63.5 ties to even 64
    c, s = T.quant_int8(np.zeros((2, 8), np.float32))
    assert not c.any() and not s.any()
    c, s = T.quant_int8(np.full((1, 8), 0.75, np.float32))
    assert (c == 127).all() and s[0] == np.float32(0.75) / np.float32(127)


def test_int8_extremes_and_error_bound():
    rng = np.random.default_rng(2)
    x = T.to_bf16((rng.standard_normal((500, 128)) * rng.uniform(0.01, 50, (500, 1))).astype(np.float32))
    c, s = T.quant_int8(x)
    amax_idx = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(c[np.arange(500), amax_idx]) == 127)
    assert np.abs(c.astype(int)).max() <= 127
    xr = T.dequant_int8(c, s)
    # half a quantization step plus the bf16 rounding of the result
    bound = s[:, None] * 0.5 * (1 + 1e-6) + np.abs(xr) * 2.0 ** -8
    assert np.all(np.abs(xr - x) <= bound)
    # odd symmetry
    c2, s2 = T.quant_int8(-x)
    assert np.array_equal(c2, -c) and np.array_equal(s2, s)


def test_e4m3_exhaustive_round_trip():
    table = T.e4m3_decode_table()
    finite = [c for c in range(256) if not np.isnan(table[c])]
    assert len(finite) == 254 and np.isnan(table[0x7F]) and np.isnan(table[0xFF])
    codes = T.e4m3_encode(table[finite].astype(np.float32))
    assert list(codes) == finite
    assert table[0x7E] == 448 and table[0x38] == 1 and table[0x01] == 2.0 ** -9
    assert table[0x08] == 2.0 ** -6 and table[0xC0] == -2


def test_e4m3_nearest_even_against_brute_force():
    table = T.e4m3_decode_table()
    finite = np.array([c for c in range(256) if not np.isnan(table[c]) and c != 0x80])
    vals = table[finite]
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-0.05, 0.05, 20000),
                        [1 + 1 / 16, 1 + 3 / 16, 1.5 * 2 ** -9, 0.5 * 2 ** -9, 447.9, 440.0]])
    y = y.astype(np.float32)
    got = T.e4m3_encode(y)
    gv = table[got]
    dist = np.abs(vals[None, :] - y[:, None].astype(np.float64))
    best = dist.min(1)
    assert np.all(np.abs(gv - y) == best)             # a nearest value
    ties = (dist == best[:, None]).sum(1) > 1
    # on a tie the even mantissa wins
    assert np.all((got[ties] & 1) == 0)
    assert T.e4m3_encode(np.float32(1 + 1 / 16)) == 0x38
    assert T.e4m3_encode(np.float32(1 + 3 / 16)) == 0x3A
    assert T.e4m3_encode(np.float32(1.5 * 2 ** -9)) == 0x02
    assert T.e4m3_encode(np.float32(0.5 * 2 ** -9)) == 0x00


def test_fp8_row_extremes():
    x = np.array([[0.0, -3.0, 1.5, 2.0]], np.float32)
    c, s = T.quant_fp8(x)
    assert s[0] == np.float32(3.0) / np.float32(448)
    assert c[0, 1] == 0xFE                              # -448
    xr = T.dequant_fp8(c, s)
    assert xr[0, 1] == -3.0 and xr[0, 0] == 0.0


def _bf16_rand(rng, shape, scale=1.0):
    return T.to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("P,B,H,Ns,d", [(2, 1, 4, 3, 64), (4, 2, 8, 5, 128), (1, 1, 2, 7, 128)])
def test_qkv_exchange_layout(P, B, H, Ns, d):
    rng = np.random.default_rng(4)
    Hp = H // P
    full = [_bf16_rand(rng, (B, H, P * Ns, d), 3.0) for _ in range(3)]   # q, k, v
    # rank s holds the sequence shard s of every head
    sends = [T.pack_qkv_int8(*(x[:, :, s * Ns:(s + 1) * Ns] for x in full), P) for s in range(P)]
    assert sends[0].shape == (P, B, Hp, Ns, 3, T.record_bytes(d))
    recv = T.all_to_all(sends)
    for p in range(P):
        got = T.unpack_qkv_int8(recv[p], d)
        for x, g in zip(full, got):
            c, s = T.quant_int8(x[:, p * Hp:(p + 1) * Hp])
            assert np.array_equal(g, T.dequant_int8(c, s))
    # padding bytes are zero
    assert not sends[0][..., d + 4:].any()


@pytest.mark.parametrize("P,B,Hp,Ns,d", [(2, 1, 2, 3, 64), (4, 1, 1, 5, 128)])
def test_output_exchange_layout(P, B, Hp, Ns, d):
    rng = np.random.default_rng(5)
    # rank p holds heads p*Hp .. of the full sequence
    outs = [_bf16_rand(rng, (B, Hp, P * Ns, d)) for _ in range(P)]
    sends = [T.pack_out_fp8(o, P) for o in outs]
    recv = T.all_to_all(sends)
    for r in range(P):
        got = T.unpack_out_fp8(recv[r], d)
        assert got.shape == (B, P * Hp, Ns, d)
        for p in range(P):
            c, s = T.quant_fp8(outs[p][:, :, r * Ns:(r + 1) * Ns])
            assert np.array_equal(got[:, p * Hp:(p + 1) * Hp], T.dequant_fp8(c, s))
