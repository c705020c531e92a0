"""Oracle of the sequence-parallel transport kernels.  TEST INFRASTRUCTURE ONLY.

Plain numpy, float32 arithmetic where a rounding decides an integer code, so
that it takes each decision in the same precision as the GPU.  Shares no code
with the GPU library; only the tests, the smoke check and the benchmark's CPU
leg may import it.

What the pages say (page "MiniMax 官宣 NVIDIA Sol 团队 H3 加速:5 秒视频 1.653
秒生成并开源", section "提速来自流水线每一段的叠加", multi-GPU item; page
"英伟达开源 Sol-H3，给 MiniMax-H3 加速，5 秒视频 1.4 秒出", section "2.2 剩下三层
加速", communication paragraph): Q/K/V are packed per destination GPU and
exchanged with one all-to-all; the fastest setting sends Q/K/V as INT8 with
block quantization and the attention output as FP8, in records aligned from
132 to 144 bytes.  Readings taken here:

  * a quantization block is one token's d-vector of one head (one record):
    d codes plus one fp32 scale = d + 4 bytes (132 at d = 128), padded with
    zero bytes to a multiple of 16 (144 at d = 128);
  * INT8: amax = max |x| over the row; scale s = amax / 127 and inverse
    inv = 127 / amax, both fp32 divisions rounded to nearest even;
    code = clamp(round_half_even(x * inv), -127, 127) with x * inv an fp32
    product; a zero row has s = 0 and codes 0.  Dequantized value: the fp32
    product code * s rounded to bf16 (nearest even);
  * FP8: the OCP E4M3 format (bias 7, 3 mantissa bits, largest finite 448,
    no infinities), with s = amax / 448, inv = 448 / amax (fp32),
    y = clamp(x * inv, -448, 448) in fp32 and code = y rounded to the
    nearest E4M3 value, ties to even mantissa; dequantized: bf16(decode(code) * s);
  * layouts ("packed per destination"), with P ranks, H = P * Hp heads and
    sequence shards of Ns tokens:
      Q/K/V send buffer of sequence shard s: [P][B][Hp][Ns][3][rec], chunk p
      holding heads p*Hp .. p*Hp + Hp - 1, tensor order q, k, v;
      after the exchange, rank p holds [P(source s)][B][Hp][Ns][3][rec] and
      unpacks it to q, k, v [B][Hp][P*Ns][d], token s*Ns + t;
      output send buffer of head group p: [P][B][Hp][Ns][rec], chunk r
      holding tokens r*Ns .. r*Ns + Ns - 1; rank r receives
      [P(source p)][B][Hp][Ns][rec] and unpacks it to o [B][P*Hp][Ns][d].
"""
import numpy as np

F32 = np.float32
E4M3_MAX = 448.0


def record_bytes(d: int) -> int:
    return (d + 4 + 15) // 16 * 16


def to_bf16(x) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float32 values."""
    x = np.ascontiguousarray(x, dtype=F32)
    b = x.view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    out = (r << 16).astype(np.uint32).view(F32)
    return np.where(np.isnan(x), x, out)


def quant_int8(x: np.ndarray):
    """Rows of x (last axis) -> (codes int8, scale fp32)."""
    x = np.asarray(x, dtype=F32)
    amax = np.max(np.abs(x), axis=-1)
    zero = amax == 0
    safe = np.where(zero, F32(1), amax).astype(F32)
    s = np.where(zero, F32(0), safe / F32(127)).astype(F32)
    inv = np.where(zero, F32(0), F32(127) / safe).astype(F32)
    y = (x * inv[..., None]).astype(F32)
    codes = np.clip(np.rint(y), -127, 127).astype(np.int8)
    return codes, s


def dequant_int8(codes: np.ndarray, s: np.ndarray) -> np.ndarray:
    return to_bf16(codes.astype(F32) * np.asarray(s, F32)[..., None])


def e4m3_decode_table() -> np.ndarray:
    """Value of every E4M3 code 0..255 (NaN for the two NaN codes)."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * m * 2.0 ** -9
        else:
            vals[c] = sign * (1 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """float32 values with |y| <= 448 -> E4M3 codes, round to nearest even."""
    y = np.asarray(y, dtype=np.float64)   # float32 values are exact in float64
    assert np.all(np.abs(y) <= E4M3_MAX)
    a = np.abs(y)
    sign = (np.signbit(y)).astype(np.uint8) << 7
    code = np.zeros(y.shape, np.int64)
    sub = a < 2.0 ** -6
    # subnormals (and zero): a = m * 2^-9, m = 0..8 (8 carries into the
    # smallest normal, whose code is 8 as well)
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub
    m_, e_ = np.frexp(a[nrm])             # a = m_ * 2^e_, m_ in [0.5, 1)
    e = e_ - 1                            # a = (2 m_) * 2^e, 2 m_ in [1, 2)
    mant = np.rint((2 * m_ - 1) * 8).astype(np.int64)
    carry = mant == 8
    e = e + carry
    mant = np.where(carry, 0, mant)
    code[nrm] = ((e + 7) << 3) | mant
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quant_fp8(x: np.ndarray):
    """Rows of x -> (E4M3 codes uint8, scale fp32)."""
    x = np.asarray(x, dtype=F32)
    amax = np.max(np.abs(x), axis=-1)
    zero = amax == 0
    safe = np.where(zero, F32(1), amax).astype(F32)
    s = np.where(zero, F32(0), safe / F32(E4M3_MAX)).astype(F32)
    inv = np.where(zero, F32(0), F32(E4M3_MAX) / safe).astype(F32)
    y = np.clip((x * inv[..., None]).astype(F32), -E4M3_MAX, E4M3_MAX).astype(F32)
    return e4m3_encode(y), s


def dequant_fp8(codes: np.ndarray, s: np.ndarray) -> np.ndarray:
    v = e4m3_decode_table()[codes.astype(np.int64)].astype(F32)
    return to_bf16(v * np.asarray(s, F32)[..., None])


def _records(codes: np.ndarray, s: np.ndarray, d: int) -> np.ndarray:
    """codes [..., d] (int8 or uint8), s [...] -> records [..., rec] uint8."""
    rec = record_bytes(d)
    out = np.zeros(codes.shape[:-1] + (rec,), np.uint8)
    out[..., :d] = codes.view(np.uint8)
    out[..., d:d + 4] = np.ascontiguousarray(np.asarray(s, F32)[..., None]).view(np.uint8)
    return out


def pack_qkv_int8(q, k, v, P: int) -> np.ndarray:
    """q, k, v [B][H][Ns][d] (float values, bf16-representable) of one
    sequence shard -> send buffer [P][B][Hp][Ns][3][rec] uint8."""
    B, H, Ns, d = q.shape
    assert H % P == 0
    Hp = H // P
    recs = []
    for x in (q, k, v):
        c, s = quant_int8(x)
        recs.append(_records(c, s, d))                       # [B][H][Ns][rec]
    r = np.stack(recs, axis=3)                               # [B][H][Ns][3][rec]
    r = r.reshape(B, P, Hp, Ns, 3, -1).transpose(1, 0, 2, 3, 4, 5)
    return np.ascontiguousarray(r)


def unpack_qkv_int8(recv: np.ndarray, d: int):
    """recv [P][B][Hp][Ns][3][rec] -> q, k, v [B][Hp][P*Ns][d] (bf16 values)."""
    P, B, Hp, Ns, three, rec = recv.shape
    codes = recv[..., :d].copy().view(np.int8)
    s = recv[..., d:d + 4].copy().view(F32)[..., 0]
    x = dequant_int8(codes, s)                               # [P][B][Hp][Ns][3][d]
    x = x.transpose(4, 1, 2, 0, 3, 5).reshape(3, B, Hp, P * Ns, d)
    return x[0], x[1], x[2]


def pack_out_fp8(o: np.ndarray, P: int) -> np.ndarray:
    """o [B][Hp][P*Ns][d] of one head group -> send buffer [P][B][Hp][Ns][rec]."""
    B, Hp, N, d = o.shape
    assert N % P == 0
    Ns = N // P
    c, s = quant_fp8(o)
    r = _records(c, s, d).reshape(B, Hp, P, Ns, -1).transpose(2, 0, 1, 3, 4)
    return np.ascontiguousarray(r)


def unpack_out_fp8(recv: np.ndarray, d: int) -> np.ndarray:
    """recv [P][B][Hp][Ns][rec] (chunk s from head group s) -> o [B][P*Hp][Ns][d]."""
    P, B, Hp, Ns, rec = recv.shape
    codes = recv[..., :d].copy()
    s = recv[..., d:d + 4].copy().view(F32)[..., 0]
    x = dequant_fp8(codes, s)                                # [P][B][Hp][Ns][d]
    return np.ascontiguousarray(x.transpose(1, 0, 2, 3, 4).reshape(B, P * Hp, Ns, d))


def all_to_all(sends):
    """The exchange itself, emulated: sends[s] = [P][...] from rank s ->
    recv[p] = [P(source s)][...] with recv[p][s] = sends[s][p]."""
    P = len(sends)
    return [np.stack([sends[s][p] for s in range(P)]) for p in range(P)]
