"""Oracle of the fused Q/K producer: QKNorm then partial RoPE.  TEST
INFRASTRUCTURE ONLY.

Plain numpy in float64.  Shares no code with the GPU library; only the tests,
the smoke check and the benchmark's CPU leg may import it.

What the pages say: the engine fuses the chain "QKNorm + partial RoPE" so
that its intermediates stay in registers (page "MiniMax 官宣 NVIDIA Sol 团队
H3 加速:5 秒视频 1.653 秒生成并开源", section "提速来自流水线每一段的叠加",
fused-operator item; page "NVIDIA 與 SANA Sol-Engine" news, section "技術組成":
QKNorm + RoPE among the fused lossless kernels that cut HBM traffic).  They
give neither the norm's parameters nor the rotary layout, so these readings
are taken:

  * QKNorm is an RMSNorm over each head's d channels of one token:
    y = x / sqrt(mean(x^2) + eps) * gamma, gamma a length-d weight shared by
    all heads (None: all ones), eps > 0;
  * partial RoPE rotates the first r channels (r even, 0 <= r <= d) of the
    normalised vector in adjacent pairs (2i, 2i+1), i < r/2, by the angle
    whose cosine and sine the caller tabulates per token:
    (y0, y1) -> (y0 c - y1 s, y0 s + y1 c) with c = cos[t][i], s = sin[t][i];
    channels r .. d-1 pass through.  (Any other pairing of the channels is a
    fixed permutation of them, which the projection weights can absorb.)
    The norm comes first and its weight belongs to it; the rotation acts on
    the weighted result;
  * the attention consumes the results rounded to the input's element type
    (bf16: nearest, ties to even, straight from the exact value).

tests/test_producer_oracle.py pins each step (a hand-worked row, invariants,
complex multiplication, brute-force rounding); against the pages, which print
no formula, the readings above are parity unpinned.
"""
import numpy as np


def qknorm_rope(x, gamma, eps: float, rope_cos=None, rope_sin=None) -> np.ndarray:
    """x [..., N, d] -> the normalised, rotated rows in float64.

    gamma: [d] or None; rope_cos / rope_sin: [N][r/2] (None when r = 0)."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    ms = np.sum(x * x, axis=-1, keepdims=True) / d
    y = x / np.sqrt(ms + float(eps))
    if gamma is not None:
        y = y * np.asarray(gamma, np.float64)
    if rope_cos is None:
        return y
    c = np.asarray(rope_cos, np.float64)
    s = np.asarray(rope_sin, np.float64)
    half = c.shape[-1]
    assert 2 * half <= d and c.shape == s.shape and c.shape[0] == x.shape[-2]
    out = y.copy()
    y0 = y[..., 0:2 * half:2]
    y1 = y[..., 1:2 * half:2]
    out[..., 0:2 * half:2] = y0 * c - y1 * s
    out[..., 1:2 * half:2] = y0 * s + y1 * c
    return out


def round_bf16(v) -> np.ndarray:
    """float64 -> the nearest bf16 value (8 significant bits, ties to even),
    rounded once from the exact value, returned as float64.  Values must be
    zero or of magnitude in bf16's normal range."""
    v = np.asarray(v, np.float64)
    m, e = np.frexp(v)                          # v = m 2^e, 0.5 <= |m| < 1
    nz = v != 0
    assert np.all(np.abs(v[nz]) >= 2.0 ** -126) and np.all(np.abs(v[nz]) < 2.0 ** 128)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def produce(x, gamma, eps: float, rope_cos=None, rope_sin=None, dtype: str = "bf16"):
    """The producer's output in the element type the attention reads:
    float32 values, bf16-representable for dtype "bf16"."""
    y = qknorm_rope(x, gamma, eps, rope_cos, rope_sin)
    if dtype == "bf16":
        return round_bf16(y).astype(np.float32)
    return y.astype(np.float32)
