"""Seeded synthetic inputs for the Sol-Attn workloads.

This module only draws random numbers and lays them out; it holds none of the
attention method's arithmetic (no pooling, scoring, routing or softmax).  Both
the HIP path (through the tests and the benchmark) and the CPU oracle receive
the arrays it returns, so the two sides always see bit-identical inputs.

Workload shapes follow the latent geometry the pages give for the two stages
of the Sol-H3 pipeline:

* draft stage: 672x384 canvas, 124 frames, 16x spatial compression
  (page "NVIDIA 团队开源 Sol-H3 的 DGX Spark 版本", section "潜空间直传";
  page "英伟达开源 Sol-H3", section 2.1 for the 16x / 32x VAE factors);
* refine stage: 1344x768, 121 frames, 32x spatial / 8x temporal compression
  (same pages, same sections).

A packed sequence puts an always-exact prefix (text, conditioning video, audio)
ahead of the target video tokens (page "英伟达开源 Sol-H3", section 2.2).  The
prefix tokens here are i.i.d. normal stand-ins; the video tokens are a smooth
3-D sinusoid field on the latent grid plus noise, so block scores vary the way
spatially coherent latents make them vary.  Real latents need the model
weights, which are not part of this operator.

Random streams: every (batch, head) slice has its own PCG64 stream seeded with
``SeedSequence([seed, b, h])``, so any subset of heads can be regenerated on
its own.  Values are drawn in float64, cast to float32, and (for bf16
workloads) rounded to the nearest bf16 value, ties to even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

BLOCK = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str            # "f32" or "bf16"
    prefix_len: int
    taus: tuple           # tau values the workload is run at
    grid: Optional[tuple]  # (T, Y, X) latent grid of the video tokens, None for iid
    kind: str             # "iid_offset" (Q, K, V), "iid_qk_offset" (Q, K only) or "field"

    @property
    def nb(self) -> int:
        return (self.N + BLOCK - 1) // BLOCK


# The five workloads.  Sizes: tokens = prefix + video; video = T*Y*X except
# "small", whose grid is only partly filled (see video_positions()).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1024, 64, "f32", 128, (1.0,), None, "iid_offset"),
    "small": Workload("small", 1, 4, 8192, 128, "bf16", 256, (1.25,), (8, 24, 42), "field"),
    "refine": Workload("refine", 1, 32, 256 + 16 * 24 * 42, 128, "bf16", 256,
                       (1.0, 1.25, 1.5), (16, 24, 42), "field"),
    "draft": Workload("draft", 1, 32, 512 + 32 * 24 * 42, 128, "bf16", 512,
                      (), (32, 24, 42), "field"),
    "long": Workload("long", 1, 32, 2048 + 46 * 24 * 42, 128, "bf16", 2048,
                     (1.5,), (46, 24, 42), "field"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16-representable float32 array -> its uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def video_positions(n_video: int, grid: tuple) -> np.ndarray:
    """(t, y, x) integer coordinates of the first n_video cells of the grid,
    row-major (t slowest, x fastest)."""
    T, Y, X = grid
    assert n_video <= T * Y * X
    idx = np.arange(n_video, dtype=np.int64)
    return np.stack([idx // (Y * X), (idx // X) % Y, idx % X], axis=1)


def _rng(seed: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b, h])))


def _head_iid_offset(rng, N, D, v_offset=True):
    out = []
    nb = (N + BLOCK - 1) // BLOCK
    for t in range(3):  # Q, K, V
        base = rng.standard_normal((N, D))
        offs = rng.standard_normal((nb, D)) * 1.5
        if t < 2 or v_offset:
            out.append(base + np.repeat(offs, BLOCK, axis=0)[:N])
        else:
            out.append(base)
    return out


def _head_field(rng, N, D, prefix_len, grid):
    T, Y, X = grid
    n_video = N - prefix_len
    pos = video_positions(n_video, grid).astype(np.float64)
    omega = rng.uniform(0.0, 2.0, size=(8, 3))          # cycles per axis extent
    phi = rng.uniform(0.0, 2.0 * math.pi, size=8)
    a_q = rng.standard_normal((8, D)) * math.sqrt(2.0 / 8.0)
    a_k = rng.standard_normal((8, D)) * math.sqrt(2.0 / 8.0)
    pre = [rng.standard_normal((prefix_len, D)) for _ in range(3)]
    arg = 2.0 * math.pi * (pos[:, 0:1] * omega[None, :, 0] / T
                           + pos[:, 1:2] * omega[None, :, 1] / Y
                           + pos[:, 2:3] * omega[None, :, 2] / X) + phi[None, :]
    basis = np.sin(arg)                                    # [n_video, 8]
    q_vid = basis @ a_q + rng.standard_normal((n_video, D)) * 0.5
    k_vid = basis @ a_k + rng.standard_normal((n_video, D)) * 0.5
    v_vid = rng.standard_normal((n_video, D))
    return [np.concatenate([pre[0], q_vid]), np.concatenate([pre[1], k_vid]),
            np.concatenate([pre[2], v_vid])]


def make_inputs(w: Workload, seed: int, heads: Optional[Sequence[int]] = None,
                const_key_block: Optional[int] = None):
    """Return (q, k, v) as float32 arrays [B, len(heads), N, D].

    For bf16 workloads every value is already a bf16 value.  ``heads`` selects
    a subset (default all); the values of a head do not depend on which other
    heads are generated.  ``const_key_block`` makes every key and value row of
    that key block equal to the block's first row (the "constant block" case).
    """
    heads = list(range(w.H)) if heads is None else list(heads)
    shape = (w.B, len(heads), w.N, w.D)
    q = np.empty(shape, np.float32)
    k = np.empty(shape, np.float32)
    v = np.empty(shape, np.float32)
    for b in range(w.B):
        for hi, h in enumerate(heads):
            rng = _rng(seed, b, h)
            if w.kind in ("iid_offset", "iid_qk_offset"):
                qq, kk, vv = _head_iid_offset(rng, w.N, w.D, v_offset=w.kind == "iid_offset")
            else:
                qq, kk, vv = _head_field(rng, w.N, w.D, w.prefix_len, w.grid)
            q[b, hi], k[b, hi], v[b, hi] = qq, kk, vv
    if const_key_block is not None:
        j = const_key_block
        lo, hi_ = j * BLOCK, min(w.N, (j + 1) * BLOCK)
        k[:, :, lo:hi_] = k[:, :, lo:lo + 1]
        v[:, :, lo:hi_] = v[:, :, lo:lo + 1]
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v


def custom(B, H, N, D, dtype="bf16", prefix_len=0, seed=0, kind="iid_qk_offset",
           grid=None) -> tuple:
    """Inputs for an arbitrary shape (edge-case tests).  Default kind: Q and K
    i.i.d. N(0,1) plus a per-block N(0, 1.5^2) offset, V i.i.d. N(0,1) (unit
    variance, the regime the bf16 tolerance is stated for)."""
    if kind == "field" and grid is None:
        n_video = N - prefix_len
        grid = (1, 1, max(1, n_video))
    w = Workload("custom", B, H, N, D, dtype, prefix_len, (), grid, kind)
    return make_inputs(w, seed)


def logit_jump(B, H, N, D, dtype="bf16", jump_block=5, scale=6.0, seed=0) -> tuple:
    """Inputs whose logits rise steeply after the first key block: every
    query row is a shared direction u (i.i.d. N(0,1) per head) plus N(0, 0.25^2)
    noise; keys are i.i.d. N(0,1) except block ``jump_block``, whose rows are
    scale * u plus N(0, 0.1^2) noise; values i.i.d. N(0,1).  Against that block
    a query's logit is about scale * |u|^2 / sqrt(D) (natural units) while
    block 0's logits stay of order one -- the case where a softmax reference
    taken from the first block falls far below the row maximum."""
    q = np.empty((B, H, N, D), np.float32)
    k = np.empty((B, H, N, D), np.float32)
    v = np.empty((B, H, N, D), np.float32)
    lo, hi = jump_block * BLOCK, min(N, (jump_block + 1) * BLOCK)
    for b in range(B):
        for h in range(H):
            rng = _rng(seed, b, h)
            u = rng.standard_normal(D)
            q[b, h] = u[None, :] + 0.25 * rng.standard_normal((N, D))
            kk = rng.standard_normal((N, D))
            kk[lo:hi] = scale * u[None, :] + 0.1 * rng.standard_normal((hi - lo, D))
            k[b, h] = kk
            v[b, h] = rng.standard_normal((N, D))
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v



def rope_tables(N: int, prefix_len: int, grid: tuple, rope_dim: int,
                base: float = 10000.0) -> tuple:
    """Synthetic per-token rotary angle tables (cos, sin), float32 [N][rope_dim/2].

    A stand-in for a video model's 3-D position encoding: the rope_dim/2
    channel pairs are split over the (t, y, x) axes of the latent grid (a
    quarter each to t, the rest shared by y and x), pair i of an axis with
    n pairs turning at base^(-i/n) radians per grid step; prefix tokens sit
    at the origin (angle 0).  Only position data: the rotation itself is the
    producer's."""
    half = rope_dim // 2
    nt = half // 4
    ny = (half - nt) // 2
    nx = half - nt - ny
    pos = np.zeros((N, 3), np.float64)
    pos[prefix_len:] = video_positions(N - prefix_len, grid)
    ang = np.zeros((N, half), np.float64)
    col = 0
    for axis, n in enumerate((nt, ny, nx)):
        if n:
            omega = base ** (-np.arange(n, dtype=np.float64) / n)
            ang[:, col:col + n] = pos[:, axis:axis + 1] * omega[None, :]
        col += n
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def producer_inputs(B, H, N, D, dtype="bf16", prefix_len=0, grid=None, rope_dim=None,
                    seed=0) -> dict:
    """Inputs of the fused Q/K producer: pre-norm q and k, v, the two norm
    weights and the rotary tables.

    q, k, v come from ``custom`` (field kind when a grid is given); every
    q / k row is then multiplied by its own scale 10^u, u ~ U(-2, 1.5), so
    that rows span several decades (pre-norm activations) and eps matters
    for the smallest.  gamma_q, gamma_k: 1 + N(0, 0.2^2) per channel (a
    trained norm weight's spread), float32.  rope_dim defaults to d/2
    (partial RoPE); tables from ``rope_tables`` over the grid."""
    kind = "field" if grid is not None else "iid_qk_offset"
    q, k, v = custom(B, H, N, D, dtype, prefix_len, seed, kind=kind, grid=grid)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x51AC])))
    for x in (q, k):
        x *= (10.0 ** rng.uniform(-2.0, 1.5, size=x.shape[:-1] + (1,))).astype(np.float32)
    if dtype == "bf16":
        q, k = round_to_bf16(q), round_to_bf16(k)
    gq = (1.0 + 0.2 * rng.standard_normal(D)).astype(np.float32)
    gk = (1.0 + 0.2 * rng.standard_normal(D)).astype(np.float32)
    r = D // 2 if rope_dim is None else rope_dim
    if grid is None:
        grid = (1, 1, max(1, N - prefix_len))
    cos, sin = rope_tables(N, prefix_len, grid, r)
    return dict(q=q, k=k, v=v, gamma_q=gq, gamma_k=gk, rope_dim=r, cos=cos, sin=sin)
