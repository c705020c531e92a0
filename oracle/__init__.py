"""Sol-Attn CPU oracle (fp64) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The GPU library never loads it
and shares no code with it.  The arithmetic lives in ``solattn_oracle.c``
(plain fp64 loops, OpenMP over query blocks); this module builds it with gcc
and marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "solattn_oracle.c")
_LIB = os.path.join(_HERE, "libsolattn_oracle.so")
_lib = None

DENSE, SPARSE, TOPK = 0, 1, 2
# routing variants, added to SPARSE (both) or TOPK (PREFIX_ROWS): prefix query
# blocks keep every key block; threshold statistics over the video key blocks
PREFIX_ROWS, VIDEO_STATS = 0x10, 0x20
BLOCK = 64


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP; no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.solattn_oracle_head.argtypes = [P, P, P, I64, I64, I64, ctypes.c_double,
                                            ctypes.c_int, P, P, I64, P, P, P, P, P, P, P,
                                            ctypes.c_int]
        lib.solattn_oracle_head.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def nblocks(N: int) -> int:
    return (N + BLOCK - 1) // BLOCK


def head(q: np.ndarray, k: np.ndarray, v: np.ndarray, prefix_len: int, tau: float,
         mode: int = SPARSE, mask_override: Optional[np.ndarray] = None,
         qblocks: Optional[Sequence[int]] = None, want_out: bool = True,
         threads: int = 0) -> dict:
    """Run the oracle on one (b, h) slice.  q, k, v: [N, d] (any float dtype,
    converted exactly to float64).  Returns a dict with ``out`` ([N, d], NaN
    in rows not produced), ``mask`` ([Nb, Nb] uint8), ``score``, ``thr`` and
    the pooled means ``qbar``, ``kbar``, ``vbar``.
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    N, d = q.shape
    nb = nblocks(N)
    out = np.full((N, d), np.nan) if want_out else None
    mask = np.zeros((nb, nb), np.uint8)
    score = np.full((nb, nb), np.nan)
    thr = np.full(nb, np.nan)
    qbar = np.empty((nb, d))
    kbar = np.empty((nb, d))
    vbar = np.empty((nb, d))
    mo = None
    if mask_override is not None:
        mo = np.ascontiguousarray(mask_override, dtype=np.uint8)
        assert mo.shape == (nb, nb)
    ql = None
    nq = 0
    if qblocks is not None:
        ql = np.ascontiguousarray(np.asarray(qblocks, dtype=np.int64))
        nq = len(ql)
    rc = lib.solattn_oracle_head(_ptr(q), _ptr(k), _ptr(v), N, d, prefix_len, float(tau),
                                 int(mode), _ptr(mo), _ptr(ql), nq, _ptr(out), _ptr(mask),
                                 _ptr(score), _ptr(thr), _ptr(qbar), _ptr(kbar), _ptr(vbar),
                                 int(threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
    return dict(out=out, mask=mask, score=score, thr=thr, qbar=qbar, kbar=kbar, vbar=vbar)


def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, prefix_len: int, tau: float,
            mode: int = SPARSE, mask_override: Optional[np.ndarray] = None,
            want_out: bool = True, threads: int = 0) -> dict:
    """Whole tensors [B, H, N, d]; results stacked as [B, H, ...]."""
    B, H, N, d = q.shape
    res = []
    for b in range(B):
        for h in range(H):
            mo = None if mask_override is None else mask_override[b, h]
            res.append(head(q[b, h], k[b, h], v[b, h], prefix_len, tau, mode, mo,
                            want_out=want_out, threads=threads))
    out = {}
    for key in res[0]:
        if res[0][key] is None:
            out[key] = None
            continue
        arr = np.stack([r[key] for r in res])
        out[key] = arr.reshape((B, H) + arr.shape[1:])
    return out
