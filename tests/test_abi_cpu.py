"""C ABI checks that need no GPU: the library loads, exports every function
include/solattn.h declares, and rejects bad arguments on the host before any
device call."""
import ctypes
import glob
import math
import os
import re

import pytest

from conftest import ROOT, ensure_library

HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(solattn_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    ensure_library()
    from block_sparse_video_solattn_amd import _binding
    return _binding


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    raw = ctypes.CDLL(lib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(lib.EXPORTS)


def test_version_and_strerror(lib):
    assert "gfx950" in lib.solattn_version()
    assert lib.solattn_strerror(0) == "ok"
    assert lib.solattn_strerror(1) == "invalid argument"
    assert lib.solattn_strerror(99) == "unknown error code"


def test_workspace_bytes(lib):
    ws = lib.solattn_workspace_bytes(1, 32, 16384, 128, 1)
    # pooled fp32 (3 + transposed) + bf16 pooled operands + value tiles
    assert ws >= 32 * 16384 * 128 * 2
    assert lib.solattn_workspace_bytes(1, 1, 1024, 64, 0) > 0
    assert lib.solattn_workspace_bytes(1, 1, 1024, 96, 1) == 0


A = 0x10000  # fake, 16-byte aligned "device" addresses: never dereferenced


def fwd(lib, q=A, k=A + 0x100000, v=A + 0x200000, out=A + 0x300000, B=1, H=1, N=1024, d=64,
        prefix=0, tau=1.0, mode=1, dtype=1):
    return lib.raw_call("solattn_forward", q, k, v, out, B, H, N, d, prefix, ctypes.c_float(tau),
                        mode, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(out=0), 1), (dict(B=0), 1), (dict(H=-1), 1), (dict(N=0), 1),
    (dict(d=96), 1), (dict(prefix=-1), 1), (dict(prefix=1025), 1), (dict(tau=float("nan")), 1),
    (dict(mode=3), 1), (dict(dtype=3), 1), (dict(q=A + 8), 1), (dict(out=A + 0x100), 1),
    (dict(mode=2, tau=0.0), 1), (dict(mode=2, tau=1.5), 1), (dict(mode=2, tau=-math.inf), 1),
    (dict(mode=0x10), 1), (dict(mode=0x20), 1), (dict(mode=0x22, tau=0.5), 1), (dict(mode=0x81), 1),
    (dict(mode=0x40), 1), (dict(mode=0x42, tau=0.5), 1), (dict(mode=0x41, dtype=0), 2),
    (dict(mode=0x13, tau=0.5), 1), (dict(N=64 * 4096 + 1), 2),
])
def test_forward_rejects_before_device(lib, kw, code):
    assert fwd(lib, **kw) == code
    assert lib.solattn_last_error() != ""


def test_other_entry_points_validate(lib):
    f = ctypes.c_float
    assert lib.raw_call("solattn_forward_ws", A, A + 0x100000, A + 0x200000, A + 0x300000,
                        1, 1, 1024, 64, 0, f(1.0), 1, 1, None, 0, None) == 1  # NULL ws
    assert lib.raw_call("solattn_forward_ws", A, A + 0x100000, A + 0x200000, A + 0x300000,
                        1, 1, 1024, 64, 0, f(1.0), 1, 1, A + 0x400000, 16, None) == 1  # too small
    assert lib.raw_call("solattn_prepare_ws", None, A, A, 1, 1, 64, 64, 1, 1, A, 1 << 30, None) == 1
    assert lib.raw_call("solattn_attend_ws", A, A, A, A + 0x1000000, 1, 1, 64, 128, 0, f(math.nan),
                        1, 1, A, 1 << 30, None) == 1
    assert lib.raw_call("solattn_forward_debug", A, A, A, None, 1, 1, 64, 64, 0, f(1.0), 1, 1,
                        None, None, None, None) == 1
    assert lib.raw_call("solattn_pool", A, A, A, None, None, None, 1, 1, 64, 32, 1, None) == 1
    assert lib.raw_call("solattn_route", A, A, A, 1, 1, 64, 64, 65, f(1.0), 1, None, None, None,
                        None) == 1
    assert lib.raw_call("solattn_route_ws", A, 1, 1, 64, 64, 0, f(1.0), 1, None, 1 << 30, None,
                        None, None, None) == 1                       # NULL ws
    assert lib.raw_call("solattn_route_ws", A, 1, 1, 64, 64, 0, f(1.0), 1, A, 16, None, None,
                        None, None) == 1                             # too small
    # the routing plan: bf16 SPARSE / TOPK only, workspace checked on the host
    plan = lambda mode, dtype, ws=A + 0x1000000, nbytes=1 << 30, tau=1.0: lib.raw_call(
        "solattn_plan_ws", A, 1, 1, 1024, 64, 0, f(tau), mode, dtype, ws, nbytes, None)
    attend_plan = lambda mode, dtype, out=A + 0x800000, ws=A + 0x1000000, nbytes=1 << 30: (
        lib.raw_call("solattn_attend_plan_ws", A, out, 1, 1, 1024, 64, mode, dtype, ws, nbytes,
                     None))
    assert plan(1, 1, ws=None) == 1 and plan(1, 1, nbytes=16) == 1
    assert plan(0, 1) == 2 and plan(1, 0) == 2 and plan(0x41, 1) == 2   # dense, fp32, taylor1
    assert plan(2, 1, tau=0.0) == 1 and plan(2, 1, tau=2.0) == 1         # topk kept fraction
    assert plan(1, 1, tau=math.nan) == 1
    assert attend_plan(0, 1) == 2 and attend_plan(1, 0) == 2 and attend_plan(0x41, 1) == 2
    assert attend_plan(1, 1, out=None) == 1 and attend_plan(1, 1, ws=None) == 1
    assert attend_plan(1, 1, out=A) == 1                                 # out overlaps q


def test_noalloc_rejects_oversize_shapes_on_host(lib):
    # the fixed workspace of solattn_forward_noalloc: a shape that needs more
    # is refused before any device call (fake addresses, never dereferenced)
    f = ctypes.c_float
    call = lambda H, N: lib.raw_call("solattn_forward_noalloc", A, A + 0x10000000, A + 0x20000000,
                                     A + 0x30000000, 1, H, N, 128, 0, f(1.0), 1, 1, None)
    assert lib.solattn_workspace_bytes(1, 32, 16384, 128, 1) > lib.NOALLOC_SCRATCH_BYTES
    assert call(32, 16384) == lib.EUNSUPPORTED
    assert "workspace" in lib.solattn_last_error()
    assert call(0, 16384) == lib.EINVAL


def test_import_without_library_fails_loudly(tmp_path):
    # a copy of the Python package without the shared library refuses to import
    import shutil
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "block_sparse_video_solattn_amd")
    dst = tmp_path / "block_sparse_video_solattn_amd"
    dst.mkdir()
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            shutil.copy(os.path.join(pkg, f), dst / f)
    code = "import block_sparse_video_solattn_amd as m; m.solattn_forward"
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=str(tmp_path))
    assert r.returncode != 0 and "not built" in r.stderr


def test_probe_rejects_bad_arguments_on_host(lib):
    probe = lambda sink, waves, iters: lib.raw_call("solattn_probe_mfma_bf16", sink, waves, iters, None)
    assert probe(None, 1024, 16) == lib.EINVAL
    assert "sink" in lib.solattn_last_error()
    assert probe(A + 4, 1024, 16) == lib.EINVAL  # misaligned
    assert probe(A, 0, 16) == lib.EINVAL
    assert probe(A, (1 << 20) + 1, 16) == lib.EINVAL
    assert probe(A, 1024, 0) == lib.EINVAL
    assert "iters" in lib.solattn_last_error()


def test_transport_record_bytes(lib):
    assert lib.solattn_transport_record_bytes(128) == 144
    assert lib.solattn_transport_record_bytes(64) == 80
    assert lib.solattn_transport_record_bytes(96) == 0


def test_transport_entry_points_validate(lib):
    # every rejection happens on the host, before any device call
    X, Y, Z, S = A, A + 0x1000000, A + 0x2000000, A + 0x3000000
    pack = lambda q=X, k=Y, v=Z, B=1, H=4, Ns=64, d=128, P=2, send=S: lib.raw_call(
        "solattn_pack_qkv_int8", q, k, v, B, H, Ns, d, P, send, None)
    assert pack(q=None) == 1
    assert pack(send=S + 8) == 1
    assert pack(d=96) == 1
    assert pack(P=0) == 1
    assert pack(H=6, P=4) == 1
    assert pack(send=X + 0x100) == 1          # output overlaps q
    assert pack(B=1 << 40) == 2
    unpack = lambda B=1, Hp=2, Ns=64, d=128, P=2, q=X, k=Y, v=Z: lib.raw_call(
        "solattn_unpack_qkv_int8", S, B, Hp, Ns, d, P, q, k, v, None)
    assert unpack(k=X) == 1                   # two outputs overlap
    assert unpack(Hp=0) == 1
    assert lib.raw_call("solattn_pack_out_fp8", X, 1, 2, 64, 64, 2, None, None) == 1
    assert lib.raw_call("solattn_unpack_out_fp8", S, 1, 2, 64, 32, 2, X, None) == 1
    assert lib.solattn_last_error() != ""


def test_producer_entry_points_validate(lib):
    # every rejection happens on the host, before any device call
    f = ctypes.c_float
    X, Y, Z, QO, KO, G, C, S, W = (A, A + 0x1000000, A + 0x2000000, A + 0x3000000,
                                   A + 0x4000000, A + 0x5000000, A + 0x6000000, A + 0x7000000,
                                   A + 0x8000000)

    def alone(q=X, k=Y, gq=G, gk=G, eps=1e-6, r=64, c=C, s=S, qo=QO, ko=KO, N=1024, d=128,
              dtype=1):
        return lib.raw_call("solattn_qknorm_rope", q, k, gq, gk, f(eps), r, c, s, qo, ko,
                            1, 2, N, d, dtype, None)

    def fused(q=X, k=Y, v=Z, eps=1e-6, r=64, c=C, s=S, qo=QO, ko=KO, mode=1, dtype=1,
              ws=W, ws_bytes=1 << 30):
        return lib.raw_call("solattn_prepare_qknorm_rope_ws", q, k, v, G, G, f(eps), r, c, s,
                            qo, ko, 1, 2, 1024, 128, mode, dtype, ws, ws_bytes, None)

    for bad in (dict(eps=0.0), dict(eps=-1e-6), dict(eps=math.inf), dict(eps=math.nan),
                dict(r=63), dict(r=130), dict(r=-2), dict(c=None), dict(s=None),
                dict(qo=None), dict(ko=None), dict(qo=QO + 8), dict(gq=G + 2),
                dict(c=C + 1), dict(qo=X + 0x100), dict(ko=QO + 0x100), dict(ko=G - 0x100),
                dict(d=96), dict(N=0), dict(dtype=2), dict(q=None)):
        assert alone(**bad) == lib.EINVAL, bad
        assert lib.solattn_last_error() != ""
    # no rotation: tables may be NULL; NULL weights mean ones (rejections
    # above came from the argument named, the rest is accepted up to the
    # first device call, which these fake addresses never reach)
    for bad in (dict(ws=None), dict(ws_bytes=16), dict(eps=0.0), dict(mode=5),
                dict(ko=None, dtype=0), dict(v=None), dict(qo=Z + 0x100)):
        assert fused(**bad) == lib.EINVAL, bad
    # bf16 attend reads neither k nor v: NULL accepted past validation, so
    # probe only the rejections that remain
    assert lib.raw_call("solattn_attend_ws", None, None, None, A + 0x1000000, 1, 1, 64, 128, 0,
                        f(1.0), 1, 1, A, 1 << 30, None) == lib.EINVAL
    assert lib.raw_call("solattn_attend_ws", A, None, None, A + 0x1000000, 1, 1, 64, 128, 0,
                        f(1.0), 1, 0, A, 1 << 30, None) == lib.EINVAL   # fp32 needs k, v


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "solattn.h"
#include "solattn_probe.h"
#include "solattn_producer.h"
#include "solattn_transport.h"

int main(void) {
    /* every call below is rejected on the host before any device call */
    int rc = solattn_forward(NULL, NULL, NULL, NULL, 1, 1, 64, 64, 0, 1.0f, SOLATTN_SPARSE,
                             SOLATTN_BF16, NULL);
    if (rc != SOLATTN_EINVAL || strlen(solattn_last_error()) == 0) return 1;
    rc = solattn_qknorm_rope(NULL, NULL, NULL, NULL, 1e-6f, 0, NULL, NULL, NULL, NULL, 1, 1, 64,
                             64, SOLATTN_BF16, NULL);
    if (rc != SOLATTN_EINVAL) return 2;
    if (solattn_transport_record_bytes(128) != 144) return 3;
    if (solattn_workspace_bytes(1, 1, 64, 64, SOLATTN_F32) == 0) return 4;
    if (solattn_probe_mfma_bf16(NULL, 1, 1, NULL) != SOLATTN_EINVAL) return 5;
    printf("%s|%s\n", solattn_version(), solattn_strerror(SOLATTN_EUNSUPPORTED));
    return 0;
}
"""


def test_headers_compile_as_c_and_link(lib, tmp_path):
    # the public headers are plain C: a C99 program includes all of them,
    # links against the library and calls its host-side checks
    import subprocess
    src = tmp_path / "use_abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "use_abi"
    libdir = os.path.dirname(lib.LIB_PATH)
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                           "-L", libdir, "-lsolattn", "-Wl,-rpath," + libdir])
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, (r.returncode, r.stderr)
    version, err = r.stdout.strip().split("|")
    assert "gfx950" in version and err == lib.solattn_strerror(2)
