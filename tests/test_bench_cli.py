"""bench.py's command line, on the CPU: more than one GPU is refused with a
message (this operator is measured at one GPU's share), and an unknown
extra leg is rejected before any device work."""
import os
import subprocess
import sys

from conftest import ROOT


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, cwd=ROOT, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "8")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_unknown_leg_is_rejected():
    r = _run("--legs", "dense_sweep,no_such_leg")
    assert r.returncode == 2
    assert "no_such_leg" in r.stderr and r.stdout == ""


def test_legs_listed_in_help():
    r = _run("--help")
    assert r.returncode == 0
    text = "".join(r.stdout.split())      # argparse wraps the list where it likes
    for leg in ("mfma_probe", "dense_sweep", "torch_sdpa", "taylor1", "qk_producer", "long_clip"):
        assert leg in text
