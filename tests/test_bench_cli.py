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


def test_traffic_constants_follow_the_committed_counter_summary():
    # roofline.traffic comes from the FETCH_SIZE / WRITE_SIZE figures of the
    # committed counter summary: the constants bench.py keeps must be that
    # summary's numbers and hash; with the attention sources as they stand
    # the bench reports that traffic, and once they change it reports null
    # (until the counters are taken again)
    import re
    sys.path.insert(0, ROOT)
    import bench
    c = bench.ATTN_COUNTERS
    with open(os.path.join(ROOT, c["profile"])) as f:
        text = f.read()
    m = re.search(r"roofline\.traffic = \(([\d.]+) x ([\d.]+) \+ ([\d.]+)\) x 1024 = (\d+) bytes",
                  text)
    assert m, "no roofline.traffic line in the summary"
    fetch, fscale, write, total = float(m.group(1)), float(m.group(2)), float(m.group(3)), int(m.group(4))
    assert (fetch, fscale, write) == (c["fetch_kib"], c["fetch_scale"], c["write_kib"])
    assert round((fetch * fscale + write * c["write_scale"]) * 1024) == total
    assert c["sources_sha256"] in "".join(text.split())
    if bench.attn_sources_sha256() == c["sources_sha256"]:
        assert bench.attn_traffic_bytes() == total
    else:
        assert bench.attn_traffic_bytes() is None
