import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

LIB = os.path.join(ROOT, "block_sparse_video_solattn_amd", "libsolattn.so")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def ensure_library():
    """Build libsolattn.so when it is missing (hipcc cross-compiles without a GPU)."""
    if not os.path.exists(LIB):
        from block_sparse_video_solattn_amd import build
        build.build()
    return LIB
