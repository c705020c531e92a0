"""Host-side checks of the Python binding and the parity helpers, run without
a GPU: tensors outside GPU memory are refused before any call reaches the
library (a host pointer handed to a kernel would fault the device), and the
error helper of the parity tests cannot pass a NaN or inf output."""
import math

import numpy as np
import pytest

from conftest import ensure_library
from gpu_util import TOL_BF16_ABS, max_abs_diff, out_error


@pytest.fixture(scope="module")
def sa():
    ensure_library()
    import block_sparse_video_solattn_amd as m
    return m


def test_cpu_tensors_are_rejected_before_any_call(sa):
    import torch
    q = torch.zeros((1, 1, 128, 64), dtype=torch.bfloat16)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    calls = [
        lambda: sa.solattn_forward(q, q, q, None, 0, 1.0, "sparse"),
        lambda: sa.solattn_forward_ws(q, q, q, q.clone(), 0, 1.0, "sparse", ws),
        lambda: sa.solattn_prepare_ws(q, q, q, "sparse", ws),
        lambda: sa.solattn_attend_ws(q, q, q, q.clone(), 0, 1.0, "sparse", ws),
        lambda: sa.solattn_forward_debug(q, q, q, None, 0, 1.0, "sparse"),
        lambda: sa.solattn_pool(q, q, q),
        lambda: sa.solattn_route(q, q, q, 0, 1.0),
        lambda: sa.solattn_probe_mfma_bf16(torch.zeros(64), 1, 1),
        lambda: sa.solattn_pack_qkv_int8(q, q, q, 1),
        lambda: sa.solattn_unpack_qkv_int8(torch.zeros((1, 1, 1, 128, 3, 80), dtype=torch.uint8), 64),
        lambda: sa.solattn_pack_out_fp8(q, 1),
        lambda: sa.solattn_unpack_out_fp8(torch.zeros((1, 1, 1, 128, 80), dtype=torch.uint8), 64),
        lambda: sa.solattn_qknorm_rope(q, q, None, None, 1e-6, 0),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="GPU tensor"):
            call()


def test_error_helper_fails_non_finite_outputs():
    o = np.zeros((4, 8))
    g = o.copy()
    assert out_error(g, o) == (0.0, 0.0)
    for bad in (np.nan, np.inf, -np.inf):
        g = o.copy()
        g[2, 3] = bad
        ab, rel = out_error(g, o)
        assert ab == math.inf and rel == math.inf
        # the callers fold errors with max(); inf survives it, NaN would not
        worst = 0.0
        worst = max(worst, ab)
        assert not worst <= TOL_BF16_ABS
        assert max_abs_diff(g, o) == math.inf
    # rows the oracle did not produce (NaN there) are still skipped
    o2 = o.copy()
    o2[1] = np.nan
    g2 = o.copy()
    g2[1] = 5.0
    assert out_error(g2, o2)[0] == 0.0
