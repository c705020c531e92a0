"""GPU tests of the planned attention launch: the routing kernel writes each
query block's keep bits and tile count, the order kernel a per-(head, XCD)
longest-first dispatch order, and the attention kernel follows both.  Its
output must equal, bit for bit, the launch that routes inside the attention
kernel (every query block's arithmetic is the same; only the order differs),
and on a row of more than 64 mask words it is held to the oracle.  Outputs
start as NaN, so a query block the order skipped or ran twice in place of
another shows."""
import numpy as np
import pytest

import oracle
from block_sparse_video_solattn_amd import inputs
from gpu_util import TOL_BF16_ABS, block_rows, device_tensors, mask_compare, out_error

pytestmark = pytest.mark.gpu

PLAN_MIN_ITEMS = 2048   # launches from this many query blocks on are planned


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_video_solattn_amd  # noqa: F401  (raises when the library is missing)


def _nan_like(t):
    import torch
    return torch.full_like(t, float("nan"))


@pytest.mark.parametrize("H,N,d,prefix,tau,mode", [
    (2, 3000, 128, 128, 1.25, "sparse"),
    (3, 64 * 20 + 7, 64, 64, 1.0, "sparse"),
    (2, 3000, 128, 128, 0.25, "topk"),
    (2, 3000, 128, 256, 1.25, "sparse+prefix_rows"),
    (2, 3000, 128, 128, 1.0, "sparse+video_stats"),
    (1, 1000, 128, 0, float("inf"), "sparse"),
    (1, 1000, 128, 0, -float("inf"), "sparse"),
])
def test_plan_stages_match_fused_launch(H, N, d, prefix, tau, mode):
    # below the planning size solattn_attend_ws routes inside the attention
    # kernel; the two plan stages on the same workspace give the same bits
    import torch
    import block_sparse_video_solattn_amd as sa
    q, k, v = inputs.custom(1, H, N, d, "bf16", prefix_len=prefix, seed=120, kind="field",
                            grid=(4, 24, 40))
    qd, kd, vd = device_tensors(q, k, v, "bf16")
    assert H * ((N + 63) // 64) < PLAN_MIN_ITEMS
    ws = torch.empty(sa.solattn_workspace_bytes(1, H, N, d, sa.BF16), dtype=torch.uint8,
                     device="cuda")
    fused = _nan_like(qd)
    sa.solattn_prepare_ws(qd, kd, vd, mode, ws)
    sa.solattn_attend_ws(qd, kd, vd, fused, prefix, tau, mode, ws)
    planned = _nan_like(qd)
    sa.solattn_plan_ws(qd, prefix, tau, mode, ws)
    sa.solattn_attend_plan_ws(qd, planned, mode, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(fused.float()).all()
    assert torch.equal(fused, planned)


@pytest.mark.parametrize("N,mode,tau", [(8192, "sparse", 1.25), (8192 - 40, "sparse", 1.0),
                                        (8192, "topk", 0.1)])
def test_planned_launch_matches_per_head_launches(N, mode, tau):
    # 16 heads of 128 query blocks: the whole launch is planned, each head
    # alone (128 blocks) routes inside the attention kernel
    import torch
    import block_sparse_video_solattn_amd as sa
    H, d, prefix = 16, 128, 256
    q, k, v = inputs.custom(1, H, N, d, "bf16", prefix_len=prefix, seed=121, kind="field",
                            grid=(4, 32, 64))
    qd, kd, vd = device_tensors(q, k, v, "bf16")
    assert H * ((N + 63) // 64) >= PLAN_MIN_ITEMS > (N + 63) // 64
    whole = _nan_like(qd)
    sa.solattn_forward(qd, kd, vd, whole, prefix, tau, mode)
    torch.cuda.synchronize()
    for h in range(H):
        qh, kh, vh = (t[:, h:h + 1].contiguous() for t in (qd, kd, vd))
        one = sa.solattn_forward(qh, kh, vh, _nan_like(qh), prefix, tau, mode)
        torch.cuda.synchronize()
        assert torch.equal(one[0, 0], whole[0, h]), h


def test_planned_rows_of_more_than_64_mask_words():
    # 2101 key blocks (66 mask words per row, ragged 17-token tail): the
    # planned kernel reads the words past the first 64 in a second pass;
    # masks on every row, outputs on sampled query blocks on both sides of
    # block 2048, against the oracle with the GPU's mask
    import torch
    import block_sparse_video_solattn_amd as sa
    B, H, N, d, prefix, tau = 1, 1, 64 * 2100 + 17, 128, 512, 1.25
    q, k, v = inputs.custom(B, H, N, d, "bf16", prefix_len=prefix, seed=122, kind="field",
                            grid=(16, 90, 96))
    qd, kd, vd = device_tensors(q, k, v, "bf16")
    nb = (N + 63) // 64
    assert nb >= PLAN_MIN_ITEMS and (nb + 31) // 32 > 64
    out, words, _, _ = sa.solattn_forward_debug(qd, kd, vd, _nan_like(qd), prefix, tau, "sparse",
                                                want_scores=False)
    torch.cuda.synchronize()
    gmask = sa.unpack_mask(words, nb)
    otau = float(np.float32(tau))
    r = oracle.head(q[0, 0], k[0, 0], v[0, 0], prefix, otau, want_out=False)
    mask_compare(gmask, r, 0, 0)
    blocks = [0, 7, 1024, 2047, 2048, 2080, nb - 1]
    ro = oracle.head(q[0, 0], k[0, 0], v[0, 0], prefix, otau,
                     mask_override=gmask[0, 0].astype(np.uint8), qblocks=blocks)
    g = out.float().cpu().numpy()[0, 0].astype(np.float64)
    ab, _ = out_error(g, ro["out"], block_rows(blocks, N))
    assert ab <= TOL_BF16_ABS, ab
    assert torch.isfinite(out.float()).all()


def test_plan_entry_points_reject_unplannable_modes():
    import torch
    import block_sparse_video_solattn_amd as sa
    q, k, v = inputs.custom(1, 1, 256, 64, "bf16", seed=123)
    qd, _, _ = device_tensors(q, k, v, "bf16")
    ws = torch.empty(sa.solattn_workspace_bytes(1, 1, 256, 64, sa.BF16), dtype=torch.uint8,
                     device="cuda")
    for mode in ("dense", "sparse+taylor1"):
        with pytest.raises(sa.SolAttnError) as e:
            sa.solattn_plan_ws(qd, 0, 1.0, mode, ws)
        assert e.value.code == sa.EUNSUPPORTED
        with pytest.raises(sa.SolAttnError) as e:
            sa.solattn_attend_plan_ws(qd, torch.empty_like(qd), mode, ws)
        assert e.value.code == sa.EUNSUPPORTED
    qf = qd.float()
    wsf = torch.empty(sa.solattn_workspace_bytes(1, 1, 256, 64, sa.F32), dtype=torch.uint8,
                      device="cuda")
    with pytest.raises(sa.SolAttnError) as e:
        sa.solattn_plan_ws(qf, 0, 1.0, "sparse", wsf)
    assert e.value.code == sa.EUNSUPPORTED
