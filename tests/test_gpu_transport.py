"""GPU parity of the sequence-parallel transport kernels against the oracle
(oracle/transport.py): INT8 and FP8 codes, scales and padding bit for bit,
unpacked bf16 values bit for bit, and a whole exchange among P emulated ranks
on one GPU (the all-to-all itself is a chunk copy here)."""
import numpy as np
import pytest

from oracle import transport as T

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bf16_values(rng, shape):
    """float32 arrays of bf16-representable values with row scales spread
    over several decades, a zero row and quantization ties."""
    x = rng.standard_normal(shape) * np.exp(rng.uniform(-6, 6, shape[:-1] + (1,)))
    x = T.to_bf16(x.astype(np.float32))
    flat = x.reshape(-1, shape[-1])
    flat[0] = 0.0                                        # zero row: scale 0
    flat[1] = 0.0
    flat[1, :4] = [127.0, 63.5, -0.5, 1.5]               # INT8 ties to even (inv = 1)
    if flat.shape[0] > 2:
        flat[2] = 0.0
        flat[2, :5] = [448.0, 1.0625, 1.1875, 1.5 * 2 ** -9, -0.5 * 2 ** -9]  # E4M3 ties (inv = 1)
    return x


def to_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(torch.bfloat16).contiguous()


def to_np_bf16(t):
    import torch
    return t.float().cpu().numpy()


@pytest.mark.parametrize("P,B,H,Ns,d", [(2, 1, 4, 37, 128), (4, 2, 8, 5, 64), (1, 1, 3, 130, 128)])
def test_pack_qkv_int8_bit_exact(P, B, H, Ns, d):
    import torch
    import block_sparse_video_solattn_amd as sa
    rng = np.random.default_rng(11)
    q, k, v = (bf16_values(rng, (B, H, Ns, d)) for _ in range(3))
    send = sa.solattn_pack_qkv_int8(to_dev(q), to_dev(k), to_dev(v), P)
    torch.cuda.synchronize()
    ref = T.pack_qkv_int8(q, k, v, P)
    got = send.cpu().numpy()
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("P,B,Hp,Ns,d", [(2, 1, 2, 37, 128), (3, 2, 1, 7, 64)])
def test_unpack_qkv_int8_bit_exact(P, B, Hp, Ns, d):
    import torch
    import block_sparse_video_solattn_amd as sa
    rng = np.random.default_rng(12)
    # receive buffer as P ranks' pack calls would leave it (oracle-made)
    shards = [[bf16_values(rng, (B, Hp * P, Ns, d)) for _ in range(3)] for _ in range(P)]
    recv = T.all_to_all([T.pack_qkv_int8(*sh, P) for sh in shards])[0]
    got = sa.solattn_unpack_qkv_int8(torch.from_numpy(recv).cuda(), d)
    torch.cuda.synchronize()
    ref = T.unpack_qkv_int8(recv, d)
    for g, r in zip(got, ref):
        assert np.array_equal(to_np_bf16(g).view(np.uint32), r.view(np.uint32))


@pytest.mark.parametrize("P,B,Hp,Ns,d", [(2, 1, 2, 37, 128), (4, 1, 3, 5, 64), (1, 2, 1, 130, 128)])
def test_pack_out_fp8_bit_exact(P, B, Hp, Ns, d):
    import torch
    import block_sparse_video_solattn_amd as sa
    rng = np.random.default_rng(13)
    o = bf16_values(rng, (B, Hp, P * Ns, d))
    send = sa.solattn_pack_out_fp8(to_dev(o), P)
    torch.cuda.synchronize()
    ref = T.pack_out_fp8(o, P)
    got = send.cpu().numpy()
    assert got.shape == ref.shape
    bad = np.argwhere(got != ref)
    assert bad.size == 0, (bad[:5], got[tuple(bad[0])], ref[tuple(bad[0])])


@pytest.mark.parametrize("P,B,Hp,Ns,d", [(2, 1, 2, 37, 128), (3, 1, 1, 7, 64)])
def test_unpack_out_fp8_bit_exact(P, B, Hp, Ns, d):
    import torch
    import block_sparse_video_solattn_amd as sa
    rng = np.random.default_rng(14)
    outs = [bf16_values(rng, (B, Hp, P * Ns, d)) for _ in range(P)]
    recv = T.all_to_all([T.pack_out_fp8(o, P) for o in outs])[1 % P]
    got = sa.solattn_unpack_out_fp8(torch.from_numpy(recv).cuda(), d)
    torch.cuda.synchronize()
    ref = T.unpack_out_fp8(recv, d)
    assert np.array_equal(to_np_bf16(got).view(np.uint32), ref.view(np.uint32))


def test_exchange_round_trip_on_one_gpu():
    # P ranks emulated on one GPU: pack per destination, exchange the chunks,
    # unpack; then the output back the same way.  Every value must equal the
    # oracle's, and the round trip stays within the quantization error.
    import torch
    import block_sparse_video_solattn_amd as sa
    P, B, H, Ns, d = 4, 1, 8, 48, 128
    Hp = H // P
    rng = np.random.default_rng(15)
    full = [bf16_values(rng, (B, H, P * Ns, d)) for _ in range(3)]
    sends = [sa.solattn_pack_qkv_int8(*(to_dev(x[:, :, s * Ns:(s + 1) * Ns]) for x in full), P)
             for s in range(P)]
    recvs = [torch.stack([sends[s][p] for s in range(P)]).contiguous() for p in range(P)]
    got = [sa.solattn_unpack_qkv_int8(recvs[p], d) for p in range(P)]
    torch.cuda.synchronize()
    ref = T.all_to_all([T.pack_qkv_int8(*(x[:, :, s * Ns:(s + 1) * Ns] for x in full), P)
                        for s in range(P)])
    for p in range(P):
        rq = T.unpack_qkv_int8(ref[p], d)
        for g, r, x in zip(got[p], rq, full):
            gv = to_np_bf16(g)
            assert np.array_equal(gv, r)
            xs = x[:, p * Hp:(p + 1) * Hp]
            amax = np.abs(xs).max(-1, keepdims=True)
            assert np.all(np.abs(gv - xs) <= amax / 127 * 0.5 * 1.001 + np.abs(gv) * 2.0 ** -8)
    # output: rank p holds heads p*Hp.. over the full sequence
    o_heads = [to_dev(bf16_values(rng, (B, Hp, P * Ns, d))) for _ in range(P)]
    osend = [sa.solattn_pack_out_fp8(o, P) for o in o_heads]
    orecv = [torch.stack([osend[s][r] for s in range(P)]).contiguous() for r in range(P)]
    oback = [sa.solattn_unpack_out_fp8(orecv[r], d) for r in range(P)]
    torch.cuda.synchronize()
    for r in range(P):
        for p in range(P):
            ref_rows = T.dequant_fp8(*T.quant_fp8(to_np_bf16(o_heads[p])[:, :, r * Ns:(r + 1) * Ns]))
            assert np.array_equal(to_np_bf16(oback[r])[:, p * Hp:(p + 1) * Hp], ref_rows)


def test_transport_at_the_benchmark_shape():
    # one rank's share of the 8-GPU refine step that bench.py times: this
    # rank's 2048-token shard of all 32 heads packed for 8 ranks, a receive
    # buffer unpacked, 4 heads of output packed and unpacked -- every byte and
    # value against the oracle
    import torch
    import block_sparse_video_solattn_amd as sa
    P, B, H, Ns, d = 8, 1, 32, 2048, 128
    Hp = H // P
    rng = np.random.default_rng(16)
    q, k, v = (bf16_values(rng, (B, H, Ns, d)) for _ in range(3))
    send = sa.solattn_pack_qkv_int8(to_dev(q), to_dev(k), to_dev(v), P)
    torch.cuda.synchronize()
    ref = T.pack_qkv_int8(q, k, v, P)
    assert np.array_equal(send.cpu().numpy(), ref)
    del send
    # receive buffer: chunks from two distinct shards, alternating by source
    ref2 = T.pack_qkv_int8(*(bf16_values(rng, (B, H, Ns, d)) for _ in range(3)), P)
    recv = T.all_to_all([ref, ref2] * (P // 2))[0]
    got = sa.solattn_unpack_qkv_int8(torch.from_numpy(recv).cuda(), d)
    torch.cuda.synchronize()
    for g, r in zip(got, T.unpack_qkv_int8(recv, d)):
        assert np.array_equal(to_np_bf16(g).view(np.uint32), r.view(np.uint32))
    del got, recv
    o = bf16_values(rng, (B, Hp, P * Ns, d))
    osend = sa.solattn_pack_out_fp8(to_dev(o), P)
    torch.cuda.synchronize()
    oref = T.pack_out_fp8(o, P)
    assert np.array_equal(osend.cpu().numpy(), oref)
    oref2 = T.pack_out_fp8(bf16_values(rng, (B, Hp, P * Ns, d)), P)
    orecv = T.all_to_all([oref, oref2] * (P // 2))[0]
    oback = sa.solattn_unpack_out_fp8(torch.from_numpy(orecv).cuda(), d)
    torch.cuda.synchronize()
    assert np.array_equal(to_np_bf16(oback).view(np.uint32), T.unpack_out_fp8(orecv, d).view(np.uint32))


@pytest.mark.parametrize("P,B,Hp,Ns,d,mode", [
    (2, 1, 2, 100, 128, "sparse"),      # blocks straddle the two sequence shards, ragged tail
    (3, 2, 1, 64, 64, "sparse"),
    (4, 1, 2, 96, 128, "dense"),
    (2, 1, 3, 130, 128, "topk"),
    (8, 1, 4, 2048, 128, "sparse"),     # one rank of 8 at the refine shape
])
def test_fused_unpack_prepare_matches_unpack_then_prepare(P, B, Hp, Ns, d, mode):
    # the receive side fused with pooling: q_out and the whole workspace bit
    # for bit as unpacking then solattn_prepare_ws, and the attention on them
    # equal to the forward call on the unpacked tensors
    import torch
    import block_sparse_video_solattn_amd as sa
    from block_sparse_video_solattn_amd import inputs
    N = P * Ns
    rng = np.random.default_rng(P * 1000 + Ns)
    if Ns >= 1024:
        grid = (-(-(N - 128) // (24 * 42)), 24, 42)
        q, k, v = inputs.custom(B, P * Hp, Ns, d, "bf16", seed=17)   # this rank's shard, all heads
        shard = [to_dev(x) for x in (q, k, v)]
        send = sa.solattn_pack_qkv_int8(*shard, P)
        recv = torch.stack([send[0]] * P).contiguous()   # every chunk from "rank 0"'s shard
    else:
        recs = []
        for _ in range(P):
            q, k, v = (bf16_values(rng, (B, P * Hp, Ns, d)) for _ in range(3))
            recs.append(sa.solattn_pack_qkv_int8(to_dev(q), to_dev(k), to_dev(v), P)[0])
        recv = torch.stack(recs).contiguous()
    torch.cuda.synchronize()
    wsb = sa.solattn_workspace_bytes(B, Hp, N, d, sa.BF16)
    ws0 = torch.zeros(wsb, dtype=torch.uint8, device="cuda")    # (alignment gaps stay zero)
    ws1 = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    qu, ku, vu = sa.solattn_unpack_qkv_int8(recv, d)
    sa.solattn_prepare_ws(qu, ku, vu, mode, ws0)
    q1 = sa.solattn_prepare_int8_ws(recv, d, mode, ws1)
    torch.cuda.synchronize()
    assert torch.equal(q1, qu)
    assert torch.equal(ws1, ws0)
    tau = {"sparse": 1.25, "dense": 0.0, "topk": 0.2}[mode]
    o0, o1 = torch.empty_like(qu), torch.empty_like(qu)
    sa.solattn_attend_ws(qu, ku, vu, o0, 0, tau, mode, ws0)
    sa.solattn_attend_ws(q1, None, None, o1, 0, tau, mode, ws1)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(o1, o0)
