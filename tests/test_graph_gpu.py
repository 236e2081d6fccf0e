"""The decode entry points under HIP graph capture (torch.cuda.CUDAGraph) and on concurrent
streams, through the C ABI.

A serving loop captures its per-layer launches once and replays them.  The library only enqueues
kernels on the caller's stream (no allocation, no memset, no synchronisation) and every call leaves
its workspace counters at zero, so a captured call must replay to the same result as the eager one,
bit for bit, on every replay, also with other work between the replays and with new inputs copied
into the captured buffers.
"""
import pytest
import torch

import grouped_query_attention_04_amd as gqa
import workloads
from oracle import ref
from tests.test_parity_gpu import DEV, compare, say

pytestmark = pytest.mark.gpu


def _bitwise(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _ws(shape):
    return gqa.new_workspace(shape, DEV)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_captured_decode_replays_bitwise(kv):
    say(f"graph capture: decode, kv={kv}")
    B, Hq, Hkv, d, L = 6, 32, 8, 128, 1000
    c = workloads.make_case(B, Hq, Hkv, d, L, "bf16", kv, seq_range=(1, L), seed=120)
    q, k, v, sl = c["q"].to(DEV), c["k"].to(DEV), c["v"].to(DEV), c["seq_lens"].to(DEV)
    shape = gqa.make_shape(B, Hq, Hkv, L, d, gqa.BF16, gqa._CODE[k.dtype], gqa.BF16)
    ws = _ws(shape)
    eager = gqa.decode(q, k, v, sl, c["scale"], workspace=ws)
    out = torch.empty_like(eager)
    # a second, unrelated decode with its own workspace runs eagerly between the replays
    c2 = workloads.make_case(2, 8, 2, 64, 300, "bf16", "bf16", seq_lens=(300, 77), seed=121)
    d2 = {n: c2[n].to(DEV) for n in ("q", "k", "v", "seq_lens")}
    ws2 = _ws(gqa.make_shape(2, 8, 2, 300, 64, gqa.BF16, gqa.BF16, gqa.BF16))
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gqa.decode(q, k, v, sl, c["scale"], out=out, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        other = gqa.decode(d2["q"], d2["k"], d2["v"], d2["seq_lens"], c2["scale"], workspace=ws2)
        torch.cuda.synchronize()
        assert _bitwise(out, eager), f"replay {rep} differs from the eager result"
    compare(other, ref.decode(c2["q"], c2["k"], c2["v"], c2["seq_lens"].numpy(), c2["scale"], "bf16", "bf16"),
            "bf16", "eager call between replays")

    # new inputs copied into the captured buffers: the replay reads them
    c3 = workloads.make_case(B, Hq, Hkv, d, L, "bf16", kv, seq_range=(1, L), seed=122)
    q.copy_(c3["q"].to(DEV))
    sl.copy_(c3["seq_lens"].to(DEV))
    g.replay()
    torch.cuda.synchronize()
    want = ref.decode(c3["q"], c["k"], c["v"], c3["seq_lens"].numpy(), c["scale"], "bf16", kv)
    compare(out, want, kv, "replay on new inputs")


def test_captured_fused_append_paged_replays_bitwise():
    say("graph capture: fused append + paged decode")
    B, Hq, Hkv, d, L, bs = 4, 64, 8, 128, 512, 16
    c = workloads.make_case(B, Hq, Hkv, d, L, "bf16", "bf16", seq_lens=(512, 300, 17, 1), seed=123)
    pg = workloads.paginate(c, bs, seed=16, spare_pages=3)
    g_ = torch.Generator().manual_seed(124)
    kn = torch.randn(B, Hkv, d, generator=g_).to(torch.bfloat16).to(DEV)
    vn = torch.randn(B, Hkv, d, generator=g_).to(torch.bfloat16).to(DEV)
    q, sl, table = c["q"].to(DEV), c["seq_lens"].to(DEV), pg["block_table"].to(DEV)
    kp, vp = pg["k_pages"].to(DEV), pg["v_pages"].to(DEV)
    shape = gqa.make_paged_shape(B, Hq, Hkv, d, bs, table.shape[1], pg["num_blocks"], gqa.BF16, gqa.BF16, gqa.BF16)
    ws = _ws(shape)
    eager = gqa.decode_append_paged(q, kn, vn, kp, vp, table, sl, c["scale"], workspace=ws)
    kp_e, vp_e = kp.clone(), vp.clone()
    out = torch.empty_like(eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gqa.decode_append_paged(q, kn, vn, kp, vp, table, sl, c["scale"], out=out, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert _bitwise(out, eager), f"replay {rep} differs from the eager result"
        assert _bitwise(kp, kp_e) and _bitwise(vp, vp_e), f"replay {rep} changed the pages differently"


def test_two_streams_with_their_own_workspaces():
    """Calls that overlap in time on two streams, each with its own workspace (the binding keeps
    one per stream), both match the oracle; the library never synchronises."""
    say("two streams")
    cases = [workloads.make_case(8, 32, 8, 128, 2000, "bf16", "bf16", seq_range=(1, 2000), seed=130 + i)
             for i in range(2)]
    dev = [{n: c[n].to(DEV) for n in ("q", "k", "v", "seq_lens")} for c in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = [[], []]
    for rep in range(3):
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                outs[i].append(gqa.decode(dev[i]["q"], dev[i]["k"], dev[i]["v"], dev[i]["seq_lens"],
                                          cases[i]["scale"], out_dtype=torch.float32))
    torch.cuda.synchronize()
    for i in (0, 1):
        want = ref.decode(cases[i]["q"], cases[i]["k"], cases[i]["v"], cases[i]["seq_lens"].numpy(),
                          cases[i]["scale"], "bf16", "bf16")
        compare(outs[i][0], want, "bf16", f"stream {i}")
        assert all(_bitwise(o, outs[i][0]) for o in outs[i][1:]), f"stream {i}: repeated calls differ"
