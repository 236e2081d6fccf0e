"""gqa_decode_static: the decode entry point that allocates nothing (its workspace is a fixed array
inside the library, one per GPU), checked through the C ABI against gqa_decode on the same inputs:
bitwise equal outputs (the same kernels) and the oracle's gates, on two calls in a row, the second
with a smaller input, then a shape whose workspace exceeds the array."""
import ctypes

import pytest
import torch

import grouped_query_attention_04_amd as gqa
import workloads
from tests.test_parity_gpu import DEV, TORCH, compare, oracle_full, say

pytestmark = pytest.mark.gpu


def _static(case, out_dtype, wg=0):
    d = {n: case[n].to(DEV) for n in ("q", "k", "v", "seq_lens")}
    B, Hq, dd = case["q"].shape
    _, Hkv, L, _ = case["k"].shape
    code = {"f32": gqa.F32, "bf16": gqa.BF16, "fp8_e4m3": gqa.FP8_E4M3}
    shape = gqa.make_shape(B, Hq, Hkv, L, dd, code[case["q_dtype"]], code[case["kv_dtype"]], code[out_dtype],
                           case["k_descale"], case["v_descale"], wg)
    out = torch.full((B, Hq, dd), float("nan"), dtype=TORCH[out_dtype], device=DEV)
    rc = gqa.lib.gqa_decode_static(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                                   d["seq_lens"].data_ptr(), float(case["scale"]), out.data_ptr(),
                                   ctypes.byref(shape), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return rc, out, d


def _static_call(d, case, out, shape):
    return gqa.lib.gqa_decode_static(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                                     d["seq_lens"].data_ptr(), float(case["scale"]), out.data_ptr(),
                                     ctypes.byref(shape), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_static_scratch_under_graph_capture():
    """A call captured into a graph (possibly the device's first, whose set-up then goes into the
    graph too), an eager call made before the graph is ever replayed, and three replays with eager
    calls between them: every result equals gqa_decode's, bitwise."""
    say("static scratch under graph capture")
    case = workloads.make_case(4, 32, 8, 128, 1500, "bf16", "bf16", seq_range=(1, 1500), seed=203)
    other = workloads.make_case(2, 16, 2, 128, 900, "bf16", "fp8_e4m3", seq_lens=(900, 17), seed=204)
    d = {n: case[n].to(DEV) for n in ("q", "k", "v", "seq_lens")}
    d2 = {n: other[n].to(DEV) for n in ("q", "k", "v", "seq_lens")}
    shape = gqa.make_shape(4, 32, 8, 1500, 128, gqa.BF16, gqa.BF16, gqa.BF16)
    shape2 = gqa.make_shape(2, 16, 2, 900, 128, gqa.BF16, gqa.FP8_E4M3, gqa.F32)
    want = gqa.decode(d["q"], d["k"], d["v"], d["seq_lens"], case["scale"])
    want2 = gqa.decode(d2["q"], d2["k"], d2["v"], d2["seq_lens"], other["scale"], out_dtype=torch.float32)
    out = torch.full_like(want, float("nan"))
    out2 = torch.full_like(want2, float("nan"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert _static_call(d, case, out, shape) == 0
    torch.cuda.synchronize()
    assert _static_call(d2, other, out2, shape2) == 0      # eager, before any replay
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.uint8), want2.view(torch.uint8)), "eager call before the first replay"
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), want.view(torch.uint8)), f"replay {rep}"
        out2.fill_(float("nan"))
        assert _static_call(d2, other, out2, shape2) == 0
        torch.cuda.synchronize()
        assert torch.equal(out2.view(torch.uint8), want2.view(torch.uint8)), f"eager call after replay {rep}"


def test_static_scratch_decode_matches_the_workspace_decode():
    cases = [
        # a large call first (shared segments merged through the static array), then a smaller one
        (workloads.make_case(6, 64, 8, 128, 3000, "bf16", "bf16", seq_range=(1, 3000), seed=201), "bf16", 0),
        (workloads.make_case(2, 16, 4, 128, 700, "bf16", "fp8_e4m3", seq_lens=(700, 233), seed=202), "f32", 37),
        # 64 query heads on one KV head: run as four 16-head sub-groups, a workspace of their size
        (workloads.make_case(4, 64, 1, 128, 800, "bf16", "bf16", seq_lens=(800, 1, 0, 513), seed=205), "bf16", 0),
    ]
    for i, (case, od, wg) in enumerate(cases):
        say(f"static scratch call {i}: B{case['B']} Hq{case['Hq']} Hkv{case['Hkv']} kv={case['kv_dtype']}")
        rc, got, d = _static(case, od, wg)
        assert rc == 0, gqa.status_string(rc)
        ref_out = gqa.decode(d["q"], d["k"], d["v"], d["seq_lens"], case["scale"], out_dtype=TORCH[od],
                             num_workgroups=wg)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.uint8), ref_out.view(torch.uint8)), "differs from gqa_decode"
        compare(got, oracle_full(case), case["kv_dtype"], f"static call {i}")


def test_static_scratch_rejects_shapes_beyond_its_size():
    # 4096 workgroups x 2 slots x 32 rows x (128 + 2) floats is well past the array
    shape = gqa.make_shape(4, 64, 2, 1000, 128, gqa.BF16, gqa.BF16, gqa.BF16, num_workgroups=4096)
    assert gqa.workspace_bytes(shape) > (24 << 20)
    p = ctypes.c_void_p(1 << 20)   # never dereferenced: the size check fails first
    rc = gqa.lib.gqa_decode_static(p, p, p, p, 0.1, p, ctypes.byref(shape), None)
    assert rc == 3, gqa.status_string(rc)   # GQA_ERR_WORKSPACE
