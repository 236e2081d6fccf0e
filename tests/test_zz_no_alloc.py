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


def test_static_scratch_decode_matches_the_workspace_decode():
    cases = [
        # a large call first (shared segments merged through the static array), then a smaller one
        (workloads.make_case(6, 64, 8, 128, 3000, "bf16", "bf16", seq_range=(1, 3000), seed=201), "bf16", 0),
        (workloads.make_case(2, 16, 4, 128, 700, "bf16", "fp8_e4m3", seq_lens=(700, 233), seed=202), "f32", 37),
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
