"""GPU parity of the prefill kernel (gqa_prefill) against the fp64 oracle, through the C ABI.

bf16 inputs with fp32 accumulation; the weights are rounded to bf16 before P V, as in decode, so the
bf16 gates apply (1e-2 absolute, and relative to the reference's scale).
"""
import time

import numpy as np
import pytest
import torch

import grouped_query_attention_04_amd as gqa
import workloads
from oracle import ref
from tests.test_parity_gpu import DEV, compare, say

pytestmark = pytest.mark.gpu


def run(case, causal=True, out_dtype=torch.bfloat16):
    out = gqa.prefill(case["q"].to(DEV), case["k"].to(DEV), case["v"].to(DEV), case["scale"],
                      out_dtype=out_dtype, causal=causal)
    torch.cuda.synchronize()
    return out


SMALL = [
    # (B, Hq, Hkv, S, d)
    (1, 4, 1, 70, 64),       # G = 4, ragged last query block
    (2, 8, 2, 129, 128),     # G = 4
    (1, 2, 2, 300, 64),      # G = 1: 256 positions per workgroup, waves on different positions
    (2, 4, 2, 200, 128),     # G = 2
    (1, 16, 2, 100, 128),    # G = 8
    (1, 16, 1, 33, 64),      # G = 16
    (1, 32, 1, 60, 128),     # G = 32: a 16-row tile spans two heads
    (1, 8, 8, 1, 128),       # a one-token prompt
    (1, 40, 8, 90, 128),     # G = 5: 51 positions per workgroup, one padding row
    (2, 12, 4, 100, 64),     # G = 3: 85 positions, one padding row
    (1, 7, 1, 300, 128),     # G = 7: 36 positions, four padding rows
    (1, 24, 1, 70, 128),     # G = 24: 10 positions, sixteen padding rows (one whole tile)
    (1, 48, 1, 37, 64),      # G = 48: 5 positions, a wave of padding rows
    (1, 64, 1, 20, 128),     # G = 64: 4 positions
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: "B{}Hq{}Hkv{}S{}d{}".format(*c))
def test_prefill_small_parity(cfg, causal):
    B, Hq, Hkv, S, d = cfg
    say(f"prefill parity {cfg} causal={causal}")
    case = workloads.make_prefill_case(B, Hq, Hkv, d, S, seed=hash(cfg) % 10000)
    want = ref.prefill(case["q"], case["k"], case["v"], case["scale"], "bf16", causal)
    compare(run(case, causal), want, "bf16", "bf16 out")
    compare(run(case, causal, torch.float32), want, "bf16", "f32 out")


def test_prefill_first_position_is_its_value_row_and_last_is_the_decode():
    say("prefill: position 0 and position S-1")
    B, Hq, Hkv, S, d = 2, 16, 4, 300, 128
    case = workloads.make_prefill_case(B, Hq, Hkv, d, S, seed=91)
    out = run(case, out_dtype=torch.float32).cpu()
    G = Hq // Hkv
    for h in range(Hq):
        assert torch.allclose(out[:, h, 0], case["v"][:, h // G, 0].float(), atol=0, rtol=0)
    dec = gqa.decode(case["q"][:, :, S - 1].contiguous().to(DEV), case["k"].to(DEV), case["v"].to(DEV),
                     torch.full((B,), S, dtype=torch.int32, device=DEV), case["scale"],
                     out_dtype=torch.float32).cpu()
    assert (out[:, :, S - 1] - dec).abs().max() < 2e-3


def test_prefill_is_deterministic():
    case = workloads.make_prefill_case(1, 32, 8, 128, 777, seed=92)
    a, b = run(case), run(case)
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["prefill-8b", "prefill-40b", "prefill-70b"])
def test_prefill_workload_parity(name):
    """Full-size prefill workloads against the oracle (rows cut over the host's CPUs).  prefill-8b
    and prefill-40b: every (b, h, i) row.  prefill-70b (1.1 TFLOP of fp64 oracle work in all): every
    position of the first and the last query group (the 8 heads of KV heads 0 and 7, a quarter of
    the rows) and 2000 random rows of the other groups."""
    w = workloads.PREFILL_WORKLOADS[name]
    say(f"prefill workload {name}: {w.name}")
    case = workloads.make_prefill(name)
    got = run(case).cpu()
    t0 = time.perf_counter()
    if name != "prefill-70b":
        want = ref.prefill(case["q"], case["k"], case["v"], case["scale"], "bf16", True, rows="all",
                           threads=ref.host_threads())
        label = f"{name} all {w.B * w.Hq * w.S} rows"
    else:
        rng = np.random.default_rng(93)
        heads = list(range(w.G)) + list(range(w.Hq - w.G, w.Hq))
        rows = [(b, h, i) for b in range(w.B) for h in heads for i in range(w.S)]
        rows += [(int(rng.integers(w.B)), int(rng.integers(w.G, w.Hq - w.G)), int(rng.integers(w.S)))
                 for _ in range(2000)]
        want = ref.prefill(case["q"], case["k"], case["v"], case["scale"], "bf16", True, rows=rows,
                           threads=ref.host_threads())
        got = torch.stack([got[b, h, i] for b, h, i in rows])
        label = f"{name} {len(rows)} rows"
    say(f"  oracle: {time.perf_counter() - t0:.1f} s on {ref.host_threads()} threads")
    compare(got, want, "bf16", label)


@pytest.mark.parametrize("scale", [-0.11, -1.0, 0.0, -0.0])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_nonpositive_scales(scale, causal):
    """Any finite scale is a valid call: a negative one flips the order of the scores, and zero
    makes every visible key weigh the same (the mean of the visible value rows)."""
    say(f"prefill scale {scale} causal={causal}")
    B, Hq, Hkv, S, d = 2, 8, 2, 150, 128
    case = workloads.make_prefill_case(B, Hq, Hkv, d, S, seed=93)
    case["scale"] = scale
    got = run(case, causal, torch.float32)
    want = ref.prefill(case["q"], case["k"], case["v"], scale, "bf16", causal)
    compare(got, want, "bf16", f"scale {scale}")
    if scale == 0.0:
        v = case["v"].double()
        G = Hq // Hkv
        n = torch.arange(1, S + 1, dtype=torch.float64)[:, None]
        mean = v.cumsum(2) / n if causal else v.mean(2, keepdim=True).expand_as(v)
        mean = mean.repeat_interleave(G, dim=1)
        # the weights are exactly 1 (bf16), so only the fp32 accumulation order separates the two
        assert (got.cpu().double() - mean).abs().max() < 1e-5


def _random_prefill(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8, 16, 32]))
        d = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 3))
        S = int(rng.integers(1, 400))
        causal = bool(rng.integers(0, 2))
        out.append((B, G * Hkv, Hkv, S, d, causal))
    return out


def _random_prefill_any_group(n, seed):
    """Group sizes 1..64 that need not divide 256 (padding rows in every workgroup)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 3]))
        G = int(rng.integers(1, 65))
        d = int(rng.choice([64, 128]))
        S = int(rng.integers(1, 300))
        out.append((int(rng.integers(1, 3)), G * Hkv, Hkv, S, d, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("cfg", _random_prefill(12, 13) + _random_prefill_any_group(12, 14),
                         ids=lambda c: "B{}Hq{}Hkv{}S{}d{}-causal{}".format(*c))
def test_prefill_random_shapes(cfg):
    """Seeded random prompt shapes (every supported group size, ragged query and key blocks)."""
    B, Hq, Hkv, S, d, causal = cfg
    say(f"prefill random shape {cfg}")
    case = workloads.make_prefill_case(B, Hq, Hkv, d, S, seed=(131 * B + 17 * Hq + 7 * Hkv + 3 * S + d) % 100000)
    want = ref.prefill(case["q"], case["k"], case["v"], case["scale"], "bf16", causal)
    compare(run(case, causal, torch.float32), want, "bf16", f"prefill random {cfg}")
