"""Pins of the oracle's causal prefill to facts outside it.

The prefill is the scaled_dot_product_attention call with is_causal and enable_gqa of "Grouped Query
Attention: Why 8 KV Heads Decide Your Batch Size" (section "Why doesn't GQA speed up my fine-tuned
model?").  Pins: torch's own SDPA in fp64 with the same flags (a library routine), each query position
being the already-pinned decode over the positions up to it, position 0 returning its value row, the
worked example of "Grouped Query Attention (GQA): Efficient Multi-Head Attention" (Worked example 2)
as the last row of a two-token prompt, a pure-Python brute force, and planted mask mistakes.
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import brute, ref
from tests.conftest import GOLDEN

with open(os.path.join(GOLDEN, "worked_example_2.json")) as f:
    WE2 = json.load(f)


def _rand(B, Hq, Hkv, S, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = workloads.cast(torch.randn(B, Hq, S, d, generator=g), dtype)
    k = workloads.cast(torch.randn(B, Hkv, S, d, generator=g), dtype)
    v = workloads.cast(torch.randn(B, Hkv, S, d, generator=g), dtype)
    return q, k, v


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (6, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_sdpa_fp64(Hq, Hkv, causal):
    q, k, v = _rand(2, Hq, Hkv, 29, 16, "f32", seed=Hq * 10 + Hkv)
    got = ref.prefill(q, k, v, 0.3, "f32", causal)
    want = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double(),
                                                            is_causal=causal, enable_gqa=True, scale=0.3)
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_each_position_is_the_decode_over_its_prefix(dtype):
    B, Hq, Hkv, S, d = 2, 8, 4, 21, 8
    q, k, v = _rand(B, Hq, Hkv, S, d, dtype, seed=5)
    out = ref.prefill(q, k, v, 0.4, dtype)
    for i in range(S):
        dec = ref.decode(q[:, :, i].contiguous(), k, v, [i + 1] * B, 0.4, dtype, dtype)
        assert np.array_equal(out[:, :, i], dec), i


def test_position_zero_returns_its_value_row():
    q, k, v = _rand(1, 4, 2, 9, 8, "f32", seed=6)
    out = ref.prefill(q, k, v, 0.7, "f32")
    for h in range(4):
        np.testing.assert_allclose(out[0, h, 0], v[0, h // 2, 0].numpy(), rtol=0, atol=1e-12)


def test_worked_example_2_as_a_two_token_prompt():
    # the example's query per head is the second prompt position; its keys and values are positions 0, 1
    q = torch.zeros(1, 4, 2, 2)
    q[0, :, 1] = torch.tensor(WE2["q"], dtype=torch.float32)
    q[0, :, 0] = torch.tensor([[5.0, -3.0]] * 4)         # anything: position 0 sees only itself
    k = torch.tensor(WE2["k"], dtype=torch.float32)[None]
    v = torch.tensor(WE2["v"], dtype=torch.float32)[None]
    out = ref.prefill(q, k, v, WE2["scale"], "f32")
    np.testing.assert_allclose(out[0, :, 1], np.array(WE2["out"]), rtol=0, atol=WE2["tolerance"])
    for h in range(4):
        np.testing.assert_allclose(out[0, h, 0], v[0, h // 2, 0].numpy(), rtol=0, atol=1e-12)


def test_brute_force_agrees_on_tiny_shapes():
    for seed, (B, Hq, Hkv, S, d) in enumerate([(1, 4, 2, 5, 3), (2, 2, 1, 4, 2), (1, 3, 3, 6, 4)]):
        for causal in (True, False):
            q, k, v = _rand(B, Hq, Hkv, S, d, "bf16", seed=20 + seed)
            got = ref.prefill(q, k, v, 0.9, "bf16", causal)
            want = np.array(brute.prefill(ref.raw(q, "bf16").tolist(), ref.raw(k, "bf16").tolist(),
                                          ref.raw(v, "bf16").tolist(), 0.9, "bf16", causal))
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_sampled_rows_equal_full_result():
    q, k, v = _rand(2, 8, 2, 40, 16, "bf16", seed=7)
    full = ref.prefill(q, k, v, 0.25, "bf16")
    rows = [(0, 0, 0), (1, 7, 39), (0, 3, 17), (1, 4, 1)]
    part = ref.prefill(q, k, v, 0.25, "bf16", rows=rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.array_equal(part[n], full[b, h, i])


# --------------------------------------------------------------------------- planted mistakes
def _numpy_prefill(q, k, v, scale, mistake=None):
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            j = h % Hkv if mistake == "interleaved_heads" else h // G
            for i in range(S):
                n = {"no_diagonal": i, "one_ahead": i + 2, "no_mask": S}.get(mistake, i + 1)
                n = max(1, min(n, S))
                s = k[b, j, :n] @ q[b, h, i] * scale
                p = np.exp(s - s.max())
                out[b, h, i] = v[b, j, :n].T @ (p / p.sum())
    return out


def _prefill_pins_pass(fn):
    q, k, v = _rand(1, 4, 2, 12, 8, "f32", seed=8)
    want = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double(),
                                                            is_causal=True, enable_gqa=True, scale=0.5)
    if not np.allclose(fn(q.numpy(), k.numpy(), v.numpy(), 0.5), want.numpy(), atol=1e-9):
        return False
    qq = torch.zeros(1, 4, 2, 2)
    qq[0, :, 1] = torch.tensor(WE2["q"])
    kk = torch.tensor(WE2["k"])[None]
    vv = torch.tensor(WE2["v"])[None]
    return np.allclose(fn(qq.numpy(), kk.numpy(), vv.numpy(), WE2["scale"])[0, :, 1], WE2["out"],
                       atol=WE2["tolerance"])


def test_prefill_pins_accept_correct_definition():
    assert _prefill_pins_pass(_numpy_prefill)
    assert _prefill_pins_pass(lambda q, k, v, s: ref.prefill(np.float32(q), np.float32(k), np.float32(v), s, "f32"))


@pytest.mark.parametrize("mistake", ["interleaved_heads", "no_diagonal", "one_ahead", "no_mask"])
def test_prefill_pins_reject_planted_mistake(mistake):
    assert not _prefill_pins_pass(lambda *a: _numpy_prefill(*a, mistake=mistake))


@pytest.mark.parametrize("scale", [-0.3, 0.0])
def test_nonpositive_scales(scale):
    """A negative scale is |scale| on -q (negation is exact), pinned to torch's SDPA in that form (its
    fp64 math path returns NaN for a negative or zero scale under the causal mask); a zero scale
    weighs every visible key the same, so each row is the mean of the visible value rows."""
    q, k, v = _rand(1, 4, 2, 17, 8, "f32", seed=9)
    for causal in (True, False):
        got = ref.prefill(q, k, v, scale, "f32", causal)
        if scale < 0:
            want = torch.nn.functional.scaled_dot_product_attention(-q.double(), k.double(), v.double(),
                                                                    is_causal=causal, enable_gqa=True,
                                                                    scale=-scale)
            np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-13)
        else:
            vv = v.double().repeat_interleave(2, dim=1)
            n = torch.arange(1, 18, dtype=torch.float64)[:, None]
            mean = vv.cumsum(2) / n if causal else vv.mean(2, keepdim=True).expand_as(vv)
            np.testing.assert_allclose(got, mean.numpy(), rtol=0, atol=1e-14)
