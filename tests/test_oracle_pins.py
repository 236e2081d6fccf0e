"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks the oracle against something the pages or mathematics fix: printed worked-example
values, printed KV-byte figures, library routines (torch's fp8/bf16 decoding, its SDPA with
``enable_gqa``), closed forms, invariants and an independent pure-Python brute force.  The last block
plants plausible mistakes in small re-implementations and shows that the pins reject each of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, ref
from tests.conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


# --------------------------------------------------------------------------- worked example 2
WE2 = _load("worked_example_2.json")


def _we2_inputs():
    q = _f32(WE2["q"])[None]             # [1, 4, 2]
    k = _f32(WE2["k"])[None]             # [1, 2, 2, 2]
    v = _f32(WE2["v"])[None]
    return q, k, v, np.array([2], np.int32), WE2["scale"]


def test_worked_example_2_outputs():
    q, k, v, sl, scale = _we2_inputs()
    out = ref.decode(q, k, v, sl, scale)
    np.testing.assert_allclose(out[0], np.array(WE2["out"]), rtol=0, atol=WE2["tolerance"])


def test_worked_example_2_weights_and_scores():
    q, k, v, sl, scale = _we2_inputs()
    for h in range(4):
        w = ref.weights(q, k, v, sl, scale, 0, h)
        np.testing.assert_allclose(w, WE2["weights"][h], rtol=0, atol=WE2["tolerance"])
    # head 1's scores are (q . k_t) / sqrt(2): recover them from the weights' log-ratio
    w = ref.weights(q, k, v, sl, scale, 0, 0)
    assert abs(math.log(w[0] / w[1]) - (WE2["head1_scores"][0] - WE2["head1_scores"][1])) < 1e-4


def test_worked_example_2_brute_agrees():
    q, k, v, sl, scale = _we2_inputs()
    out = np.array(brute.decode(q.tolist(), k.tolist(), v.tolist(), sl.tolist(), scale))
    np.testing.assert_allclose(out[0], np.array(WE2["out"]), rtol=0, atol=WE2["tolerance"])


# --------------------------------------------------------------------------- KV-bytes formula
KVB = _load("kv_bytes.json")


@pytest.mark.parametrize("row", KVB["per_token"], ids=lambda r: f"{r[0]}L-{r[1]}kv-{r[3]}B")
def test_kv_bytes_per_token_printed(row):
    layers, kvh, hd, db, printed, _src = row
    assert ref.kv_bytes_per_token(layers, kvh, hd, db) == printed


def test_kv_cache_total_printed():
    c = KVB["cache_total"]
    for kvh, gb in c["entries"]:
        per_tok = ref.kv_bytes_per_token(c["layers"], kvh, c["head_dim"], c["dtype_bytes"])
        assert round(per_tok * c["seq_len"] * c["batch"] / 1e9, 3) == gb


def test_kv_reduction_and_savings_printed():
    r = KVB["reduction"]
    a = ref.kv_bytes_per_token(r["layers"], r["from"], r["head_dim"], r["dtype_bytes"])
    b = ref.kv_bytes_per_token(r["layers"], r["to"], r["head_dim"], r["dtype_bytes"])
    assert a / b == r["factor"]
    s = KVB["savings_kib"]
    for hi, lo, kib in s["steps"]:
        d = (ref.kv_bytes_per_token(s["layers"], hi, s["head_dim"], s["dtype_bytes"])
             - ref.kv_bytes_per_token(s["layers"], lo, s["head_dim"], s["dtype_bytes"]))
        assert d == kib * 1024


# --------------------------------------------------------------------------- decoders vs torch
def test_fp8_decoder_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib_vals = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        mine = ref.fp8_e4m3_to_double(c)
        py = brute.fp8_e4m3_code_to_float(c)
        if math.isnan(lib_vals[c]):
            assert math.isnan(mine) and math.isnan(py), c
        else:
            assert mine == lib_vals[c] == py, c


def test_bf16_decoder_matches_torch_all_patterns():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    lib_vals = bits.view(torch.bfloat16).to(torch.float64).numpy()
    for b in list(range(0, 65536, 97)) + [0x0000, 0x8000, 0x0001, 0x7F80, 0xFF80, 0x7FC0, 0x3F80]:
        mine = ref.bf16_to_double(b)
        if math.isnan(lib_vals[b]):
            assert math.isnan(mine)
        else:
            assert mine == lib_vals[b] == brute.bf16_bits_to_float(b), hex(b)


# --------------------------------------------------------------------------- brute force, tiny shapes
def _rand_raw(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    t = torch.from_numpy(x)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return t.clamp(-4, 4).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("dtypes", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8_e4m3")])
def test_brute_force_matches_oracle_on_every_tiny_shape(dtypes):
    qd, kd = dtypes
    rng = np.random.default_rng(7)
    checked = 0
    for B, Hkv, G, d, L in itertools.product((1, 2), (1, 2), (1, 2, 3), (1, 2, 3), (1, 2, 3, 4)):
        Hq = Hkv * G
        q = _rand_raw(rng, (B, Hq, d), qd)
        k = _rand_raw(rng, (B, Hkv, L, d), kd)
        v = _rand_raw(rng, (B, Hkv, L, d), kd)
        scale = 1.0 / math.sqrt(d)
        for sl in itertools.product(range(L + 1), repeat=B):
            o = ref.decode(q, k, v, sl, scale, qd, kd, 0.75, 1.25)
            b = np.array(brute.decode(q.tolist(), k.tolist(), v.tolist(), sl, scale, qd, kd, 0.75,
                                      1.25))
            np.testing.assert_allclose(o, b.reshape(o.shape), rtol=1e-12, atol=1e-13)
            checked += 1
    assert checked > 1000


# --------------------------------------------------------------------------- library cross-checks
def _case_f64(seed, B=3, Hq=8, Hkv=2, d=16, L=20, seq_lens=(20, 0, 7)):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, Hkv, L, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, Hkv, L, d, generator=g, dtype=torch.float64)
    return q, k, v, np.array(seq_lens, np.int32)


def _repeat_kv(x, n_rep):
    # expand the KV-head axis over the group, then fold it into the head axis (a copy, not a view)
    b, hkv, s, d = x.shape
    if n_rep == 1:
        return x
    return x[:, :, None, :, :].expand(b, hkv, n_rep, s, d).reshape(b, hkv * n_rep, s, d)


def _mha_per_head(q, k, v, seq_lens, scale):
    # ordinary multi-head attention, one query head against its own K/V head (torch fp64)
    B, H, d = q.shape
    out = torch.zeros(B, H, d, dtype=torch.float64)
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        s = (k[b, :, :n, :] @ q[b, :, :, None])[..., 0] * scale      # [H, n]
        p = torch.softmax(s, dim=-1)
        out[b] = (p[:, None, :] @ v[b, :, :n, :])[:, 0, :]
    return out.numpy()


@pytest.mark.parametrize("Hkv", [1, 2, 4, 8])
def test_repeat_kv_then_mha_matches_oracle(Hkv):
    q, k, v, sl = _case_f64(11 + Hkv, Hkv=Hkv)
    G = 8 // Hkv
    scale = 0.3
    got = ref.decode(q.float().numpy(), k.float().numpy(), v.float().numpy(), sl, scale)
    # the oracle reads fp32 storage, so the library path runs on the same fp32-rounded values
    want = _mha_per_head(q.float().double(), _repeat_kv(k.float().double(), G),
                         _repeat_kv(v.float().double(), G), sl, scale)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv", [(64, 1), (128, 2), (48, 1)])
def test_repeat_kv_then_mha_matches_oracle_large_groups(Hq, Hkv):
    """Groups of 48 and 64 query heads per KV head (the multi-query end of a 64-head model)."""
    q, k, v, sl = _case_f64(31 + Hq, Hq=Hq, Hkv=Hkv)
    G = Hq // Hkv
    got = ref.decode(q.float().numpy(), k.float().numpy(), v.float().numpy(), sl, 0.3)
    want = _mha_per_head(q.float().double(), _repeat_kv(k.float().double(), G),
                         _repeat_kv(v.float().double(), G), sl, 0.3)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_group_size_one_is_plain_mha():
    q, k, v, sl = _case_f64(5, Hq=6, Hkv=6)
    q, k, v = (x.float().double() for x in (q, k, v))
    want = _mha_per_head(q, k, v, sl, 0.25)
    got = ref.decode(q.float().numpy(), k.float().numpy(), v.float().numpy(), sl, 0.25)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_sdpa_enable_gqa_matches_oracle():
    F = torch.nn.functional
    q, k, v, sl = _case_f64(3, B=4, Hq=12, Hkv=3, d=8, L=17, seq_lens=(17, 1, 9, 4))
    q, k, v = (x.float().double() for x in (q, k, v))
    mask = (torch.arange(17)[None, :] < torch.from_numpy(sl).long()[:, None])[:, None, None, :]
    want = F.scaled_dot_product_attention(q[:, :, None, :], k, v, attn_mask=mask, scale=0.4,
                                          enable_gqa=True)[:, :, 0, :].numpy()
    got = ref.decode(q.float().numpy(), k.float().numpy(), v.float().numpy(), sl, 0.4)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------- closed forms
def test_weights_sum_to_one_and_are_positive():
    q, k, v, sl = _case_f64(9, seq_lens=(20, 3, 11))
    qf, kf, vf = (x.float().numpy() for x in (q, k, v))
    for b in range(3):
        for h in range(8):
            w = ref.weights(qf, kf, vf, sl, 0.7, b, h)
            assert len(w) == sl[b]
            assert abs(w.sum() - 1.0) < 1e-12 and (w > 0).all()


def test_constant_v_per_kv_head_gives_group_index():
    # softmax weights sum to one, so a V that is constant per (b, kv head) comes out unchanged;
    # the value j + 10 b also fixes the head-to-group map and the batch index.
    B, Hq, Hkv, d, L = 3, 12, 3, 5, 9
    rng = np.random.default_rng(1)
    q = _f32(rng.standard_normal((B, Hq, d)) * 3)
    k = _f32(rng.standard_normal((B, Hkv, L, d)) * 3)
    v = np.zeros((B, Hkv, L, d), np.float32)
    for b in range(B):
        for j in range(Hkv):
            v[b, j] = j + 10 * b
    sl = np.array([9, 4, 1], np.int32)
    out = ref.decode(q, k, v, sl, 1.3)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(out[b, h], h // G + 10 * b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("how", ["zero_query", "zero_scale"])
def test_uniform_weights_give_mean_of_prefix(how):
    B, Hq, Hkv, d, L = 2, 4, 2, 3, 10
    rng = np.random.default_rng(2)
    q = _f32(rng.standard_normal((B, Hq, d)))
    k = _f32(rng.standard_normal((B, Hkv, L, d)))
    v = np.zeros((B, Hkv, L, d), np.float32)
    v[:] = np.arange(L, dtype=np.float32)[None, None, :, None]   # v_t = t
    scale = 0.9
    if how == "zero_query":
        q[:] = 0
    else:
        scale = 0.0
    sl = np.array([10, 7], np.int32)
    out = ref.decode(q, k, v, sl, scale)
    for b in range(B):
        np.testing.assert_allclose(out[b], (sl[b] - 1) / 2.0, rtol=0, atol=1e-12)


def test_single_token_returns_its_value_row():
    rng = np.random.default_rng(3)
    q = _f32(rng.standard_normal((2, 6, 4)))
    k = _f32(rng.standard_normal((2, 3, 5, 4)))
    v = _f32(rng.standard_normal((2, 3, 5, 4)))
    out = ref.decode(q, k, v, [1, 1], 0.5)
    for b in range(2):
        for h in range(6):
            np.testing.assert_array_equal(out[b, h], v[b, h // 2, 0].astype(np.float64))


def test_needle_inside_prefix_and_decoy_outside():
    # one key far above the rest at t = n-1 wins; a still larger decoy at t = n must be ignored
    B, Hq, Hkv, d, L, n = 1, 4, 1, 8, 12, 9
    rng = np.random.default_rng(4)
    q = _f32(rng.standard_normal((B, Hq, d)))
    q[0, :] = q[0, 0]                                # all heads ask the same question
    k = _f32(rng.standard_normal((B, Hkv, L, d)) * 0.1)
    v = _f32(rng.standard_normal((B, Hkv, L, d)))
    unit = q[0, 0] / np.linalg.norm(q[0, 0])
    k[0, 0, n - 1] = unit * 40.0
    k[0, 0, n] = unit * 80.0                         # decoy, outside the valid prefix
    out = ref.decode(q, k, v, [n], 1.0)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], v[0, 0, n - 1], rtol=0, atol=1e-6)


def test_zero_length_row_is_zero_and_out_of_range_rejected():
    rng = np.random.default_rng(5)
    q = _f32(rng.standard_normal((2, 2, 3)))
    k = _f32(rng.standard_normal((2, 1, 4, 3)))
    out = ref.decode(q, k, k, [0, 2], 1.0)
    assert (out[0] == 0).all() and (out[1] != 0).any()
    with pytest.raises(ValueError):
        ref.decode(q, k, k, [5, 2], 1.0)
    with pytest.raises(ValueError):
        ref.decode(q, k, k, [-1, 2], 1.0)


def test_token_permutation_and_padding_invariance():
    rng = np.random.default_rng(6)
    B, Hq, Hkv, d, L = 2, 6, 2, 7, 15
    q = _f32(rng.standard_normal((B, Hq, d)))
    k = _f32(rng.standard_normal((B, Hkv, L, d)))
    v = _f32(rng.standard_normal((B, Hkv, L, d)))
    sl = np.array([15, 10], np.int32)
    base = ref.decode(q, k, v, sl, 0.6)
    perm = rng.permutation(10)
    k2, v2 = k.copy(), v.copy()
    k2[1, :, :10] = k[1][:, perm]
    v2[1, :, :10] = v[1][:, perm]
    k2[1, :, 10:] = np.nan                           # padding is never read
    v2[1, :, 10:] = np.nan
    got = ref.decode(q, k2, v2, sl, 0.6)
    np.testing.assert_allclose(got, base, rtol=1e-12, atol=1e-14)


def test_descales_act_as_score_and_output_scales():
    rng = np.random.default_rng(8)
    q = _f32(rng.standard_normal((1, 4, 6)))
    k = _rand_raw(rng, (1, 2, 9, 6), "fp8_e4m3")
    v = _rand_raw(rng, (1, 2, 9, 6), "fp8_e4m3")
    base = ref.decode(q, k, v, [9], 0.5, "f32", "fp8_e4m3")
    got = ref.decode(q, k, v, [9], 0.25, "f32", "fp8_e4m3", k_descale=2.0, v_descale=3.0)
    np.testing.assert_allclose(got, 3.0 * base, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------- planted mistakes
def _numpy_decode(q, k, v, sl, scale, mistake=None):
    """A small float64 re-implementation in which one plausible mistake can be planted."""
    B, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        n = int(sl[b]) + (1 if mistake == "off_by_one_mask" else 0)
        n = min(n, L)
        for h in range(Hq):
            j = h % Hkv if mistake == "interleaved_heads" else h // G
            kk = k[b, j, :n].astype(np.float64)
            vv = v[b, j, :n].astype(np.float64)
            if mistake == "k_rows_reversed":
                kk = kk[::-1]
            s = kk @ q[b, h].astype(np.float64)
            if mistake != "no_scale":
                s = s * scale
            if mistake == "no_max_shift_wrong_sign":
                s = -s
            if n == 0:
                continue
            p = np.exp(s - s.max())
            if mistake != "unnormalised":
                p = p / p.sum()
            out[b, h] = (vv.T @ p) if mistake != "value_from_keys" else (kk.T @ p)
    return out


MISTAKES = ["interleaved_heads", "off_by_one_mask", "k_rows_reversed", "no_scale",
            "no_max_shift_wrong_sign", "unnormalised", "value_from_keys"]


def _pins_pass(fn):
    """Run the worked example, constant-V and needle pins against a decode function."""
    q, k, v, sl, scale = _we2_inputs()
    if not np.allclose(fn(q, k, v, sl, scale)[0], np.array(WE2["out"]), atol=WE2["tolerance"]):
        return False
    B, Hq, Hkv, d, L = 2, 8, 2, 4, 6
    rng = np.random.default_rng(12)
    q = _f32(rng.standard_normal((B, Hq, d)))
    k = _f32(rng.standard_normal((B, Hkv, L, d)))
    v = np.zeros((B, Hkv, L, d), np.float32)
    for b in range(B):
        for j in range(Hkv):
            v[b, j] = j + 10 * b
    sl = np.array([6, 3], np.int32)
    want = np.array([[[h // 4 + 10 * b] * d for h in range(Hq)] for b in range(B)], float)
    if not np.allclose(fn(q, k, v, sl, 0.5), want, atol=1e-9):
        return False
    n = 5
    q = _f32(rng.standard_normal((1, 2, d)))
    q[0, 1] = q[0, 0]
    k = _f32(rng.standard_normal((1, 1, 8, d)) * 0.1)
    v = _f32(rng.standard_normal((1, 1, 8, d)))
    unit = q[0, 0] / np.linalg.norm(q[0, 0])
    k[0, 0, n - 1] = unit * 40
    k[0, 0, n] = unit * 80
    return np.allclose(fn(q, k, v, [n], 1.0)[0, 0], v[0, 0, n - 1], atol=1e-6)


def test_pins_accept_the_correct_reimplementation():
    assert _pins_pass(lambda *a: _numpy_decode(*a))
    assert _pins_pass(lambda q, k, v, sl, s: ref.decode(q, k, v, sl, s))


@pytest.mark.parametrize("mistake", MISTAKES)
def test_pins_reject_planted_mistake(mistake):
    assert not _pins_pass(lambda *a: _numpy_decode(*a, mistake=mistake))
