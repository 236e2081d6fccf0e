"""Pins of the oracle's cache append and storage encoders to facts outside the oracle.

An fp8 cache stores 8-bit values with per-tensor scales ("Grouped-Query Attention: How Sharing KV
Heads Shrinks Inference Memory", section "FP8 KV cache: the other factor of two"); the format is OCP
e4m3fn.  The encoders are pinned by: every code encoding back to itself, midpoints between neighbouring
codes going to the even one, torch's own float8_e4m3fn and bfloat16 casts wherever those are defined
the same way, exact power-of-two descales, saturation at the largest finite value, and an independent
pure-Python encoder over every bf16 input.  The append is pinned by what it may and may not touch, by
paging commuting with it, and by a decode that must find the row it wrote.
"""
import math
import struct

import numpy as np
import pytest
import torch

import workloads
from oracle import brute, ref


def _f32_from_bits(bits):
    return struct.unpack("<f", struct.pack("<I", bits))[0]


# --------------------------------------------------------------------------- fp8 e4m3fn encoder
def test_fp8_every_code_encodes_to_itself():
    for c in range(256):
        v = ref.fp8_e4m3_to_double(c)
        if math.isnan(v):
            assert ref.encode_fp8_e4m3(v) == (0x7F | (c & 0x80)) or ref.encode_fp8_e4m3(v) in (0x7F, 0xFF)
            continue
        assert ref.encode_fp8_e4m3(v) == c, hex(c)


def test_fp8_midpoints_go_to_the_even_code():
    for c in range(0, 0x7E):                       # positive finite neighbours (c, c + 1)
        lo, hi = ref.fp8_e4m3_to_double(c), ref.fp8_e4m3_to_double(c + 1)
        mid = (lo + hi) / 2                        # exact in binary32 for every pair
        want = c if c % 2 == 0 else c + 1
        assert ref.encode_fp8_e4m3(mid) == want, (hex(c), mid)
        assert ref.encode_fp8_e4m3(-mid) == want | 0x80
        # just off the midpoint, the nearer neighbour wins
        assert ref.encode_fp8_e4m3(np.nextafter(np.float32(mid), np.float32(0))) == c
        assert ref.encode_fp8_e4m3(np.nextafter(np.float32(mid), np.float32(1000))) == c + 1


def test_fp8_matches_torch_cast_within_range():
    rng = np.random.default_rng(50)
    xs = np.concatenate([rng.standard_normal(4000) * 50, rng.uniform(-464, 464, 4000),
                         rng.standard_normal(2000) * 1e-3,
                         np.array([0.0, -0.0, 448.0, -448.0, 464.0, -464.0, 2.0 ** -9, 2.0 ** -10])])
    xs = xs.astype(np.float32)
    t = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([ref.encode_fp8_e4m3(x) for x in xs], dtype=np.uint8)
    assert np.array_equal(mine, t)


def test_fp8_saturates_instead_of_overflowing():
    # torch's cast overflows to NaN past 464; the cache encoder keeps the largest finite value
    for x in (465.0, 1e4, 3.0e38, math.inf):
        assert ref.encode_fp8_e4m3(x) == 0x7E
        assert ref.encode_fp8_e4m3(-x) == 0xFE
    assert ref.encode_fp8_e4m3(math.nan) & 0x7F == 0x7F


@pytest.mark.parametrize("k", [-3, -1, 1, 2, 5])
def test_fp8_power_of_two_descale_is_an_exact_rescale(k):
    s = 2.0 ** k
    rng = np.random.default_rng(51 + k)
    for x in rng.uniform(-300, 300, 500).astype(np.float32):
        x = float(x)
        if abs(x) < 2.0 ** -6 * max(1.0, s) * 4:     # keep clear of the subnormal range
            continue
        assert ref.encode_fp8_e4m3(x * s, s) == ref.encode_fp8_e4m3(x), (x, s)


def test_fp8_and_bf16_encoders_agree_with_brute_force_on_every_bf16_input():
    for bits in range(0, 1 << 16, 1):
        x = _f32_from_bits(bits << 16)
        for s in (1.0, 0.375):
            assert brute.encode_fp8_e4m3(x, s) == ref.encode_fp8_e4m3(x, s), (hex(bits), s)


# --------------------------------------------------------------------------- bf16 encoder
def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(52)
    bits = rng.integers(0, 1 << 32, 20000, dtype=np.uint64).astype(np.uint32)
    xs = bits.view(np.float32)
    xs = xs[~np.isnan(xs)]
    extra = np.array([3.3895313892515355e38, 3.39e38, 3.4e38, -3.4e38, np.inf, 1e-45, 0.0, -0.0], np.float32)
    xs = np.concatenate([xs, extra])
    t = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = np.array([ref.encode_bf16(x) for x in xs], dtype=np.uint16)
    assert np.array_equal(mine, t)
    for x in xs[:3000]:
        assert brute.encode_bf16(float(x)) == ref.encode_bf16(x)
    assert ref.encode_bf16(math.nan) == 0x7FC0


# --------------------------------------------------------------------------- append
def _case(kv, B=3, Hkv=2, d=8, L=10, seed=60):
    c = workloads.make_case(B, 2 * Hkv, Hkv, d, L, "bf16", kv, seq_lens=[L] * B, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    kn = torch.randn(B, Hkv, d, generator=g) * 3
    vn = torch.randn(B, Hkv, d, generator=g) * 3
    return c, kn, vn


@pytest.mark.parametrize("kv,new", [("bf16", "bf16"), ("bf16", "f32"), ("fp8_e4m3", "bf16"),
                                    ("fp8_e4m3", "f32"), ("f32", "f32")])
def test_append_writes_exactly_the_encoded_rows(kv, new):
    c, kn, vn = _case(kv)
    kn, vn = workloads.cast(kn, new) if new == "bf16" else kn, workloads.cast(vn, new) if new == "bf16" else vn
    pos = [4, -1, 9]                                 # sequence 1 inactive this step
    kd, vd = 0.5, 0.25
    kc, vc, skipped = ref.append(kn, vn, new, c["k"], c["v"], kv, pos, kd, vd)
    assert skipped == 0
    k0, v0 = ref.raw(c["k"], kv), ref.raw(c["v"], kv)
    knr, vnr = ref.raw(kn, new), ref.raw(vn, new)
    changed = np.argwhere(np.any(kc != k0, axis=-1) | np.any(vc != v0, axis=-1))
    assert {tuple(x) for x in changed} <= {(b, j, pos[b]) for b in (0, 2) for j in range(2)}
    for b in (0, 2):
        for j in range(2):
            for cc in range(8):
                xk = float(knr[b, j, cc]) if new == "f32" else brute.bf16_bits_to_float(knr[b, j, cc])
                xv = float(vnr[b, j, cc]) if new == "f32" else brute.bf16_bits_to_float(vnr[b, j, cc])
                if kv == "fp8_e4m3":
                    assert kc[b, j, pos[b], cc] == brute.encode_fp8_e4m3(xk, kd)
                    assert vc[b, j, pos[b], cc] == brute.encode_fp8_e4m3(xv, vd)
                elif kv == "bf16":
                    assert kc[b, j, pos[b], cc] == brute.encode_bf16(xk)
                    assert vc[b, j, pos[b], cc] == brute.encode_bf16(xv)
                else:
                    assert kc[b, j, pos[b], cc] == np.float32(xk) and vc[b, j, pos[b], cc] == np.float32(xv)


def test_append_past_the_end_is_counted_not_written():
    c, kn, vn = _case("bf16")
    kn, vn = kn.to(torch.bfloat16), vn.to(torch.bfloat16)
    kc, vc, skipped = ref.append(kn, vn, "bf16", c["k"], c["v"], "bf16", [10, 3, 11])
    assert skipped == 2
    assert np.array_equal(np.delete(kc, 1, axis=0), np.delete(ref.raw(c["k"], "bf16"), 1, axis=0))


def test_paging_commutes_with_append():
    c, kn, vn = _case("fp8_e4m3", B=3, Hkv=2, d=8, L=24, seed=61)
    c["seq_lens"] = torch.tensor([24, 7, 16], dtype=torch.int32)
    pos = [23, 7, 16]
    kn, vn = kn.to(torch.bfloat16), vn.to(torch.bfloat16)
    # dense append, then page the result ...
    kc, vc, _ = ref.append(kn, vn, "bf16", c["k"], c["v"], "fp8_e4m3", pos, 0.5, 2.0)
    after = dict(c, k=torch.from_numpy(kc).view(torch.float8_e4m3fn),
                 v=torch.from_numpy(vc).view(torch.float8_e4m3fn),
                 seq_lens=torch.tensor([24, 8, 17], dtype=torch.int32))
    want = workloads.paginate(after, 4, seed=3)
    # ... equals paging first (room for the new positions) and appending through the table
    before = dict(c, seq_lens=torch.tensor([24, 8, 17], dtype=torch.int32))
    pg = workloads.paginate(before, 4, seed=3)
    kp, vp, skipped = ref.append(kn, vn, "bf16", pg["k_pages"], pg["v_pages"], "fp8_e4m3", pos, 0.5, 2.0,
                                 block_table=pg["block_table"])
    assert skipped == 0
    assert torch.equal(pg["block_table"], want["block_table"])
    live = want["block_table"][want["block_table"] >= 0].unique()
    for page in live.tolist():   # every used page matches (unused page rows are NaN fill in both)
        a, b = kp[page].astype(np.int32), ref.raw(want["k_pages"], "fp8_e4m3")[page].astype(np.int32)
        same = (a == b) | ((a & 0x7F) == 0x7F) & ((b & 0x7F) == 0x7F)
        assert same.all(), page
        a, b = vp[page].astype(np.int32), ref.raw(want["v_pages"], "fp8_e4m3")[page].astype(np.int32)
        assert ((a == b) | ((a & 0x7F) == 0x7F) & ((b & 0x7F) == 0x7F)).all(), page


def test_decode_finds_the_row_just_appended():
    # a key far along the query direction, appended at position n, dominates a decode over n + 1
    B, Hq, Hkv, d, L, n = 1, 4, 1, 16, 12, 7
    c = workloads.make_case(B, Hq, Hkv, d, L, "bf16", "bf16", seq_lens=[n], seed=62)
    q = c["q"].float()
    q[0, :] = q[0, 0]
    c["q"] = q.to(torch.bfloat16)
    unit = c["q"][0, 0].float() / c["q"][0, 0].float().norm()
    kn = (unit * 30).reshape(1, 1, d)
    vn = torch.arange(d, dtype=torch.float32).reshape(1, 1, d) / 4
    kc, vc, _ = ref.append(kn, vn, "f32", c["k"], c["v"], "bf16", [n])
    kt = torch.from_numpy(kc.view(np.int16)).view(torch.bfloat16)
    vt = torch.from_numpy(vc.view(np.int16)).view(torch.bfloat16)
    out = ref.decode(c["q"], kt, vt, [n + 1], 1.0, "bf16", "bf16")
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], vn[0, 0].numpy(), rtol=0, atol=1e-6)
    # without the new position the decode does not see it
    out0 = ref.decode(c["q"], kt, vt, [n], 1.0, "bf16", "bf16")
    assert np.abs(out0[0, 0] - vn[0, 0].numpy()).max() > 0.1
