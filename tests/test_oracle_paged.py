"""Pins of the oracle's paged-cache definition to facts outside it.

A paged cache changes where a position's K and V rows live, not what attention computes.  The pins:
the one-page-per-sequence special case, which is the dense layout byte for byte; invariance under any
placement of the pages; the worked example of "Grouped Query Attention (GQA): Efficient Multi-Head
Attention" (Worked example 2) stored one position per page in reversed order; a needle that the page
table must find while decoys sit in unused pages and past the sequence end; an independent pure-Python
gather; and planted indexing mistakes that these pins reject.
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import brute, ref
from tests.conftest import GOLDEN


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


with open(os.path.join(GOLDEN, "worked_example_2.json")) as f:
    WE2 = json.load(f)


@pytest.mark.parametrize("dt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8_e4m3")])
def test_one_page_per_sequence_is_the_dense_layout(dt):
    # block_size = L and page b for sequence b: [num_blocks=B][Hkv][L][d] is the dense [B][Hkv][L][d]
    qd, kd = dt
    c = workloads.make_case(3, 8, 2, 16, 40, qd, kd, seq_lens=(40, 17, 0), seed=21)
    table = np.arange(3, dtype=np.int32).reshape(3, 1)
    dense = ref.decode(c["q"], c["k"], c["v"], c["seq_lens"], c["scale"], qd, kd)
    paged = ref.decode_paged(c["q"], c["k"], c["v"], table, c["seq_lens"], c["scale"], None, qd, kd)
    assert np.array_equal(dense, paged)


@pytest.mark.parametrize("bs", [1, 4, 16])
def test_page_placement_does_not_change_the_result(bs):
    c = workloads.make_case(3, 6, 3, 8, 37, "bf16", "bf16", seq_lens=(37, 5, 21), seed=22)
    a = workloads.paginate(c, bs, seed=1, spare_pages=3)
    b = workloads.paginate(c, bs, seed=2, spare_pages=5)
    assert not torch.equal(a["block_table"], b["block_table"])
    oa = ref.decode_paged(c["q"], a["k_pages"], a["v_pages"], a["block_table"], c["seq_lens"], 0.3)
    ob = ref.decode_paged(c["q"], b["k_pages"], b["v_pages"], b["block_table"], c["seq_lens"], 0.3)
    assert np.array_equal(oa, ob) and np.isfinite(oa).all()   # the NaN-filled spare pages are never read
    dense = ref.decode(c["q"], c["k"], c["v"], c["seq_lens"], 0.3, "bf16", "bf16")
    assert np.array_equal(oa, dense)


def test_worked_example_2_one_position_per_page_reversed():
    # two positions per KV head, stored in pages of one position, the later position first
    q = _f32(WE2["q"])[None]                          # [1, 4, 2]
    k = _f32(WE2["k"])                                # [Hkv=2][t=2][d=2]
    v = _f32(WE2["v"])
    kp = np.full((3, 2, 1, 2), np.nan, np.float32)    # page 2 is an unused NaN page
    vp = np.full((3, 2, 1, 2), np.nan, np.float32)
    for t, page in ((0, 1), (1, 0)):
        kp[page, :, 0] = k[:, t]
        vp[page, :, 0] = v[:, t]
    table = np.array([[1, 0]], np.int32)
    out = ref.decode_paged(q, kp, vp, table, [2], WE2["scale"], None, "f32", "f32")
    np.testing.assert_allclose(out[0], np.array(WE2["out"]), rtol=0, atol=WE2["tolerance"])


def test_needle_found_through_the_table_and_decoys_ignored():
    B, Hq, Hkv, d, bs, n = 1, 4, 1, 8, 4, 10
    rng = np.random.default_rng(23)
    q = _f32(rng.standard_normal((B, Hq, d)))
    q[0, :] = q[0, 0]
    unit = q[0, 0] / np.linalg.norm(q[0, 0])
    num_blocks = 6
    kp = _f32(rng.standard_normal((num_blocks, Hkv, bs, d)) * 0.1)
    vp = _f32(rng.standard_normal((num_blocks, Hkv, bs, d)))
    table = np.array([[4, 0, 2, 5]], np.int32)       # pages 1 and 3 unused
    needle_page, needle_row = table[0, (n - 1) // bs], (n - 1) % bs
    kp[needle_page, 0, needle_row] = unit * 40
    kp[needle_page, 0, needle_row + 1] = unit * 80   # position n: past the sequence end
    kp[1, 0, :] = unit * 90                          # unused pages full of decoys
    kp[3, 0, :] = unit * 90
    out = ref.decode_paged(q, kp, vp, table, [n], 1.0, None, "f32", "f32")
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], vp[needle_page, 0, needle_row], rtol=0, atol=1e-6)


@pytest.mark.parametrize("dt", [("f32", "f32"), ("bf16", "bf16"), ("f32", "fp8_e4m3")])
def test_brute_force_gather_agrees(dt):
    qd, kd = dt
    for seed, (B, Hq, Hkv, d, L, bs) in enumerate([(2, 4, 2, 3, 9, 2), (1, 3, 1, 4, 8, 4),
                                                   (3, 2, 2, 2, 5, 1)]):
        c = workloads.make_case(B, Hq, Hkv, d, L, qd, kd, seq_range=(0, L), seed=30 + seed)
        pg = workloads.paginate(c, bs, seed=seed, spare_pages=1)
        got = ref.decode_paged(c["q"], pg["k_pages"], pg["v_pages"], pg["block_table"], c["seq_lens"],
                               0.7, None, qd, kd, 1.0, 1.0)
        raw = {n: ref.raw(pg[n], kd).tolist() for n in ("k_pages", "v_pages")}
        want = np.array(brute.decode_paged(ref.raw(c["q"], qd).tolist(), raw["k_pages"], raw["v_pages"],
                                           pg["block_table"].tolist(), c["seq_lens"].tolist(), 0.7, qd, kd))
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_live_entries_checked_dead_entries_ignored():
    c = workloads.make_case(2, 4, 2, 4, 12, "f32", "f32", seq_lens=(12, 5), seed=24)
    pg = workloads.paginate(c, 4, seed=3, dead_entry=10**6)   # dead entries far outside the pool
    out = ref.decode_paged(c["q"], pg["k_pages"], pg["v_pages"], pg["block_table"], c["seq_lens"], 0.5,
                           None, "f32", "f32")
    assert np.isfinite(out).all()
    bad = pg["block_table"].clone()
    bad[1, 1] = pg["num_blocks"]                     # position 4..7 of sequence 1 is live
    with pytest.raises(ValueError):
        ref.decode_paged(c["q"], pg["k_pages"], pg["v_pages"], bad, c["seq_lens"], 0.5, None, "f32", "f32")
    bad[1, 1] = -1
    with pytest.raises(ValueError):
        ref.decode_paged(c["q"], pg["k_pages"], pg["v_pages"], bad, c["seq_lens"], 0.5, None, "f32", "f32")


# --------------------------------------------------------------------------- planted mistakes
def _numpy_paged(q, kp, vp, table, sl, scale, mistake=None):
    q = np.asarray(q, np.float64)
    kp, vp = np.asarray(kp, np.float64), np.asarray(vp, np.float64)
    B, Hq, d = q.shape
    nb, Hkv, bs, _ = kp.shape
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        n = int(sl[b])
        if n == 0:
            continue
        for h in range(Hq):
            j = h // G
            rows = []
            for t in range(n):
                page, row = table[b][t // bs], t % bs
                if mistake == "row_and_page_swapped":
                    page, row = table[b][t % bs] if t % bs < len(table[b]) else 0, t // bs % bs
                if mistake == "table_row_by_head":
                    page = table[j % B][t // bs]
                if mistake == "token_major_pool":        # reads [nb][bs][Hkv][d] as if it were ours
                    flat = kp.reshape(nb, bs, Hkv, d)
                    rows.append((flat[page, row, j], vp.reshape(nb, bs, Hkv, d)[page, row, j]))
                    continue
                rows.append((kp[page, j, row], vp[page, j, row]))
            kk = np.array([r[0] for r in rows])
            vv = np.array([r[1] for r in rows])
            s = kk @ q[b, h] * scale
            p = np.exp(s - s.max())
            out[b, h] = vv.T @ (p / p.sum())
    return out


def _paged_pins_pass(fn):
    q = _f32(WE2["q"])[None]
    k, v = _f32(WE2["k"]), _f32(WE2["v"])
    kp = np.zeros((2, 2, 1, 2), np.float32)
    vp = np.zeros((2, 2, 1, 2), np.float32)
    for t, page in ((0, 1), (1, 0)):
        kp[page, :, 0] = k[:, t]
        vp[page, :, 0] = v[:, t]
    if not np.allclose(fn(q, kp, vp, [[1, 0]], [2], WE2["scale"])[0], WE2["out"], atol=WE2["tolerance"]):
        return False
    c = workloads.make_case(2, 4, 2, 4, 16, "f32", "f32", seq_lens=(16, 11), seed=25)
    pg = workloads.paginate(c, 4, seed=4)
    want = ref.decode(c["q"], c["k"], c["v"], c["seq_lens"], 0.5)   # the dense definition
    got = fn(c["q"].numpy(), pg["k_pages"].numpy(), pg["v_pages"].numpy(), pg["block_table"].tolist(),
             c["seq_lens"].tolist(), 0.5)
    return np.allclose(got, want, atol=1e-9)


def test_paged_pins_accept_correct_gather():
    assert _paged_pins_pass(_numpy_paged)
    assert _paged_pins_pass(lambda q, kp, vp, t, sl, s: ref.decode_paged(
        _f32(q), _f32(kp), _f32(vp), np.asarray(t, np.int32), sl, s, None, "f32", "f32"))


@pytest.mark.parametrize("mistake", ["row_and_page_swapped", "table_row_by_head", "token_major_pool"])
def test_paged_pins_reject_planted_mistake(mistake):
    assert not _paged_pins_pass(lambda *a: _numpy_paged(*a, mistake=mistake))
