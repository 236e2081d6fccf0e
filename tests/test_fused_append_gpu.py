"""Fused append + decode (gqa_decode_append, gqa_decode_append_paged) through the C ABI.

The fused call stores the new token's K/V rows at position seq_lens[b] - 1 and attends over the first
seq_lens[b] positions in one launch.  Its expected result is the oracle's append of the same rows
(bit-exact: the whole cache, byte for byte) followed by the oracle's decode over the appended cache
(the decode gates of the parity tests).  The rows the new token lands on are poisoned with NaN before
the call, so a decode that read the stale cache row instead of the new one fails.  A second check
asks for more than parity: the fused output and cache are bitwise those of the two separate GPU
calls it replaces, at small sizes and at the full size of the 70B-layer step.
"""
import numpy as np
import pytest
import torch

import grouped_query_attention_04_amd as gqa
import workloads
from oracle import ref
from tests.test_parity_gpu import DEV, compare, rows_off, say

pytestmark = pytest.mark.gpu

RAW_TORCH = {"bf16": torch.int16, "fp8_e4m3": torch.uint8}
POISON = workloads.POISON_BITS


def _raw(t, dt):
    return t.detach().cpu().contiguous().view(RAW_TORCH[dt]).numpy()


def _new_rows(B, Hkv, d, seed):
    g = torch.Generator().manual_seed(seed)
    kn = (torch.randn(B, Hkv, d, generator=g) * 2.0).to(torch.bfloat16)
    vn = (torch.randn(B, Hkv, d, generator=g) * 2.0).to(torch.bfloat16)
    return kn, vn


def _poison_dense(t, dt, positions):
    """NaN into row positions[b] of every KV head of sequence b (positions inside the cache only)."""
    raw = t.view(RAW_TORCH[dt])
    for b, p in enumerate(positions):
        if 0 <= p < t.shape[2]:
            raw[b, :, p] = POISON[dt]


def _poison_paged(t, dt, table, bs, positions):
    raw = t.view(RAW_TORCH[dt])
    for b, p in enumerate(positions):
        if 0 <= p < table.shape[1] * bs:
            page = int(table[b, p // bs])
            if 0 <= page < t.shape[0]:
                raw[page, :, p % bs] = POISON[dt]


# Lengths (new token included) that put the new position at a tile's first and last rows, at the
# first and last positions of the cache, past the cache (skipped), on an empty sequence, and in
# ragged tails.  L = 320 is 20 tiles of 16 and 5 pages of 64.
L_SMALL = 320
SEQ = [1, 16, 17, 320, 0, 321, 150, 255, 33, 64]


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (64, 2), (64, 1)])   # (64, 1): split into four sub-groups
@pytest.mark.parametrize("wg", [0, 7])
def test_fused_matches_oracle(paged, kv, d, Hq, Hkv, wg):
    say(f"fused append+decode paged={paged} kv={kv} d={d} Hq={Hq} Hkv={Hkv} workgroups={wg}")
    B, L = len(SEQ), L_SMALL
    sl = np.array(SEQ, dtype=np.int32)
    clamped = np.clip(sl, 0, L)
    c = workloads.make_case(B, Hq, Hkv, d, L, "bf16", kv, seq_lens=clamped.tolist(), seed=90 + d + Hq)
    kd, vd = (0.5, 1.25) if kv == "fp8_e4m3" else (1.0, 1.0)
    kn, vn = _new_rows(B, Hkv, d, 91 + d)
    pos = sl - 1
    skipped = torch.zeros(1, dtype=torch.int32, device=DEV)
    if not paged:
        _poison_dense(c["k"], kv, pos)
        _poison_dense(c["v"], kv, pos)
        kc, vc = c["k"].to(DEV), c["v"].to(DEV)
        got = gqa.decode_append(c["q"].to(DEV), kn.to(DEV), vn.to(DEV), kc, vc, torch.from_numpy(sl).to(DEV),
                                c["scale"], out_dtype=torch.float32, k_descale=kd, v_descale=vd,
                                num_workgroups=wg, skipped=skipped)
        torch.cuda.synchronize()
        wk, wv, wskip = ref.append(kn, vn, "bf16", c["k"], c["v"], kv, pos, kd, vd)
        want = ref.decode(c["q"], wk, wv, clamped, c["scale"], "bf16", kv, kd, vd)
        assert wskip == 1
    else:
        bs = 64
        pg = workloads.paginate(c, bs, seed=13, spare_pages=2)
        table = pg["block_table"].clone()
        # the new position of sequence 6 (length 150) sits on a page outside the pool
        table[6, 149 // bs] = pg["num_blocks"] + 7
        _poison_paged(pg["k_pages"], kv, table, bs, pos)
        _poison_paged(pg["v_pages"], kv, table, bs, pos)
        kp, vp = pg["k_pages"].to(DEV), pg["v_pages"].to(DEV)
        got = gqa.decode_append_paged(c["q"].to(DEV), kn.to(DEV), vn.to(DEV), kp, vp, table.to(DEV),
                                      torch.from_numpy(sl).to(DEV), c["scale"], out_dtype=torch.float32,
                                      k_descale=kd, v_descale=vd, num_workgroups=wg, skipped=skipped)
        torch.cuda.synchronize()
        wk, wv, wskip = ref.append(kn, vn, "bf16", pg["k_pages"], pg["v_pages"], kv, pos, kd, vd,
                                   block_table=table.numpy())
        assert wskip == 2                     # past the cache, and the out-of-pool page
        # the out-of-pool page reads as zeros: the oracle decodes with an added all-zero page there
        zeros = np.zeros((1,) + wk.shape[1:], dtype=wk.dtype)
        ztab = table.clone()
        ztab[6, 149 // bs] = pg["num_blocks"]
        want = ref.decode_paged(c["q"], np.concatenate([wk, zeros]), np.concatenate([wv, zeros]), ztab.numpy(),
                                clamped, c["scale"], None, "bf16", kv, kd, vd)
        kc, vc = kp, vp
    assert int(skipped.item()) == wskip
    assert np.array_equal(_raw(kc, kv), wk.view(_raw(kc, kv).dtype)), "K cache differs from the oracle's append"
    assert np.array_equal(_raw(vc, kv), wv.view(_raw(vc, kv).dtype)), "V cache differs from the oracle's append"
    compare(got, want, kv, "fused")
    assert (got[4] == 0).all()                # empty sequence: zero row


def _separate_and_fused(c, kn, vn, sl, kd, vd, wg=0, paged_bs=None, out_dtype=None):
    """Runs append_kv + decode and decode_append on two copies of the same cache; returns both
    (out, k, v) triples, on the host (out in out_dtype, default q's)."""
    q = c["q"].to(DEV)
    sld = sl.to(DEV)
    knd, vnd = kn.to(DEV), vn.to(DEV)
    res = []
    for fused in (False, True):
        if paged_bs is None:
            k, v = c["k"].to(DEV), c["v"].to(DEV)
            if fused:
                out = gqa.decode_append(q, knd, vnd, k, v, sld, c["scale"], k_descale=kd, v_descale=vd,
                                        num_workgroups=wg, out_dtype=out_dtype)
            else:
                gqa.append_kv(knd, vnd, k, v, sld - 1, k_descale=kd, v_descale=vd)
                out = gqa.decode(q, k, v, sld, c["scale"], k_descale=kd, v_descale=vd, num_workgroups=wg,
                                 out_dtype=out_dtype)
        else:
            k, v, t = c["k_pages"].to(DEV), c["v_pages"].to(DEV), c["block_table"].to(DEV)
            if fused:
                out = gqa.decode_append_paged(q, knd, vnd, k, v, t, sld, c["scale"], k_descale=kd,
                                              v_descale=vd, num_workgroups=wg, out_dtype=out_dtype)
            else:
                gqa.append_kv_paged(knd, vnd, k, v, t, sld - 1, k_descale=kd, v_descale=vd)
                out = gqa.decode_paged(q, k, v, t, sld, c["scale"], k_descale=kd, v_descale=vd,
                                       num_workgroups=wg, out_dtype=out_dtype)
        torch.cuda.synchronize()
        res.append((out.cpu(), k.cpu(), v.cpu()))
        del k, v
    return res


def _bitwise(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("paged_bs", [None, 16])
@pytest.mark.parametrize("wg", [0, 37, 512])
def test_fused_is_bitwise_the_two_calls(kv, paged_bs, wg):
    say(f"fused vs append_kv + decode, kv={kv} block_size={paged_bs} workgroups={wg}")
    B, Hq, Hkv, d, L = 6, 64, 8, 128, 1024
    c = workloads.make_case(B, Hq, Hkv, d, L, "bf16", kv, seq_range=(1, L), seed=95)
    if paged_bs is not None:
        c = workloads.paginate(c, paged_bs, seed=14, spare_pages=4)
    kn, vn = _new_rows(B, Hkv, d, 96)
    (o1, k1, v1), (o2, k2, v2) = _separate_and_fused(c, kn, vn, c["seq_lens"], 0.75, 0.75, wg, paged_bs)
    assert _bitwise(k1, k2) and _bitwise(v1, v2), "caches differ"
    assert _bitwise(o1, o2), "outputs differ"


FUSED_FULL = [(3, None), (3, 16), (2, None), (2, 32), ("4-gqa", 64), ("4-mqa64", None), ("4-mqa64", 16),
              (5, None), (5, 64)]


@pytest.mark.parametrize("wid,paged_bs", FUSED_FULL, ids=lambda x: str(x))
def test_fused_full_size(wid, paged_bs):
    """Named workloads at full size (the 70B layer, the 8B layer, the group-size sweep's GQA-8 point
    and the long fp8 cache), library's workgroup count: every output row against the oracle's
    append + decode, the whole cache bit-exact against the oracle's append, and everything bitwise
    against the two separate calls."""
    w = workloads.WORKLOADS[wid]
    say(f"fused full size: {w.name}, block_size {paged_bs}")
    c = workloads.make(wid)
    B, Hkv, d, kv = w.B, w.Hkv, w.d, w.kv_dtype
    kn, vn = _new_rows(B, Hkv, d, 97)
    sl = c["seq_lens"]
    if paged_bs is not None:
        c = workloads.paginate(c, paged_bs, seed=15, spare_pages=8)
    (o1, k1, v1), (o2, k2, v2) = _separate_and_fused(c, kn, vn, sl, 1.0, 1.0, 0, paged_bs)
    assert _bitwise(k1, k2) and _bitwise(v1, v2), "caches differ"
    assert _bitwise(o1, o2), "outputs differ"
    pos = (sl - 1).numpy()
    if paged_bs is None:
        wk, wv, wskip = ref.append(kn, vn, "bf16", c["k"], c["v"], kv, pos)
    else:
        wk, wv, wskip = ref.append(kn, vn, "bf16", c["k_pages"], c["v_pages"], kv, pos,
                                   block_table=c["block_table"].numpy())
    assert wskip == 0
    assert np.array_equal(_raw(k2, kv), wk.view(_raw(k2, kv).dtype)), "K cache differs from the oracle's append"
    assert np.array_equal(_raw(v2, kv), wv.view(_raw(v2, kv).dtype)), "V cache differs from the oracle's append"
    del k1, v1, k2, v2
    if paged_bs is None:
        want = ref.decode_all(c["q"], wk, wv, sl.numpy(), c["scale"], "bf16", kv)
    else:
        want = ref.decode_paged(c["q"], wk, wv, c["block_table"].numpy(), sl.numpy(), c["scale"], "all",
                                "bf16", kv, threads=ref.host_threads())
    bad = rows_off(o2, want, kv)
    if bad:
        say(f"  rows off the oracle: {bad[:20]}")
    compare(o2, want, kv, f"fused full size, all {w.B * w.Hq} rows")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("paged_bs", [None, 32])
@pytest.mark.parametrize("B,wg", [(300, 37), (1000, 0)], ids=lambda x: str(x))
def test_fused_batches_above_256(B, wg, paged_bs, kv):
    """The fused append + decode with more sequences than 256 and than workgroups: the whole cache
    bit-exact against the oracle's append, every output row against the oracle's decode.  The output
    is f32: many sequences hold one or a few positions, so rows are close to single value rows of
    magnitude up to ~8, where bf16 output rounding alone would exceed the absolute gate."""
    from tests.test_parity_gpu import _serving_lengths

    L = 300
    sl = torch.tensor(_serving_lengths(B, L, seed=5 * B + wg), dtype=torch.int32)
    say(f"fused batch {B}, {wg} workgroups, kv={kv}, block_size {paged_bs}")
    c = workloads.make_case(B, 16, 2, 128, L, "bf16", kv, seq_lens=sl.tolist(), seed=B * 3 + wg)
    kn, vn = _new_rows(B, 2, 128, 98)
    if paged_bs is not None:
        c = workloads.paginate(c, paged_bs, seed=17, spare_pages=3)
    (o1, k1, v1), (o2, k2, v2) = _separate_and_fused(c, kn, vn, sl, 1.0, 1.0, wg, paged_bs, torch.float32)
    assert _bitwise(k1, k2) and _bitwise(v1, v2), "caches differ"
    assert _bitwise(o1, o2), "outputs differ"
    pos = (sl - 1).numpy()
    if paged_bs is None:
        wk, wv, wskip = ref.append(kn, vn, "bf16", c["k"], c["v"], kv, pos)
        want = ref.decode_all(c["q"], wk, wv, sl.numpy(), c["scale"], "bf16", kv)
    else:
        wk, wv, wskip = ref.append(kn, vn, "bf16", c["k_pages"], c["v_pages"], kv, pos,
                                   block_table=c["block_table"].numpy())
        want = ref.decode_paged(c["q"], wk, wv, c["block_table"].numpy(), sl.numpy(), c["scale"], "all",
                                "bf16", kv, threads=ref.host_threads())
    assert wskip == 0
    assert np.array_equal(_raw(k2, kv), wk.view(_raw(k2, kv).dtype)), "K cache differs from the oracle's append"
    assert np.array_equal(_raw(v2, kv), wv.view(_raw(v2, kv).dtype)), "V cache differs from the oracle's append"
    compare(o2, want, kv, f"fused B{B} wg{wg}")
