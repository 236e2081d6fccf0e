"""Caches, page pools and prefill buffers larger than 4 GiB, through the C ABI.

Byte offsets past 2^32 must survive every address computation: the segment bases of a dense cache,
the page bases of a pool, the rows the fused append writes, and the query and output rows of the
prefill.  The big buffers are built on the
device and filled with NaN; the rows of a small seeded case are copied to their places far inside
them (positions past each sequence's end stay NaN), so the oracle runs on the small case, and a read
of a wrong row, or of a row never written, shows.
"""
import math

import numpy as np
import pytest
import torch

import grouped_query_attention_04_amd as gqa
import workloads
from oracle import ref
from tests.test_parity_gpu import DEV, compare, say

pytestmark = pytest.mark.gpu

RAW = {"bf16": torch.int16, "fp8_e4m3": torch.uint8}
ELT = {"bf16": 2, "fp8_e4m3": 1}
B, HQ, HKV, D, LS = 3, 16, 8, 128, 2048
SEQ = (2047, 1999, 1)      # before the new token; the fused call appends at these positions


def _nan_buffer(shape, kd):
    raw = torch.full(shape, workloads.POISON_BITS[kd], dtype=RAW[kd], device=DEV)
    return raw.view(workloads.TORCH_DTYPES[kd])


def _small_case(kd, seed):
    """The seeded small case, with every cache row at or past its sequence's end set to NaN."""
    c = workloads.make_case(B, HQ, HKV, D, LS, "bf16", kd, seq_lens=SEQ, seed=seed)
    for b, n in enumerate(SEQ):
        c["k"].view(RAW[kd])[b, :, n:] = workloads.POISON_BITS[kd]
        c["v"].view(RAW[kd])[b, :, n:] = workloads.POISON_BITS[kd]
    g = torch.Generator().manual_seed(seed + 1)
    kn = torch.randn(B, HKV, D, generator=g).to(torch.bfloat16)
    vn = torch.randn(B, HKV, D, generator=g).to(torch.bfloat16)
    return c, kn, vn


def _expected(c, kn, vn, kd):
    """Oracle: the decode over the small case, and its append + decode one position further."""
    sl = np.array(SEQ, dtype=np.int32)
    want = ref.decode(c["q"], c["k"], c["v"], sl, c["scale"], "bf16", kd)
    wk, wv, skipped = ref.append(kn, vn, "bf16", c["k"], c["v"], kd, sl)
    assert skipped == 0
    want_f = ref.decode(c["q"], wk, wv, sl + 1, c["scale"], "bf16", kd)
    return want, want_f, wk, wv


@pytest.mark.parametrize("kd", ["bf16", "fp8_e4m3"])
def test_dense_cache_beyond_4gib(kd):
    """B3 Hkv8 segments of 256 MiB each (L = 2^28 / (d * bytes)): 6 GiB per cache, so the last
    segments start past 5 GiB."""
    L = (1 << 28) // (D * ELT[kd])
    say(f"dense cache beyond 4 GiB: B{B} Hq{HQ} Hkv{HKV} d{D} L{L} kv={kd}")
    c, kn, vn = _small_case(kd, 170)
    want, want_f, wk, wv = _expected(c, kn, vn, kd)
    kc, vc = _nan_buffer((B, HKV, L, D), kd), _nan_buffer((B, HKV, L, D), kd)
    kc.view(RAW[kd])[:, :, :LS] = c["k"].view(RAW[kd]).to(DEV)
    vc.view(RAW[kd])[:, :, :LS] = c["v"].view(RAW[kd]).to(DEV)
    q, sl = c["q"].to(DEV), torch.tensor(SEQ, dtype=torch.int32, device=DEV)
    assert (B * HKV - 1) * L * D * ELT[kd] > (1 << 32)

    got = gqa.decode(q, kc, vc, sl, c["scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    compare(got, want, kd, "decode")

    got = gqa.decode_append(q, kn.to(DEV), vn.to(DEV), kc, vc, sl + 1, c["scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    compare(got, want_f, kd, "fused append + decode")
    for cache, w in ((kc, wk), (vc, wv)):
        window = cache.view(RAW[kd])[:, :, :LS].cpu().numpy()
        assert np.array_equal(window, w.view(window.dtype)), "cache rows differ from the oracle's append"
        assert (cache.view(RAW[kd])[:, :, LS:LS + 1] == workloads.POISON_BITS[kd]).all()


@pytest.mark.parametrize("kd", ["bf16", "fp8_e4m3"])
def test_paged_pool_beyond_4gib(kd):
    """16-position pages placed in random order around and past byte offset 2^32 of the pools (some
    just below it, most above it)."""
    bs = 16
    page_bytes = HKV * bs * D * ELT[kd]
    high = (1 << 32) // page_bytes + 1                    # the first page whose base lies past 4 GiB
    need = [math.ceil((n + 1) / bs) for n in SEQ]         # room for the appended position
    total = sum(need)
    num_blocks = high + 4 * total
    rng = np.random.default_rng(171)
    slots = rng.choice(np.arange(high - 64, num_blocks), size=total, replace=False).astype(np.int64)
    say(f"paged pool beyond 4 GiB: {num_blocks} pages of {page_bytes} bytes, kv={kd}")
    c, kn, vn = _small_case(kd, 172)
    want, want_f, wk, wv = _expected(c, kn, vn, kd)

    table = torch.full((B, LS // bs), -1, dtype=torch.int32)
    src_k, src_v, exp_k, exp_v = [], [], [], []
    i = 0
    for b in range(B):
        for lp in range(need[b]):
            table[b, lp] = int(slots[i])
            rows = slice(lp * bs, (lp + 1) * bs)
            src_k.append(c["k"].view(RAW[kd])[b, :, rows])
            src_v.append(c["v"].view(RAW[kd])[b, :, rows])
            exp_k.append(wk[b, :, rows])
            exp_v.append(wv[b, :, rows])
            i += 1
    idx = torch.from_numpy(slots).to(DEV)
    kp, vp = _nan_buffer((num_blocks, HKV, bs, D), kd), _nan_buffer((num_blocks, HKV, bs, D), kd)
    kp.view(RAW[kd]).index_copy_(0, idx, torch.stack(src_k).to(DEV))
    vp.view(RAW[kd]).index_copy_(0, idx, torch.stack(src_v).to(DEV))
    q, sl, t = c["q"].to(DEV), torch.tensor(SEQ, dtype=torch.int32, device=DEV), table.to(DEV)

    got = gqa.decode_paged(q, kp, vp, t, sl, c["scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    compare(got, want, kd, "paged decode")

    got = gqa.decode_append_paged(q, kn.to(DEV), vn.to(DEV), kp, vp, t, sl + 1, c["scale"],
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    compare(got, want_f, kd, "paged fused append + decode")
    for pool, exp in ((kp, exp_k), (vp, exp_v)):
        pages = pool.view(RAW[kd]).index_select(0, idx).cpu().numpy()
        expect = np.stack(exp)
        assert np.array_equal(pages, expect.view(pages.dtype)), "pages differ from the oracle's append"


def test_prefill_buffers_beyond_4gib():
    """Prefill with q and out of 4.6 GB each (B1100 Hq32 Hkv8 S512 d128): the first and the last
    batch entries hold a seeded case (the last one starts past byte offset 2^32 of q and out), every
    other entry is zero, whose output is exactly zero."""
    Bb, Hq, Hkv, S, d = 1100, 32, 8, 512, 128
    assert (Bb - 1) * Hq * S * d * 2 > (1 << 32)
    say(f"prefill beyond 4 GiB: B{Bb} Hq{Hq} Hkv{Hkv} S{S} d{d}")
    c = workloads.make_prefill_case(2, Hq, Hkv, d, S, seed=180)
    q = torch.zeros(Bb, Hq, S, d, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(Bb, Hkv, S, d, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros(Bb, Hkv, S, d, dtype=torch.bfloat16, device=DEV)
    for src, dst in ((0, 0), (1, Bb - 1)):
        q[dst] = c["q"][src].to(DEV)
        k[dst] = c["k"][src].to(DEV)
        v[dst] = c["v"][src].to(DEV)
    out = gqa.prefill(q, k, v, c["scale"], causal=True)
    torch.cuda.synchronize()
    del q, k, v
    rng = np.random.default_rng(181)
    rows = sorted({(b, int(h), int(i)) for b in (0, 1) for h, i in
                   zip(rng.integers(0, Hq, 24), rng.integers(0, S, 24))} |
                  {(1, 0, 0), (1, Hq - 1, S - 1), (0, Hq - 1, S - 1)})
    want = ref.prefill(c["q"], c["k"], c["v"], c["scale"], "bf16", True, rows=rows)
    got = torch.stack([out[0 if b == 0 else Bb - 1, h, i] for b, h, i in rows])
    compare(got, want, "bf16", f"prefill, {len(rows)} rows of the first and last entries")
    for b in (1, Bb // 2, Bb - 2):
        assert (out[b] == 0).all(), f"batch entry {b} (all zero inputs) is not zero"
