"""Pins of the oracle's row-selecting entry points to its full decode.

The full-size GPU parity tests and the CPU baseline call the oracle through ``decode_rows`` (dense
cache) and ``decode_paged(rows=...)`` (paged cache), which compute only the listed (batch, query
head) pairs.  Each listed row must be bitwise the row of the full decode -- itself pinned to the
worked example, torch SDPA, ``repeat_kv`` and brute force in ``test_oracle_pins.py`` -- in the order
given, with repeats, whatever the shape (group size 1, 32, 64; empty sequences; every cache dtype).
Pairs outside [0, B) x [0, Hq) are rejected.  The same rows are also checked against the independent
pure-Python brute force, and planted row-indexing mistakes are shown to fail these checks.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import brute, ref

SHAPES = [
    # (B, Hq, Hkv, d, L, seq_lens)
    (3, 8, 8, 16, 23, (23, 0, 9)),       # G = 1
    (2, 32, 1, 8, 17, (17, 5)),          # G = 32
    (2, 64, 1, 8, 11, (0, 11)),          # G = 64
    (4, 12, 4, 16, 30, (30, 1, 0, 19)),  # G = 3, an empty sequence in the middle
]
DTYPES = [("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8_e4m3")]


def _rows(B, Hq, seed, n=40):
    rng = np.random.default_rng(seed)
    rows = [(int(rng.integers(B)), int(rng.integers(Hq))) for _ in range(n)]
    rows += [rows[3], rows[0], (B - 1, Hq - 1), (0, 0), rows[0]]   # repeats and the corners
    rng.shuffle(rows)
    return rows


def _case(shape, dt, seed):
    B, Hq, Hkv, d, L, sl = shape
    return workloads.make_case(B, Hq, Hkv, d, L, dt[0], dt[1], seq_lens=sl, seed=seed)


def _dense_rows(c, rows):
    return ref.decode_rows(c["q"], c["k"], c["v"], c["seq_lens"], c["scale"], rows, c["q_dtype"],
                           c["kv_dtype"], 0.75, 1.5)


def _dense_full(c):
    return ref.decode(c["q"], c["k"], c["v"], c["seq_lens"], c["scale"], c["q_dtype"], c["kv_dtype"],
                      0.75, 1.5)


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: d[1])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}Hq{s[1]}Hkv{s[2]}")
def test_decode_rows_are_rows_of_the_full_decode(shape, dt):
    c = _case(shape, dt, seed=sum(shape[:5]))
    rows = _rows(shape[0], shape[1], seed=shape[1])
    full = _dense_full(c)
    part = _dense_rows(c, rows)
    assert part.shape == (len(rows), shape[3])
    for i, (b, h) in enumerate(rows):
        assert np.array_equal(part[i], full[b, h]), (i, b, h)
    # every row at once, in the order of the full result
    everything = [(b, h) for b in range(shape[0]) for h in range(shape[1])]
    assert np.array_equal(_dense_rows(c, everything).reshape(full.shape), full)


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: d[1])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}Hq{s[1]}Hkv{s[2]}")
def test_paged_rows_are_rows_of_the_full_paged_decode(shape, dt):
    if dt[1] == "f32":
        pytest.skip("paged caches hold bf16 or fp8")
    c = _case(shape, dt, seed=7 + sum(shape[:5]))
    p = workloads.paginate(c, 4, seed=3, spare_pages=2)
    rows = _rows(shape[0], shape[1], seed=11 + shape[1])
    args = (c["q"], p["k_pages"], p["v_pages"], p["block_table"], c["seq_lens"], c["scale"])
    full = ref.decode_paged(*args, None, c["q_dtype"], c["kv_dtype"], 0.75, 1.5)
    part = ref.decode_paged(*args, rows, c["q_dtype"], c["kv_dtype"], 0.75, 1.5)
    for i, (b, h) in enumerate(rows):
        assert np.array_equal(part[i], full[b, h]), (i, b, h)
    # and the paged full result is the dense one (pages are only a placement)
    assert np.array_equal(full, _dense_full(c))


def test_rows_agree_with_brute_force():
    c = _case((3, 6, 2, 4, 5, (5, 0, 3)), ("bf16", "bf16"), seed=5)
    rows = [(2, 5), (0, 1), (1, 3), (0, 1), (2, 0)]
    part = _dense_rows(c, rows)
    b = np.array(brute.decode(ref.raw(c["q"], "bf16").tolist(), ref.raw(c["k"], "bf16").tolist(),
                              ref.raw(c["v"], "bf16").tolist(), c["seq_lens"].tolist(), c["scale"],
                              "bf16", "bf16", 0.75, 1.5))
    for i, (bb, h) in enumerate(rows):
        np.testing.assert_allclose(part[i], b[bb][h], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("bad", [(-1, 0), (3, 0), (0, -1), (0, 6)])
def test_out_of_range_rows_are_rejected(bad):
    c = _case((3, 6, 2, 4, 5, (5, 0, 3)), ("bf16", "bf16"), seed=6)
    with pytest.raises(ValueError):
        _dense_rows(c, [(0, 0), bad])
    p = workloads.paginate(c, 2, seed=1)
    with pytest.raises(ValueError):
        ref.decode_paged(c["q"], p["k_pages"], p["v_pages"], p["block_table"], c["seq_lens"], 0.5,
                         [bad, (1, 1)])


# --------------------------------------------------------------------------- planted mistakes
def _rows_check_passes(select):
    """The checks above, applied to a row selector built on the full decode."""
    c = _case((3, 8, 2, 8, 9, (9, 4, 0)), ("bf16", "bf16"), seed=12)
    full = _dense_full(c)
    rows = _rows(3, 8, seed=4)
    part = select(full, rows)
    return all(np.array_equal(part[i], full[b, h]) for i, (b, h) in enumerate(rows))


MISTAKES = {
    # rows answered in sorted order instead of the order asked
    "sorted": lambda full, rows: np.stack([full[b, h] for b, h in sorted(rows)]),
    # the pair read as (head, batch)
    "swapped": lambda full, rows: np.stack([full[h % full.shape[0], b] for b, h in rows]),
    # repeated pairs computed once, the tail left as the first row
    "deduplicated": lambda full, rows: np.stack(
        [full[b, h] for b, h in dict.fromkeys(rows)] + [full[0, 0]] * (len(rows) - len(set(rows)))),
    # the neighbouring head of the same group
    "next_head": lambda full, rows: np.stack([full[b, (h + 1) % full.shape[1]] for b, h in rows]),
}


def test_row_checks_accept_the_correct_selector():
    assert _rows_check_passes(lambda full, rows: np.stack([full[b, h] for b, h in rows]))


@pytest.mark.parametrize("mistake", sorted(MISTAKES))
def test_row_checks_reject_planted_mistake(mistake):
    assert not _rows_check_passes(MISTAKES[mistake])


def test_rows_cover_every_head_of_the_group():
    """Constant V per (batch, KV head) reaches every listed row: out = j + 10 b for h in group j."""
    B, Hq, Hkv, d, L = 2, 64, 2, 8, 6
    c = workloads.make_case(B, Hq, Hkv, d, L, "bf16", "bf16", seq_lens=(6, 3), seed=13)
    v = torch.zeros(B, Hkv, L, d)
    for b in range(B):
        for j in range(Hkv):
            v[b, j] = j + 10 * b
    c["v"] = v.to(torch.bfloat16)
    rows = [(b, h) for h in range(Hq - 1, -1, -1) for b in (1, 0)]
    part = ref.decode_rows(c["q"], c["k"], c["v"], c["seq_lens"], c["scale"], rows, "bf16", "bf16")
    for i, (b, h) in enumerate(rows):
        assert np.allclose(part[i], h // (Hq // Hkv) + 10 * b, rtol=1e-15, atol=0)


# --------------------------------------------------------------------------- threaded row paths
@pytest.mark.parametrize("threads", [2, 3, 8])
def test_threaded_rows_equal_single_threaded(threads):
    """The row list cut over threads (each calling the same C function on its chunk) gives bitwise
    the single-threaded result, for the dense, paged and prefill row paths and the all-rows helper."""
    c = _case((4, 12, 4, 16, 30, (30, 1, 0, 19)), ("bf16", "fp8_e4m3"), seed=21)
    rows = _rows(4, 12, seed=22, n=57)
    one = _dense_rows(c, rows)
    many = ref.decode_rows(c["q"], c["k"], c["v"], c["seq_lens"], c["scale"], rows, c["q_dtype"],
                           c["kv_dtype"], 0.75, 1.5, threads=threads)
    assert np.array_equal(one, many)
    full = _dense_full(c)
    assert np.array_equal(ref.decode_all(c["q"], c["k"], c["v"], c["seq_lens"], c["scale"], c["q_dtype"],
                                         c["kv_dtype"], 0.75, 1.5, threads=threads), full)
    p = workloads.paginate(c, 8, seed=5, spare_pages=1)
    args = (c["q"], p["k_pages"], p["v_pages"], p["block_table"], c["seq_lens"], c["scale"])
    assert np.array_equal(ref.decode_paged(*args, "all", c["q_dtype"], c["kv_dtype"], 0.75, 1.5,
                                           threads=threads), full)
    q, k, v = (workloads.cast(torch.randn(s, generator=torch.Generator().manual_seed(i)), "bf16")
               for i, s in enumerate([(2, 4, 9, 8), (2, 2, 9, 8), (2, 2, 9, 8)]))
    pf = ref.prefill(q, k, v, 0.3, "bf16", True)
    assert np.array_equal(ref.prefill(q, k, v, 0.3, "bf16", True, rows="all", threads=threads), pf)


def test_threaded_rows_report_errors():
    c = _case((3, 6, 2, 4, 5, (5, 0, 3)), ("bf16", "bf16"), seed=6)
    with pytest.raises(ValueError):
        ref.decode_rows(c["q"], c["k"], c["v"], c["seq_lens"], 0.5, [(0, 0)] * 9 + [(0, 6)], "bf16", "bf16",
                        threads=4)
    with pytest.raises(ValueError):   # a seq_len outside [0, L] with an empty row list
        ref.decode_rows(c["q"], c["k"], c["v"], np.array([6, 0, 3], np.int32), 0.5, [], "bf16", "bf16",
                        threads=4)
