"""ctypes front end of the C oracle ``gqa_oracle.c`` (test infrastructure only).

Inputs are passed as raw storage: float32 arrays for fp32, uint16 bit patterns for bf16 and uint8 codes
for fp8-e4m3fn, together with a dtype name.  torch CPU tensors are accepted and reinterpreted as that
raw storage without any arithmetic.  Results come back as float64 numpy arrays.

``threads`` (decode_rows, decode_paged with rows, prefill with rows, and ``decode_all``): the listed
rows are cut into contiguous chunks, one per thread, and each thread calls the same single-threaded
C function on its chunk with its own scratch and output slice.  ctypes releases the GIL for the
call, so the chunks run on separate cores.  Each row is computed by the same code either way, so
the result is bitwise the single-threaded one.
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

DTYPES = {"f32": 0, "bf16": 1, "fp8_e4m3": 2}
_RAW = {"f32": np.float32, "bf16": np.uint16, "fp8_e4m3": np.uint8}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        c_void, c_int, c_dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        common = [c_void, c_int, c_void, c_void, c_int, c_dbl, c_dbl, c_void, c_dbl,
                  c_int, c_int, c_int, c_int, c_int]
        L.gqa_oracle_decode.argtypes = common + [c_void, c_void]
        L.gqa_oracle_decode.restype = c_int
        L.gqa_oracle_decode_rows.argtypes = common + [c_void, c_int, c_void, c_void]
        L.gqa_oracle_decode_rows.restype = c_int
        L.gqa_oracle_weights.argtypes = common + [c_int, c_int, c_void]
        L.gqa_oracle_weights.restype = c_int
        L.gqa_oracle_decode_paged.argtypes = [c_void, c_int, c_void, c_void, c_int, c_dbl, c_dbl, c_void,
                                              c_void, c_dbl, c_int, c_int, c_int, c_int, c_int, c_int,
                                              c_int, c_void, c_int, c_void, c_void]
        L.gqa_oracle_decode_paged.restype = c_int
        L.gqa_oracle_encode_bf16.argtypes = [ctypes.c_float]
        L.gqa_oracle_encode_bf16.restype = ctypes.c_uint16
        L.gqa_oracle_encode_fp8_e4m3.argtypes = [ctypes.c_float, ctypes.c_float]
        L.gqa_oracle_encode_fp8_e4m3.restype = ctypes.c_uint8
        L.gqa_oracle_append.argtypes = [c_void, c_void, c_int, c_void, c_void, c_int, c_dbl, c_dbl, c_void,
                                        c_int, c_int, c_int, c_int, c_void, c_int, c_int, c_int]
        L.gqa_oracle_append.restype = c_int
        L.gqa_oracle_prefill.argtypes = [c_void, c_void, c_void, c_int, c_dbl, c_int, c_int, c_int, c_int,
                                         c_int, c_int, c_void, c_int, c_void, c_void]
        L.gqa_oracle_prefill.restype = c_int
        L.gqa_oracle_kv_bytes_per_token.argtypes = [ctypes.c_uint64] * 4
        L.gqa_oracle_kv_bytes_per_token.restype = ctypes.c_uint64
        L.gqa_oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.gqa_oracle_bf16_to_double.restype = c_dbl
        L.gqa_oracle_fp8_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.gqa_oracle_fp8_e4m3_to_double.restype = c_dbl
        _lib = L
    return _lib


def raw(x, dtype_name):
    """Contiguous numpy view of the storage of x, reinterpreted as the raw type of dtype_name."""
    want = _RAW[dtype_name]
    if hasattr(x, "detach"):  # torch tensor
        import torch

        x = x.detach().cpu().contiguous()
        as_int = {np.uint16: torch.int16, np.uint8: torch.uint8, np.float32: torch.float32}[want]
        x = x.view(as_int).numpy().view(want)
    a = np.ascontiguousarray(x)
    if a.dtype != want:
        raise TypeError(f"{dtype_name} storage must be {np.dtype(want)}, got {a.dtype}")
    return a


def _args(q, k, v, seq_lens, scale, q_dtype, kv_dtype, k_descale, v_descale):
    qa, ka, va = raw(q, q_dtype), raw(k, kv_dtype), raw(v, kv_dtype)
    if qa.ndim != 3 or ka.ndim != 4 or va.shape != ka.shape:
        raise ValueError("q must be [B,Hq,d]; k and v [B,Hkv,L,d]")
    B, Hq, d = qa.shape
    Bk, Hkv, L, dk = ka.shape
    if Bk != B or dk != d:
        raise ValueError("batch or head_dim mismatch between q and the cache")
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32).reshape(-1))
    if sl.shape[0] != B:
        raise ValueError("seq_lens must have B entries")
    keep = (qa, ka, va, sl)
    args = [qa.ctypes.data, DTYPES[q_dtype], ka.ctypes.data, va.ctypes.data, DTYPES[kv_dtype],
            float(k_descale), float(v_descale), sl.ctypes.data, float(scale), B, Hq, Hkv, L, d]
    return args, keep, (B, Hq, Hkv, L, d)


def host_threads():
    """CPUs this process may run on (the affinity mask, not the machine's count)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def _run_chunks(nrows, threads, call):
    """call(lo, hi) for contiguous chunks of [0, nrows) on up to `threads` threads; returns the first
    non-zero return code (or 0)."""
    threads = max(1, min(int(threads), nrows))
    if threads == 1:
        return call(0, nrows)
    bounds = [nrows * i // threads for i in range(threads + 1)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        rcs = list(ex.map(lambda i: call(bounds[i], bounds[i + 1]), range(threads)))
    return next((rc for rc in rcs if rc), 0)


def _raise(rc):
    if rc == 1:
        raise ValueError("oracle: invalid shape or dtype")
    if rc == 2:
        raise ValueError("oracle: a seq_len lies outside [0, L]")
    if rc == 3:
        raise ValueError("oracle: a live page-table entry lies outside [0, num_blocks)")
    if rc:
        raise RuntimeError(f"oracle: error {rc}")


def decode(q, k, v, seq_lens, scale, q_dtype="f32", kv_dtype="f32", k_descale=1.0, v_descale=1.0):
    """out[B, Hq, d] in float64."""
    args, keep, (B, Hq, Hkv, L, d) = _args(q, k, v, seq_lens, scale, q_dtype, kv_dtype, k_descale,
                                           v_descale)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    w = np.zeros(max(L, 1), dtype=np.float64)
    _raise(lib().gqa_oracle_decode(*args, w.ctypes.data, out.ctypes.data))
    del keep
    return out


def decode_rows(q, k, v, seq_lens, scale, rows, q_dtype="f32", kv_dtype="f32", k_descale=1.0,
                v_descale=1.0, threads=1):
    """Only the listed (b, h) rows: returns [len(rows), d] float64."""
    args, keep, (B, Hq, Hkv, L, d) = _args(q, k, v, seq_lens, scale, q_dtype, kv_dtype, k_descale,
                                           v_descale)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
    out = np.zeros((r.shape[0], d), dtype=np.float64)

    def chunk(lo, hi):
        w = np.zeros(max(L, 1), dtype=np.float64)
        return lib().gqa_oracle_decode_rows(*args, r[lo:hi].ctypes.data, hi - lo, w.ctypes.data,
                                            out[lo:hi].ctypes.data)

    _raise(_run_chunks(r.shape[0], threads, chunk))
    del keep
    return out


def decode_all(q, k, v, seq_lens, scale, q_dtype="f32", kv_dtype="f32", k_descale=1.0, v_descale=1.0,
               threads=None):
    """Every (b, h) row, out[B, Hq, d] float64, on `threads` threads (default: every CPU this process
    may use).  Bitwise equal to decode()."""
    B, Hq = raw(q, q_dtype).shape[:2]
    rows = [(b, h) for b in range(B) for h in range(Hq)]
    out = decode_rows(q, k, v, seq_lens, scale, rows, q_dtype, kv_dtype, k_descale, v_descale,
                      threads=host_threads() if threads is None else threads)
    return out.reshape(B, Hq, -1)


def weights(q, k, v, seq_lens, scale, b, h, q_dtype="f32", kv_dtype="f32", k_descale=1.0,
            v_descale=1.0):
    """Softmax weights of query head (b, h) over its seq_lens[b] tokens (float64)."""
    args, keep, (B, Hq, Hkv, L, d) = _args(q, k, v, seq_lens, scale, q_dtype, kv_dtype, k_descale,
                                           v_descale)
    w = np.zeros(max(L, 1), dtype=np.float64)
    n = lib().gqa_oracle_weights(*args, int(b), int(h), w.ctypes.data)
    if n < 0:
        _raise(-n)
    del keep
    return w[:n].copy()


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale, rows=None, q_dtype="bf16",
                 kv_dtype="bf16", k_descale=1.0, v_descale=1.0, threads=1):
    """Decode over a paged cache.  k_pages, v_pages: [num_blocks, Hkv, block_size, d]; block_table:
    [B, max_blocks] int32.  Returns out[B, Hq, d] (rows None) or [len(rows), d], float64.  With
    rows == "all" every (b, h) row is computed through the row path (on `threads` threads) and
    returned as [B, Hq, d]."""
    qa = raw(q, q_dtype)
    ka, va = raw(k_pages, kv_dtype), raw(v_pages, kv_dtype)
    if qa.ndim != 3 or ka.ndim != 4 or va.shape != ka.shape:
        raise ValueError("q must be [B,Hq,d]; pages [num_blocks,Hkv,block_size,d]")
    B, Hq, d = qa.shape
    num_blocks, Hkv, block_size, dk = ka.shape
    if dk != d:
        raise ValueError("head_dim mismatch between q and the pages")
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    if bt.ndim != 2 or bt.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    max_blocks = bt.shape[1]
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32).reshape(-1))
    if sl.shape[0] != B:
        raise ValueError("seq_lens must have B entries")
    L = block_size * max_blocks
    every = isinstance(rows, str) and rows == "all"
    if every:
        rows = [(b, h) for b in range(B) for h in range(Hq)]
    if rows is None:
        r, nrows, out = None, 0, np.zeros((B, Hq, d), dtype=np.float64)
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        nrows, out = r.shape[0], np.zeros((r.shape[0], d), dtype=np.float64)

    def chunk(lo, hi):
        w = np.zeros(max(L, 1), dtype=np.float64)
        return lib().gqa_oracle_decode_paged(
            qa.ctypes.data, DTYPES[q_dtype], ka.ctypes.data, va.ctypes.data, DTYPES[kv_dtype],
            float(k_descale), float(v_descale), bt.ctypes.data, sl.ctypes.data, float(scale), B, Hq, Hkv,
            block_size, max_blocks, num_blocks, d, None if r is None else r[lo:hi].ctypes.data, hi - lo,
            w.ctypes.data, out[lo:hi].ctypes.data if r is not None else out.ctypes.data)

    _raise(chunk(0, 0) if r is None else _run_chunks(nrows, threads, chunk))
    del qa, ka, va, bt, sl
    return out.reshape(B, Hq, d) if every else out


def kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes=2):
    return int(lib().gqa_oracle_kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes))


def bf16_to_double(bits):
    return lib().gqa_oracle_bf16_to_double(int(bits))


def fp8_e4m3_to_double(code):
    return lib().gqa_oracle_fp8_e4m3_to_double(int(code))


def encode_bf16(x):
    """bf16 bit pattern of the binary32 value x (round to nearest even)."""
    return int(lib().gqa_oracle_encode_bf16(float(np.float32(x))))


def encode_fp8_e4m3(x, descale=1.0):
    """e4m3fn code of binary32 x / descale (nearest finite value, ties to even, saturating)."""
    return int(lib().gqa_oracle_encode_fp8_e4m3(float(np.float32(x)), float(np.float32(descale))))


def append(k_new, v_new, new_dtype, k_cache, v_cache, kv_dtype, positions, k_descale=1.0, v_descale=1.0,
           block_table=None):
    """Writes the new rows into numpy copies of the caches; returns (k_cache, v_cache, skipped).

    k_new, v_new: [B, Hkv, d] in new_dtype ("f32" or "bf16"); caches dense [B, Hkv, L, d] or, with a
    block_table [B, max_blocks], pages [num_blocks, Hkv, block_size, d]."""
    kn, vn = raw(k_new, new_dtype), raw(v_new, new_dtype)
    kc, vc = raw(k_cache, kv_dtype).copy(), raw(v_cache, kv_dtype).copy()
    B, Hkv, d = kn.shape
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32).reshape(-1))
    if pos.shape[0] != B or vn.shape != kn.shape or vc.shape != kc.shape:
        raise ValueError("shape mismatch")
    if block_table is None:
        L, bt, bs, mb, nb = kc.shape[2], None, 0, 0, 0
    else:
        bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
        nb, bs, mb = kc.shape[0], kc.shape[2], bt.shape[1]
        L = bs * mb
    rc = lib().gqa_oracle_append(kn.ctypes.data, vn.ctypes.data, DTYPES[new_dtype], kc.ctypes.data,
                                 vc.ctypes.data, DTYPES[kv_dtype], float(k_descale), float(v_descale),
                                 pos.ctypes.data, B, Hkv, L, d, None if bt is None else bt.ctypes.data,
                                 bs, mb, nb)
    if rc < 0:
        raise ValueError("oracle: bad append arguments")
    return kc, vc, rc


def prefill(q, k, v, scale, dtype="bf16", causal=True, rows=None, threads=1):
    """Prefill attention: q [B,Hq,S,d], k, v [B,Hkv,S,d] (raw storage of dtype).  Returns out
    [B,Hq,S,d] (rows None) or [len(rows), d] for the listed (b, h, i) triples, float64; rows "all"
    computes every row through the row path (on `threads` threads) and returns [B,Hq,S,d]."""
    qa, ka, va = raw(q, dtype), raw(k, dtype), raw(v, dtype)
    if qa.ndim != 4 or ka.ndim != 4 or va.shape != ka.shape:
        raise ValueError("q must be [B,Hq,S,d]; k and v [B,Hkv,S,d]")
    B, Hq, S, d = qa.shape
    Bk, Hkv, Sk, dk = ka.shape
    if (Bk, Sk, dk) != (B, S, d):
        raise ValueError("q and k/v disagree on B, S or d")
    every = isinstance(rows, str) and rows == "all"
    if every:
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(S), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
    if rows is None:
        r, nrows, out = None, 0, np.zeros((B, Hq, S, d), dtype=np.float64)
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
        nrows, out = r.shape[0], np.zeros((r.shape[0], d), dtype=np.float64)

    def chunk(lo, hi):
        w = np.zeros(max(S, 1), dtype=np.float64)
        return lib().gqa_oracle_prefill(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, DTYPES[dtype],
                                        float(scale), 1 if causal else 0, B, Hq, Hkv, S, d,
                                        None if r is None else r[lo:hi].ctypes.data, hi - lo, w.ctypes.data,
                                        out[lo:hi].ctypes.data if r is not None else out.ctypes.data)

    _raise(chunk(0, 0) if r is None else _run_chunks(nrows, threads, chunk))
    del qa, ka, va
    return out.reshape(B, Hq, S, d) if every else out
