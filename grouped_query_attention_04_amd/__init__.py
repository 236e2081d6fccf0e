"""Python binding of libgqa (single-token grouped-query-attention decode on MI355X).

Argument marshalling only: every step of the decode runs in the HIP kernels of ``libgqa.so``; torch
supplies device memory and the current stream.  The library must have been built
(``python grouped_query_attention_04_amd/build.py``); importing this package without it raises.

``decode`` computes, for each batch entry b and query head h with G = Hq // Hkv,
``out[b, h] = softmax(scale * q[b, h] . k_cache[b, h // G, :n]) @ v_cache[b, h // G, :n]`` with
``n = seq_lens[b]`` -- scaled dot-product attention per query head, contiguous groups of G query heads
sharing one KV head ("Grouped-Query Attention: How Sharing KV Heads Shrinks Inference Memory",
section "How grouped-query attention works").  ``decode_paged`` computes the same over a cache kept in
fixed-size pages addressed through a block table.
"""
import ctypes
import math
import os

import torch  # loaded first: libgqa then binds to the HIP runtime torch already mapped

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgqa.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3}
STATUS = {0: "GQA_OK", 1: "GQA_ERR_INVALID_ARG", 2: "GQA_ERR_UNSUPPORTED", 3: "GQA_ERR_WORKSPACE",
          4: "GQA_ERR_HIP"}


class GqaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(msg)
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("L", ctypes.c_int32), ("d", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("k_descale", ctypes.c_float), ("v_descale", ctypes.c_float),
                ("num_workgroups", ctypes.c_int32)]


class PrefillShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("S", ctypes.c_int32), ("d", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("causal", ctypes.c_int32)]


class TpRank(ctypes.Structure):
    _fields_ = [("q_head_begin", ctypes.c_int32), ("q_head_end", ctypes.c_int32),
                ("kv_head_begin", ctypes.c_int32), ("kv_head_end", ctypes.c_int32)]


class PagedShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("k_descale", ctypes.c_float), ("v_descale", ctypes.c_float),
                ("num_workgroups", ctypes.c_int32)]


EXPORTS = ["gqa_shape_check", "gqa_decode_workspace_bytes", "gqa_workspace_init", "gqa_decode",
           "gqa_decode_static",
           "gqa_paged_shape_check", "gqa_decode_paged_workspace_bytes", "gqa_paged_workspace_init",
           "gqa_decode_paged", "gqa_append_kv", "gqa_append_kv_paged", "gqa_decode_append",
           "gqa_decode_append_paged", "gqa_prefill_shape_check",
           "gqa_prefill", "gqa_tp_plan",
           "gqa_max_concurrency", "gqa_max_cached_tokens", "gqa_kv_bytes_per_token", "gqa_validate_seq_lens", "gqa_stream_read",
           "gqa_stream_read_sink_words", "gqa_status_string"]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python grouped_query_attention_04_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz, pS = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.POINTER(Shape)
    lib.gqa_shape_check.argtypes = [pS]
    lib.gqa_shape_check.restype = ctypes.c_int
    lib.gqa_decode_workspace_bytes.argtypes = [pS]
    lib.gqa_decode_workspace_bytes.restype = sz
    lib.gqa_workspace_init.argtypes = [vp, sz, pS, vp]
    lib.gqa_workspace_init.restype = ctypes.c_int
    lib.gqa_decode.argtypes = [vp, vp, vp, vp, ctypes.c_float, vp, pS, vp, sz, vp]
    lib.gqa_decode.restype = ctypes.c_int
    lib.gqa_decode_static.argtypes = [vp, vp, vp, vp, ctypes.c_float, vp, pS, vp]
    lib.gqa_decode_static.restype = ctypes.c_int
    pP = ctypes.POINTER(PagedShape)
    lib.gqa_paged_shape_check.argtypes = [pP]
    lib.gqa_paged_shape_check.restype = ctypes.c_int
    lib.gqa_decode_paged_workspace_bytes.argtypes = [pP]
    lib.gqa_decode_paged_workspace_bytes.restype = sz
    lib.gqa_paged_workspace_init.argtypes = [vp, sz, pP, vp]
    lib.gqa_paged_workspace_init.restype = ctypes.c_int
    lib.gqa_decode_paged.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, pP, vp, sz, vp]
    lib.gqa_decode_paged.restype = ctypes.c_int
    lib.gqa_append_kv.argtypes = [vp, vp, i32, vp, vp, pS, vp, vp, vp]
    lib.gqa_append_kv.restype = ctypes.c_int
    lib.gqa_append_kv_paged.argtypes = [vp, vp, i32, vp, vp, vp, pP, vp, vp, vp]
    lib.gqa_append_kv_paged.restype = ctypes.c_int
    lib.gqa_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, pS, vp, vp, sz, vp]
    lib.gqa_decode_append.restype = ctypes.c_int
    lib.gqa_decode_append_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, pP, vp, vp, sz, vp]
    lib.gqa_decode_append_paged.restype = ctypes.c_int
    pF = ctypes.POINTER(PrefillShape)
    lib.gqa_prefill_shape_check.argtypes = [pF]
    lib.gqa_prefill_shape_check.restype = ctypes.c_int
    lib.gqa_prefill.argtypes = [vp, vp, vp, ctypes.c_float, vp, pF, vp]
    lib.gqa_prefill.restype = ctypes.c_int
    u64 = ctypes.c_uint64
    lib.gqa_tp_plan.argtypes = [i32, i32, i32, ctypes.POINTER(TpRank), ctypes.POINTER(i32)]
    lib.gqa_tp_plan.restype = ctypes.c_int
    lib.gqa_max_concurrency.argtypes = [u64, u64, u64]
    lib.gqa_max_concurrency.restype = u64
    lib.gqa_max_cached_tokens.argtypes = [u64, u64]
    lib.gqa_max_cached_tokens.restype = u64
    lib.gqa_kv_bytes_per_token.argtypes = [ctypes.c_uint32] * 4
    lib.gqa_kv_bytes_per_token.restype = ctypes.c_uint64
    lib.gqa_validate_seq_lens.argtypes = [vp, i32, i32, vp, vp]
    lib.gqa_validate_seq_lens.restype = ctypes.c_int
    lib.gqa_stream_read.argtypes = [vp, sz, vp, vp]
    lib.gqa_stream_read.restype = ctypes.c_int
    lib.gqa_stream_read_sink_words.argtypes = []
    lib.gqa_stream_read_sink_words.restype = sz
    lib.gqa_status_string.argtypes = [ctypes.c_int]
    lib.gqa_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def _check(code):
    if code != 0:
        raise GqaError(code, lib.gqa_status_string(code).decode())


def status_string(code: int) -> str:
    return lib.gqa_status_string(int(code)).decode()


def make_shape(B, Hq, Hkv, L, d, q_dtype=BF16, kv_dtype=BF16, out_dtype=None, k_descale=1.0,
               v_descale=1.0, num_workgroups=0) -> Shape:
    return Shape(B, Hq, Hkv, L, d, q_dtype, kv_dtype, q_dtype if out_dtype is None else out_dtype,
                 k_descale, v_descale, num_workgroups)


def make_paged_shape(B, Hq, Hkv, d, block_size, max_blocks, num_blocks, q_dtype=BF16, kv_dtype=BF16,
                     out_dtype=None, k_descale=1.0, v_descale=1.0, num_workgroups=0) -> PagedShape:
    return PagedShape(B, Hq, Hkv, d, block_size, max_blocks, num_blocks, q_dtype, kv_dtype,
                      q_dtype if out_dtype is None else out_dtype, k_descale, v_descale, num_workgroups)


def shape_check(shape) -> int:
    if isinstance(shape, PagedShape):
        return lib.gqa_paged_shape_check(ctypes.byref(shape))
    return lib.gqa_shape_check(ctypes.byref(shape))


def workspace_bytes(shape) -> int:
    if isinstance(shape, PagedShape):
        return lib.gqa_decode_paged_workspace_bytes(ctypes.byref(shape))
    return lib.gqa_decode_workspace_bytes(ctypes.byref(shape))


def kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes=2) -> int:
    return int(lib.gqa_kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes))


def tp_plan(num_q_heads, num_kv_heads, tp_size):
    """Per-rank (q_begin, q_end, kv_begin, kv_end) and the KV heads held over all ranks."""
    ranks = (TpRank * max(int(tp_size), 1))()
    held = ctypes.c_int32(0)
    _check(lib.gqa_tp_plan(int(num_q_heads), int(num_kv_heads), int(tp_size), ranks, ctypes.byref(held)))
    return [(r.q_head_begin, r.q_head_end, r.kv_head_begin, r.kv_head_end) for r in ranks[:tp_size]], held.value


def max_concurrency(free_bytes, bytes_per_token, context_tokens) -> int:
    return int(lib.gqa_max_concurrency(int(free_bytes), int(bytes_per_token), int(context_tokens)))


def max_cached_tokens(free_bytes, bytes_per_token) -> int:
    return int(lib.gqa_max_cached_tokens(int(free_bytes), int(bytes_per_token)))


def _stream_handle(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_workspaces = {}


def init_workspace(ws: torch.Tensor, shape) -> torch.Tensor:
    """Initialises a workspace tensor (uint8, on the device) with gqa_workspace_init on torch's
    current stream: the counter area cleared and the header tag written.  Returns ws."""
    with torch.cuda.device(ws.device):
        if isinstance(shape, PagedShape):
            rc = lib.gqa_paged_workspace_init(ws.data_ptr(), ws.numel(), ctypes.byref(shape),
                                              _stream_handle(ws.device))
        else:
            rc = lib.gqa_workspace_init(ws.data_ptr(), ws.numel(), ctypes.byref(shape),
                                        _stream_handle(ws.device))
    _check(rc)
    return ws


def new_workspace(shape, device, nbytes=None) -> torch.Tensor:
    """A fresh workspace of max(nbytes, the shape's requirement) bytes, initialised."""
    need = workspace_bytes(shape)
    if need == 0:
        _check(shape_check(shape))
    ws = torch.empty(max(need, nbytes or 0, 256), dtype=torch.uint8, device=device)
    return init_workspace(ws, shape)


def workspace_errors(ws: torch.Tensor) -> int:
    """Workgroups that refused this workspace for a missing header tag since its initialisation
    (header word 2; reading it synchronises with the device)."""
    return int(ws[8:12].view(torch.int32).item())


def workspace_for(shape, device) -> torch.Tensor:
    """A workspace cached per (device, stream), initialised when allocated and replaced by a larger
    one when a shape needs more.  The library leaves its counters at zero after every call, so one
    buffer serves every shape.  Calls that overlap in time on different streams get different
    buffers."""
    need = workspace_bytes(shape)
    if need == 0:
        _check(shape_check(shape))
    dev = torch.device(device)
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = new_workspace(shape, dev)
        _workspaces[key] = ws
    return ws


def _shape_from(q, k_cache, out_dtype, k_descale, v_descale, num_workgroups):
    B, Hq, d = q.shape
    _, Hkv, L, _ = k_cache.shape
    if q.dtype not in _CODE or k_cache.dtype not in _CODE or out_dtype not in _CODE:
        raise TypeError(f"unsupported dtypes q={q.dtype} kv={k_cache.dtype} out={out_dtype}")
    return make_shape(B, Hq, Hkv, L, d, _CODE[q.dtype], _CODE[k_cache.dtype], _CODE[out_dtype],
                      k_descale, v_descale, num_workgroups)


def decode(q, k_cache, v_cache, seq_lens, scale=None, out=None, *, out_dtype=None, k_descale=1.0,
           v_descale=1.0, num_workgroups=0, workspace=None):
    """Single-token GQA decode.  q [B,Hq,d]; k_cache, v_cache [B,Hkv,L,d]; seq_lens [B] int32;
    all contiguous CUDA tensors on one device.  Returns out [B,Hq,d] (dtype out_dtype, default q's).
    scale defaults to 1/sqrt(d).  num_workgroups (0 = library's choice) sets how many workgroups
    split the cache.  Enqueued on torch's current stream; no synchronisation."""
    return _decode(q, k_cache, v_cache, seq_lens, scale, out, out_dtype, k_descale, v_descale,
                   num_workgroups, workspace, None)


def decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, scale=None, out=None, *, out_dtype=None,
                  k_descale=1.0, v_descale=1.0, num_workgroups=0, workspace=None, skipped=None):
    """append_kv and decode in one launch.  k_new, v_new [B,Hkv,d] bf16 go to position
    seq_lens[b] - 1 of the dense caches [B,Hkv,L,d] (bf16 or fp8-e4m3: the code of x / descale), and
    the decode then attends over the first seq_lens[b] positions; q must be bf16.  The cache and the
    output equal those of append_kv(positions=seq_lens - 1) followed by decode.  A new position past
    the cache adds one to skipped (an int32 device tensor) if given.  Returns out."""
    return _decode(q, k_cache, v_cache, seq_lens, scale, out, out_dtype, k_descale, v_descale,
                   num_workgroups, workspace, (k_new, v_new, skipped))


def _check_new_rows(new, B, Hkv, d):
    k_new, v_new, skipped = new
    if skipped is not None and (skipped.dtype != torch.int32 or skipped.numel() < 1):
        raise ValueError("skipped must be an int32 tensor with at least one element")
    if k_new.shape != (B, Hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [B, Hkv, d] matching the cache")
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise TypeError("the fused append takes bfloat16 new rows")
    return [k_new, v_new] + ([skipped] if skipped is not None else [])


def _new_ptrs(new):
    if new is None:
        return ()
    k_new, v_new, skipped = new
    return k_new.data_ptr(), v_new.data_ptr(), None if skipped is None else skipped.data_ptr()


def _decode(q, k_cache, v_cache, seq_lens, scale, out, out_dtype, k_descale, v_descale, num_workgroups,
            workspace, new):
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,Hq,d], k_cache and v_cache [B,Hkv,L,d]")
    if k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must share a dtype")
    B, Hq, d = q.shape
    if k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError("batch size or head dim of q and the cache differ")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be an int32 tensor of shape [B]")
    tensors = [q, k_cache, v_cache, seq_lens] + ([out] if out is not None else [])
    if new is not None:
        tensors += _check_new_rows(new, B, k_cache.shape[1], d)
    dev = q.device
    if dev.type != "cuda" or any(t.device != dev for t in tensors):
        raise ValueError("all tensors must live on one CUDA (HIP) device")
    if any(not t.is_contiguous() for t in tensors):
        raise ValueError("all tensors must be contiguous")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else q.dtype
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype, device=dev)
    elif out.shape != (B, Hq, d) or out.dtype != out_dtype:
        raise ValueError("out must be [B,Hq,d] of dtype out_dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    shape = _shape_from(q, k_cache, out_dtype, k_descale, v_descale, num_workgroups)
    ws = workspace if workspace is not None else workspace_for(shape, dev)
    with torch.cuda.device(dev):
        if new is None:
            _check(lib.gqa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                  seq_lens.data_ptr(), float(scale), out.data_ptr(),
                                  ctypes.byref(shape), ws.data_ptr(), ws.numel(), _stream_handle(dev)))
        else:
            kn, vn, sk = _new_ptrs(new)
            _check(lib.gqa_decode_append(q.data_ptr(), kn, vn, k_cache.data_ptr(), v_cache.data_ptr(),
                                         seq_lens.data_ptr(), float(scale), out.data_ptr(),
                                         ctypes.byref(shape), sk, ws.data_ptr(), ws.numel(),
                                         _stream_handle(dev)))
    return out


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale=None, out=None, *, out_dtype=None,
                 k_descale=1.0, v_descale=1.0, num_workgroups=0, workspace=None):
    """Single-token GQA decode over a paged cache.  q [B,Hq,d]; k_pages, v_pages
    [num_blocks,Hkv,block_size,d] (bf16 or fp8-e4m3); block_table [B,max_blocks] int32 (position t of
    sequence b is row t % block_size of page block_table[b, t // block_size]); seq_lens [B] int32.
    Returns out [B,Hq,d].  Enqueued on torch's current stream; no synchronisation."""
    return _decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale, out, out_dtype, k_descale,
                         v_descale, num_workgroups, workspace, None)


def decode_append_paged(q, k_new, v_new, k_pages, v_pages, block_table, seq_lens, scale=None, out=None, *,
                        out_dtype=None, k_descale=1.0, v_descale=1.0, num_workgroups=0, workspace=None,
                        skipped=None):
    """decode_append for a paged cache: append_kv_paged(positions=seq_lens - 1) and decode_paged in
    one launch.  A new position past max_blocks * block_size, or on a page outside the pool, adds one
    to skipped if given.  Returns out."""
    return _decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale, out, out_dtype, k_descale,
                         v_descale, num_workgroups, workspace, (k_new, v_new, skipped))


def _decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale, out, out_dtype, k_descale, v_descale,
                  num_workgroups, workspace, new):
    if q.dim() != 3 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("expected q [B,Hq,d], k_pages and v_pages [num_blocks,Hkv,block_size,d]")
    if k_pages.dtype != v_pages.dtype:
        raise ValueError("k_pages and v_pages must share a dtype")
    B, Hq, d = q.shape
    num_blocks, Hkv, block_size, dk = k_pages.shape
    if dk != d:
        raise ValueError("head dim of q and the pages differ")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be an int32 tensor of shape [B, max_blocks]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be an int32 tensor of shape [B]")
    tensors = [q, k_pages, v_pages, block_table, seq_lens] + ([out] if out is not None else [])
    if new is not None:
        tensors += _check_new_rows(new, B, Hkv, d)
    dev = q.device
    if dev.type != "cuda" or any(t.device != dev for t in tensors):
        raise ValueError("all tensors must live on one CUDA (HIP) device")
    if any(not t.is_contiguous() for t in tensors):
        raise ValueError("all tensors must be contiguous")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else q.dtype
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype, device=dev)
    elif out.shape != (B, Hq, d) or out.dtype != out_dtype:
        raise ValueError("out must be [B,Hq,d] of dtype out_dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if q.dtype not in _CODE or k_pages.dtype not in _CODE or out_dtype not in _CODE:
        raise TypeError(f"unsupported dtypes q={q.dtype} kv={k_pages.dtype} out={out_dtype}")
    shape = make_paged_shape(B, Hq, Hkv, d, block_size, block_table.shape[1], num_blocks,
                             _CODE[q.dtype], _CODE[k_pages.dtype], _CODE[out_dtype], k_descale,
                             v_descale, num_workgroups)
    ws = workspace if workspace is not None else workspace_for(shape, dev)
    with torch.cuda.device(dev):
        if new is None:
            _check(lib.gqa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                                        block_table.data_ptr(), seq_lens.data_ptr(), float(scale),
                                        out.data_ptr(), ctypes.byref(shape), ws.data_ptr(), ws.numel(),
                                        _stream_handle(dev)))
        else:
            kn, vn, sk = _new_ptrs(new)
            _check(lib.gqa_decode_append_paged(q.data_ptr(), kn, vn, k_pages.data_ptr(), v_pages.data_ptr(),
                                               block_table.data_ptr(), seq_lens.data_ptr(), float(scale),
                                               out.data_ptr(), ctypes.byref(shape), sk, ws.data_ptr(),
                                               ws.numel(), _stream_handle(dev)))
    return out


def _check_append(k_new, v_new, positions, tensors, B, Hkv, d, cache_dtype=None, skipped=None):
    if cache_dtype is not None and cache_dtype not in _CODE:
        raise TypeError(f"unsupported cache dtype {cache_dtype}")
    if skipped is not None and (skipped.dtype != torch.int32 or skipped.numel() < 1):
        raise ValueError("skipped must be an int32 tensor with at least one element")
    if k_new.shape != (B, Hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [B, Hkv, d] matching the cache")
    if k_new.dtype not in (torch.float32, torch.bfloat16) or v_new.dtype != k_new.dtype:
        raise TypeError("new rows must both be float32 or both bfloat16")
    if positions.dtype != torch.int32 or positions.shape != (B,):
        raise ValueError("positions must be an int32 tensor of shape [B]")
    dev = k_new.device
    if dev.type != "cuda" or any(t.device != dev for t in tensors):
        raise ValueError("all tensors must live on one CUDA (HIP) device")
    if any(not t.is_contiguous() for t in tensors):
        raise ValueError("all tensors must be contiguous")
    return dev


def append_kv(k_new, v_new, k_cache, v_cache, positions, *, k_descale=1.0, v_descale=1.0, skipped=None):
    """Writes row (b, j) of k_new / v_new [B,Hkv,d] into the dense caches [B,Hkv,L,d] at position
    positions[b] (int32 [B]; negative = skip), converted to the cache dtype (fp8: code of x / descale).
    Positions past the cache add one to skipped (an int32 [1] device tensor) if given."""
    B, Hkv, L, d = k_cache.shape
    tensors = [k_new, v_new, k_cache, v_cache, positions] + ([skipped] if skipped is not None else [])
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    dev = _check_append(k_new, v_new, positions, tensors, B, Hkv, d, k_cache.dtype, skipped)
    q_code = F32 if k_cache.dtype == torch.float32 else BF16
    shape = make_shape(B, Hkv, Hkv, L, d, q_code, _CODE[k_cache.dtype], q_code, k_descale, v_descale)
    with torch.cuda.device(dev):
        _check(lib.gqa_append_kv(k_new.data_ptr(), v_new.data_ptr(), _CODE[k_new.dtype], k_cache.data_ptr(),
                                 v_cache.data_ptr(), ctypes.byref(shape), positions.data_ptr(),
                                 None if skipped is None else skipped.data_ptr(), _stream_handle(dev)))


def append_kv_paged(k_new, v_new, k_pages, v_pages, block_table, positions, *, k_descale=1.0, v_descale=1.0,
                    skipped=None):
    """append_kv for a paged cache: pages [num_blocks,Hkv,block_size,d], block_table [B,max_blocks]."""
    num_blocks, Hkv, block_size, d = k_pages.shape
    B = positions.shape[0]
    tensors = [k_new, v_new, k_pages, v_pages, block_table, positions] + ([skipped] if skipped is not None else [])
    if v_pages.shape != k_pages.shape or v_pages.dtype != k_pages.dtype:
        raise ValueError("k_pages and v_pages must match")
    dev = _check_append(k_new, v_new, positions, tensors, B, Hkv, d, k_pages.dtype, skipped)
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be an int32 tensor of shape [B, max_blocks]")
    q_code = BF16
    shape = make_paged_shape(B, Hkv, Hkv, d, block_size, block_table.shape[1], num_blocks, q_code,
                             _CODE[k_pages.dtype], q_code, k_descale, v_descale)
    with torch.cuda.device(dev):
        _check(lib.gqa_append_kv_paged(k_new.data_ptr(), v_new.data_ptr(), _CODE[k_new.dtype],
                                       k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                                       ctypes.byref(shape), positions.data_ptr(),
                                       None if skipped is None else skipped.data_ptr(), _stream_handle(dev)))


def prefill(q, k, v, scale=None, out=None, *, out_dtype=None, causal=True):
    """GQA attention of a prompt over itself: q [B,Hq,S,d], k, v [B,Hkv,S,d] (bf16, contiguous, one
    device).  Query position i of head h attends to positions <= i (all, if not causal) of KV head
    h // (Hq // Hkv).  Returns out [B,Hq,S,d] (dtype out_dtype, default bf16).  scale defaults to
    1/sqrt(d).  Enqueued on torch's current stream."""
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,Hq,S,d], k and v [B,Hkv,S,d]")
    B, Hq, S, d = q.shape
    if k.shape[0] != B or k.shape[2] != S or k.shape[3] != d:
        raise ValueError("q and k/v disagree on B, S or d")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("prefill takes bfloat16 q, k and v")
    tensors = [q, k, v] + ([out] if out is not None else [])
    dev = q.device
    if dev.type != "cuda" or any(t.device != dev for t in tensors):
        raise ValueError("all tensors must live on one CUDA (HIP) device")
    if any(not t.is_contiguous() for t in tensors):
        raise ValueError("all tensors must be contiguous")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"prefill writes bfloat16 or float32, not {out_dtype}")
    if out is None:
        out = torch.empty((B, Hq, S, d), dtype=out_dtype, device=dev)
    elif out.shape != (B, Hq, S, d) or out.dtype != out_dtype:
        raise ValueError("out must be [B,Hq,S,d] of dtype out_dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    shape = PrefillShape(B, Hq, k.shape[1], S, d, BF16, _CODE[out_dtype], 1 if causal else 0)
    with torch.cuda.device(dev):
        _check(lib.gqa_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), float(scale), out.data_ptr(),
                               ctypes.byref(shape), _stream_handle(dev)))
    return out


def validate_seq_lens(seq_lens, L) -> int:
    """Number of entries outside [0, L] (synchronises)."""
    if seq_lens.dtype != torch.int32 or seq_lens.device.type != "cuda" or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 CUDA (HIP) tensor")
    bad = torch.zeros(1, dtype=torch.int32, device=seq_lens.device)
    with torch.cuda.device(seq_lens.device):
        _check(lib.gqa_validate_seq_lens(seq_lens.data_ptr(), seq_lens.numel(), int(L),
                                         bad.data_ptr(), _stream_handle(seq_lens.device)))
    return int(bad.item())


def stream_read(src: torch.Tensor, sink: torch.Tensor = None):
    """Calibration read of every byte of src (non-temporal 16-byte loads)."""
    if src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous CUDA (HIP) tensor")
    if sink is None:
        sink = torch.empty(lib.gqa_stream_read_sink_words(), dtype=torch.int32, device=src.device)
    nbytes = src.numel() * src.element_size()
    with torch.cuda.device(src.device):
        _check(lib.gqa_stream_read(src.data_ptr(), nbytes, sink.data_ptr(),
                                   _stream_handle(src.device)))
    return sink
