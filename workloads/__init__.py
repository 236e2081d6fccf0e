"""Seeded synthetic inputs for single-token GQA decode.

This module only draws random numbers and casts them to the storage dtypes; it holds none of the
attention arithmetic.  The CPU oracle and the HIP library both receive exactly the bytes made here.

Recipe (all five workloads): a CPU ``torch.Generator`` seeded with ``1000 + workload id`` (or the seed
passed in) draws, in this order, the sequence lengths (``randint`` over an inclusive range, when they
are random), then q, K and V as float32 standard normals; the values are then cast with
round-to-nearest-even to the storage dtype.  The fp8-e4m3fn cache is clipped to [-4, 4] first and
stored with per-tensor descale 1.0.  Cache positions at or beyond a sequence's length hold the same
normal draws and are never read by a correct kernel.

Paged variants (``paginate``) move the same bytes into page pools placed by a seeded permutation.
"""
import math
from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple

import torch

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.float8_e4m3fn}
FP8_CLIP = 4.0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    L: int
    q_dtype: str
    kv_dtype: str
    seq_lens: Optional[Tuple[int, ...]] = None   # fixed lengths, or
    seq_range: Optional[Tuple[int, int]] = None  # inclusive uniform range
    seed: int = 0
    note: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def out_dtype(self) -> str:
        return self.q_dtype

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    1: Workload("tiny-fp32 B2 Hq8 Hkv2 d64 L256", 2, 8, 2, 64, 256, "f32", "f32",
                seq_lens=(256, 190), seed=1001),
    2: Workload("llama3-8b-layer B16 Hq32 Hkv8 d128 L2600", 16, 32, 8, 128, 2600, "bf16", "bf16",
                seq_range=(2000, 2600), seed=1002),
    3: Workload("llama-70b-layer B32 Hq64 Hkv8 d128 L8192", 32, 64, 8, 128, 8192, "bf16", "bf16",
                seq_range=(6000, 8192), seed=1003),
    "4-mha": Workload("sweep B8 Hq32 Hkv32 d128 L4096", 8, 32, 32, 128, 4096, "bf16", "bf16",
                      seq_lens=(4096,) * 8, seed=1004),
    "4-gqa": Workload("sweep B8 Hq32 Hkv8 d128 L4096", 8, 32, 8, 128, 4096, "bf16", "bf16",
                      seq_lens=(4096,) * 8, seed=1004),
    "4-mqa": Workload("sweep B8 Hq32 Hkv1 d128 L4096", 8, 32, 1, 128, 4096, "bf16", "bf16",
                      seq_lens=(4096,) * 8, seed=1004),
    # the group-size sweep's shape with all 64 query heads of a 70B-class model on one KV head (the
    # multi-query end of the 70B grouping)
    "4-mqa64": Workload("sweep B8 Hq64 Hkv1 d128 L4096", 8, 64, 1, 128, 4096, "bf16", "bf16",
                        seq_lens=(4096,) * 8, seed=1004),
    5: Workload("long-fp8 B2 Hq64 Hkv8 d128 L32768", 2, 64, 8, 128, 32768, "bf16", "fp8_e4m3",
                seq_lens=(32768, 30000), seed=1005),
    # one rank's share of the 70B-layer step under tensor parallelism of degree 8: one KV head and
    # its 8 query heads per GPU; same seed, so the same sequence lengths as the whole step
    "3-tp8": Workload("llama-70b-layer tp8-rank B32 Hq8 Hkv1 d128 L8192", 32, 8, 1, 128, 8192, "bf16", "bf16",
                      seq_range=(6000, 8192), seed=1003),
    # the same step with head dim 64 (the other supported head size): half the bytes per token
    "3-d64": Workload("llama-70b-layer head-dim-64 B32 Hq64 Hkv8 d64 L8192", 32, 64, 8, 64, 8192, "bf16", "bf16",
                      seq_range=(6000, 8192), seed=1003),
}


def cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "fp8_e4m3":
        x = x.clamp(-FP8_CLIP, FP8_CLIP)
    return x.to(TORCH_DTYPES[dtype])


def make_case(B: int, Hq: int, Hkv: int, d: int, L: int, q_dtype: str = "bf16",
              kv_dtype: str = "bf16", seq_lens: Optional[Sequence[int]] = None,
              seq_range: Optional[Tuple[int, int]] = None, seed: int = 0) -> dict:
    """Draw one decode problem on the CPU.  Returns a dict of CPU tensors and metadata."""
    g = torch.Generator().manual_seed(int(seed))
    if seq_lens is None:
        lo, hi = seq_range if seq_range is not None else (0, L)
        sl = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    else:
        sl = torch.tensor(list(seq_lens), dtype=torch.int32)
    q = torch.randn(B, Hq, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, Hkv, L, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, Hkv, L, d, generator=g, dtype=torch.float32)
    return {
        "q": cast(q, q_dtype), "k": cast(k, kv_dtype), "v": cast(v, kv_dtype), "seq_lens": sl,
        "scale": 1.0 / math.sqrt(d), "k_descale": 1.0, "v_descale": 1.0,
        "q_dtype": q_dtype, "kv_dtype": kv_dtype, "out_dtype": q_dtype,
        "B": B, "Hq": Hq, "Hkv": Hkv, "d": d, "L": L,
    }


POISON_BITS = {"f32": 0x7FC00000, "bf16": 0x7FC0, "fp8_e4m3": 0x7F}   # a NaN in each storage format


def poison_like(shape, dtype: str) -> torch.Tensor:
    """A tensor of the storage dtype whose every element is NaN (never read by a correct kernel)."""
    if dtype == "f32":
        return torch.full(shape, POISON_BITS["f32"], dtype=torch.int32).view(torch.float32)
    if dtype == "bf16":
        return torch.full(shape, POISON_BITS["bf16"], dtype=torch.int16).view(torch.bfloat16)
    return torch.full(shape, POISON_BITS["fp8_e4m3"], dtype=torch.uint8).view(torch.float8_e4m3fn)


def paginate(case: dict, block_size: int, seed: int = 0, spare_pages: int = 0,
             dead_entry: int = -1) -> dict:
    """Copy a dense case's cache into page pools with a seeded random page placement.

    Sequence b needs ceil(seq_lens[b] / block_size) pages; those pages, plus spare_pages unused
    ones, are placed at the positions of a random permutation of the pool.  Pools are
    [num_blocks, Hkv, block_size, d]; position t of sequence b goes to row t % block_size of page
    block_table[b, t // block_size].  Page rows past the dense cache's length, and the spare pages,
    hold NaN.  Table entries of pages a sequence does not use hold dead_entry.  Adds k_pages, v_pages,
    block_table (int32 [B, max_blocks]), block_size and num_blocks to a copy of the case."""
    k, v, sl = case["k"], case["v"], case["seq_lens"]
    B, Hkv, L, d = k.shape
    dt = case["kv_dtype"]
    max_blocks = -(-L // block_size)
    live = [-(-int(n) // block_size) for n in sl.tolist()]
    num_blocks = sum(live) + spare_pages
    g = torch.Generator().manual_seed(int(seed))
    perm = torch.randperm(num_blocks, generator=g).tolist()
    kp = poison_like((num_blocks, Hkv, block_size, d), dt)
    vp = poison_like((num_blocks, Hkv, block_size, d), dt)
    table = torch.full((B, max_blocks), int(dead_entry), dtype=torch.int32)
    nxt = 0
    for b in range(B):
        for i in range(live[b]):
            page = perm[nxt]
            nxt += 1
            table[b, i] = page
            lo, hi = i * block_size, min((i + 1) * block_size, L)
            kp[page, :, : hi - lo] = k[b, :, lo:hi]
            vp[page, :, : hi - lo] = v[b, :, lo:hi]
    out = dict(case)
    out.update(k_pages=kp, v_pages=vp, block_table=table, block_size=block_size,
               num_blocks=num_blocks)
    return out


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    S: int
    seed: int

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def flops(self) -> int:
        """Causal prefill matmul flops: 2 * d for Q K^T and 2 * d for P V per (head, query, visible key)."""
        return 4 * self.d * self.B * self.Hq * self.S * (self.S + 1) // 2


# Prefill shapes: the scaled_dot_product_attention example's q [b, 32, s, 128] / kv [b, 8, s, 128]
# (an 8B-class layer) and the 70B-class grouping (64 query heads, 8 KV heads).
PREFILL_WORKLOADS = {
    "prefill-8b": PrefillWorkload("prefill llama3-8b-layer B2 Hq32 Hkv8 d128 S4096", 2, 32, 8, 128, 4096, seed=1101),
    "prefill-70b": PrefillWorkload("prefill llama-70b-layer B1 Hq64 Hkv8 d128 S8192", 1, 64, 8, 128, 8192, seed=1102),
    # 40 query heads on 8 KV heads: a group of 5, which does not divide a workgroup's 256 rows
    "prefill-40b": PrefillWorkload("prefill 40b-class-layer B1 Hq40 Hkv8 d128 S4096", 1, 40, 8, 128, 4096, seed=1103),
}


def make_prefill_case(B: int, Hq: int, Hkv: int, d: int, S: int, seed: int = 0) -> dict:
    """q [B,Hq,S,d], k and v [B,Hkv,S,d]: float32 standard normals drawn in that order from a CPU
    generator seeded with `seed`, cast to bf16 with round-to-nearest-even."""
    g = torch.Generator().manual_seed(int(seed))
    q = torch.randn(B, Hq, S, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, Hkv, S, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, Hkv, S, d, generator=g, dtype=torch.float32)
    return {"q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16), "v": v.to(torch.bfloat16),
            "scale": 1.0 / math.sqrt(d), "B": B, "Hq": Hq, "Hkv": Hkv, "S": S, "d": d}


def make_prefill(name: str) -> dict:
    w = PREFILL_WORKLOADS[name]
    case = make_prefill_case(w.B, w.Hq, w.Hkv, w.d, w.S, w.seed)
    case["workload"] = w
    return case


def make(wid, seed: Optional[int] = None) -> dict:
    """Inputs of one named workload (ids 1, 2, 3, '4-mha', '4-gqa', '4-mqa', 5)."""
    w = WORKLOADS[wid]
    case = make_case(w.B, w.Hq, w.Hkv, w.d, w.L, w.q_dtype, w.kv_dtype, seq_lens=w.seq_lens,
                     seq_range=w.seq_range, seed=w.seed if seed is None else seed)
    case["workload"] = w
    return case
