"""Seeded synthetic inputs for single-token GQA decode.

This module only draws random numbers and casts them to the storage dtypes; it holds none of the
attention arithmetic.  The CPU oracle and the HIP library both receive exactly the bytes made here.

Recipe (all five workloads): a CPU ``torch.Generator`` seeded with ``1000 + workload id`` (or the seed
passed in) draws, in this order, the sequence lengths (``randint`` over an inclusive range, when they
are random), then q, K and V as float32 standard normals; the values are then cast with
round-to-nearest-even to the storage dtype.  The fp8-e4m3fn cache is clipped to [-4, 4] first and
stored with per-tensor descale 1.0.  Cache positions at or beyond a sequence's length hold the same
normal draws and are never read by a correct kernel.
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
    5: Workload("long-fp8 B2 Hq64 Hkv8 d128 L32768", 2, 64, 8, 128, 32768, "bf16", "fp8_e4m3",
                seq_lens=(32768, 30000), seed=1005),
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


def make(wid, seed: Optional[int] = None) -> dict:
    """Inputs of one named workload (ids 1, 2, 3, '4-mha', '4-gqa', '4-mqa', 5)."""
    w = WORKLOADS[wid]
    case = make_case(w.B, w.Hq, w.Hkv, w.d, w.L, w.q_dtype, w.kv_dtype, seq_lens=w.seq_lens,
                     seq_range=w.seq_range, seed=w.seed if seed is None else seed)
    case["workload"] = w
    return case
