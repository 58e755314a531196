"""Seeded synthetic inputs for the attention forward.

This module only draws random tensors and lays them out in memory. It holds
none of the attention arithmetic, so both the float64 oracle's tests and the
HIP path's tests and benchmark may use it without sharing any computation.

Recipe (same for every workload): a CPU ``torch.Generator`` seeded with the
workload's seed draws Q, then K, then V as float32 standard normals in BNSD
order; each is multiplied by its stated factor (a power of two, so exact) and
cast to the 16-bit dtype with round-to-nearest-even. Where a workload asks for
BSND storage, the tensor is drawn in BNSD order, copied into a BSND-contiguous
buffer and handed over as a BNSD view of it, so the values do not depend on the
storage order.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_random"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    D: int
    dtype: torch.dtype
    causal_modes: Tuple[bool, ...]
    seed: int
    q_mult: float = 1.0
    kv_layout: str = "bnsd"  # "bnsd" contiguous or "bsnd" storage viewed as BNSD
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def dtype_name(self) -> str:
        return {torch.float16: "fp16", torch.bfloat16: "bf16"}[self.dtype]


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 1, 2, 2, 128, 128, 64, torch.float16, (False, True), 1001,
                 description="tiny fp16 D=64 N=128, both masks"),
        Workload("b4h16n1024d128", 4, 16, 16, 1024, 1024, 128, torch.bfloat16, (False, True), 1002,
                 description="bf16 D=128 B=4 H=16 N=1024, both masks"),
        Workload("z128h8n1024d64_strided", 128, 8, 8, 1024, 1024, 64, torch.float16, (False,), 1003,
                 kv_layout="bsnd",
                 description="fp16 D=64 B=128 H=8 N=1024 non-causal, K/V stored BSND viewed as BNSD"),
        Workload("b2h16n4096d256_peaked", 2, 16, 16, 4096, 4096, 256, torch.bfloat16, (True,), 1004,
                 q_mult=4.0,
                 description="bf16 D=256 B=2 H=16 N=4096 causal, Q scaled by 4 so rows are peaked"),
        Workload("gqa_b1h32kv8n16384d128", 1, 32, 8, 16384, 16384, 128, torch.bfloat16, (True,), 1005,
                 description="bf16 D=128 GQA 32/8 N=16384 causal (long context)"),
    ]
}


def _draw(gen: torch.Generator, shape, mult: float, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if mult != 1.0:
        x = x * mult
    return x.to(dtype)


def _as_bsnd_view(x: torch.Tensor) -> torch.Tensor:
    """Same values as ``x`` (B, H, N, D), stored as a contiguous (B, N, H, D) buffer."""
    return x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


def make_random(B: int, Hq: int, Hkv: int, Nq: int, Nkv: int, D: int, dtype: torch.dtype,
                seed: int, q_mult: float = 1.0, kv_layout: str = "bnsd",
                q_layout: str = "bnsd") -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Draw (q, k, v) on the CPU per the recipe in the module docstring."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    q = _draw(gen, (B, Hq, Nq, D), q_mult, dtype)
    k = _draw(gen, (B, Hkv, Nkv, D), 1.0, dtype)
    v = _draw(gen, (B, Hkv, Nkv, D), 1.0, dtype)
    if kv_layout == "bsnd":
        k, v = _as_bsnd_view(k), _as_bsnd_view(v)
    elif kv_layout != "bnsd":
        raise ValueError(f"unknown kv_layout {kv_layout!r}")
    if q_layout == "bsnd":
        q = _as_bsnd_view(q)
    elif q_layout != "bnsd":
        raise ValueError(f"unknown q_layout {q_layout!r}")
    return q, k, v


def make_inputs(w: Workload) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    return make_random(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, w.dtype, w.seed, w.q_mult, w.kv_layout)
