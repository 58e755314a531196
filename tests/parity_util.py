"""Helpers shared by the GPU parity tests: tolerances and comparisons against the float64 oracle."""
from __future__ import annotations

import math
import os
from typing import Dict, Iterable, List, Sequence, Tuple

import numpy as np
import torch

import oracle

# Elementwise tolerances on O (against the float64 oracle, O upcast from its 16-bit storage) and an
# absolute tolerance on LSE.
O_TOL = {torch.bfloat16: (1e-2, 1e-2), torch.float16: (2e-3, 2e-3)}
LSE_ATOL = 1e-3


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def f32_scale(scale: float) -> float:
    """The scale the kernel receives (the ABI passes it as a float32)."""
    return float(np.float32(scale))


def o_ratio(o_gpu: np.ndarray, o_ref: np.ndarray, dtype: torch.dtype) -> float:
    atol, rtol = O_TOL[dtype]
    return float(np.max(np.abs(o_gpu - o_ref) / (atol + rtol * np.abs(o_ref)))) if o_ref.size else 0.0


def lse_err(l_gpu: np.ndarray, l_ref: np.ndarray) -> float:
    return float(np.max(np.abs(l_gpu - l_ref))) if l_ref.size else 0.0


def assert_close(o_gpu, l_gpu, o_ref, l_ref, dtype, what=""):
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    assert np.all(np.isfinite(l_gpu)), f"{what}: non-finite LSE"
    r = o_ratio(o_gpu, o_ref, dtype)
    e = lse_err(l_gpu, l_ref)
    assert r <= 1.0, f"{what}: O error ratio {r:.3f} > 1 (tolerance {O_TOL[dtype]})"
    assert e <= LSE_ATOL, f"{what}: LSE error {e:.2e} > {LSE_ATOL}"
    return r, e


def full_check(q, k, v, o, lse, causal, scale, what=""):
    """Compare every output element with the oracle."""
    o_ref, l_ref = oracle.attention_ref(to_f64(q), to_f64(k), to_f64(v), causal=causal, scale=f32_scale(scale))
    return assert_close(to_f64(o), to_f64(lse), o_ref, l_ref, q.dtype, what)


def sample_rows(n: int, tile: int, rng: np.random.Generator, n_random: int = 6) -> List[int]:
    """First, last, tile-boundary and random rows of a length-n sequence."""
    rows = {0, 1, n - 1, n // 2}
    for t in range(tile, n, tile * max(1, n // (tile * 4))):
        rows.update({t - 1, t})
    rows.update(int(x) for x in rng.integers(0, n, size=n_random))
    return sorted(r for r in rows if 0 <= r < n)


def sampled_check(q, k, v, o, lse, causal, scale, heads: Iterable[Tuple[int, int]], rows: Sequence[int],
                  what=""):
    """Compare the given (b, h) heads on the given rows with the oracle, row by row."""
    o_cpu = o.detach().cpu()
    l_cpu = lse.detach().cpu()
    qc, kc, vc = q.detach().cpu(), k.detach().cpu(), v.detach().cpu()
    worst_r, worst_e = 0.0, 0.0
    rows = list(rows)
    for b, h in heads:
        kvh = h // (q.shape[1] // k.shape[1])
        o_ref, l_ref = oracle.attention_rows(
            qc[b:b + 1, h:h + 1].to(torch.float64).numpy(), kc[b:b + 1, kvh:kvh + 1].to(torch.float64).numpy(),
            vc[b:b + 1, kvh:kvh + 1].to(torch.float64).numpy(), 0, 0, rows, causal=causal,
            scale=f32_scale(scale))
        r, e = assert_close(o_cpu[b, h, rows].to(torch.float64).numpy(), l_cpu[b, h, rows].to(torch.float64).numpy(),
                            o_ref, l_ref, q.dtype, f"{what} b={b} h={h}")
        worst_r, worst_e = max(worst_r, r), max(worst_e, e)
    return worst_r, worst_e


def pool_workers() -> int:
    """Host processes for the pooled oracle: the cores this process may use, at most 15 (the GPU
    process itself is the sixteenth)."""
    return max(1, min(15, len(os.sched_getaffinity(0))))


def full_check_pool(q, k, v, o, lse, causal, scale, what=""):
    """Compare every output element with the oracle, computed one (batch, head) per task in a pool of
    host processes. Returns the worst O error ratio and the worst LSE error over all elements."""
    qn, kn, vn = (t.detach().cpu().float().numpy() for t in (q, k, v))  # exact upcast of 16-bit values
    res, _ = oracle.attention_ref_pool(qn, kn, vn, causal=causal, scale=f32_scale(scale), workers=pool_workers())
    o_cpu, l_cpu = o.detach().cpu(), lse.detach().cpu()
    worst_r, worst_e = 0.0, 0.0
    for (b, h), (o_ref, l_ref) in sorted(res.items()):
        r, e = assert_close(o_cpu[b, h].to(torch.float64).numpy(), l_cpu[b, h].to(torch.float64).numpy(),
                            o_ref, l_ref, q.dtype, f"{what} b={b} h={h}")
        worst_r, worst_e = max(worst_r, r), max(worst_e, e)
    return worst_r, worst_e
