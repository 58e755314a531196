"""The backward's error bound (tests/grad_bound.py) checked on the CPU: a float64 emulation of the
roundings the kernel performs must stay within it, and plausible mistakes must not.

The emulation rounds exactly where the kernel does -- P to the dtype for dV, dS to the dtype for dK,
dS as a rounded value plus a rounded remainder for dQ, Delta from the 16-bit O, the stored LSE in
fp32, each gradient once at the store -- and is otherwise exact, so it must land inside the bound.
The planted mistakes (a dropped scale, gradients of the wrong key, dS as one rounded term on inputs
where dQ cancels) must land outside it.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests import grad_bound as gb


def _rnd(x: np.ndarray, dtype) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).double().numpy()


def _emulate(q, k, v, do, causal, scale, dtype, two_term=True):
    """Kernel-rounded gradients of one head, and the stored O and LSE its forward would pass in."""
    n = q.shape[0]
    o, lse = oracle.attention_ref(q[None, None], k[None, None], v[None, None], causal=causal, scale=scale)
    o16 = _rnd(o[0, 0], dtype)
    lse16 = lse[0, 0].astype(np.float32).astype(np.float64)
    p = oracle.attention_bwd.softmax_rows(q, k, np.arange(n), causal, scale)
    ds = p * (do @ v.T - np.sum(o16 * do, axis=1)[:, None])
    hi = _rnd(ds, dtype)
    lo = _rnd(ds - hi, dtype) if two_term else 0.0
    dq = _rnd(scale * ((hi + lo) @ k), dtype)
    dk = _rnd(scale * (hi.T @ q), dtype)
    dv = _rnd(_rnd(p, dtype).T @ do, dtype)
    return (dq, dk, dv), o16, lse16


def _inputs(n, d, dtype, seed, q_mult=1.0, shared=0.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(n, d, generator=g) * q_mult
    k = torch.randn(n, d, generator=g)
    if shared:  # every key shares a large component along e0 that grows with its position
        q = 0.1 * q
        q[:, 0] += shared
        k = 0.1 * k
        k[:, 0] += 0.05 * torch.arange(n, dtype=torch.float32)
    v = torch.randn(n, d, generator=g)
    do = torch.randn(n, d, generator=g)
    return tuple(t.to(dtype).double().numpy() for t in (q, k, v, do))


CASES = [(100, 64, True, 1.0), (257, 128, False, 1.0), (150, 32, True, 4.0), (64, 16, False, 1.0),
         (200, 64, True, 8.0)]


@pytest.mark.parametrize("n,d,causal,q_mult", CASES, ids=[f"n{c[0]}d{c[1]}{'c' if c[2] else 'f'}x{c[3]:g}" for c in CASES])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_emulated_kernel_within_bound_and_mistakes_outside(n, d, causal, q_mult, dtype):
    scale = float(np.float32(d ** -0.5))
    q, k, v, do = _inputs(n, d, dtype, seed=n + d, q_mult=q_mult)
    exact = oracle.head_bwd_ref(q, k, v, do, causal=causal, scale=scale)
    got, o16, lse16 = _emulate(q, k, v, do, causal, scale, dtype)
    bq, bk, bv = gb.head_bwd_bound(q, k, v, do, o16, lse16, causal=causal, scale=scale, dtype=dtype)
    bk, bv = gb.finish_kv(bk, bv, exact[1], exact[2], dtype)
    for name, g, e, b in zip(("dq", "dk", "dv"), got, exact, (bq, bk, bv)):
        assert gb.bound_ratio(g, e, b) <= 1.0, f"emulated {name} outside the bound"
    assert gb.bound_ratio(got[1] / scale, exact[1], bk) > 10, "dK without the scale passes"
    assert gb.bound_ratio(np.roll(got[2], 1, axis=0), exact[2], bv) > 10, "dV of the wrong key passes"
    assert gb.bound_ratio(got[0] * 1.01, exact[0], bq) > 1, "a 1 % error in dQ passes"


@pytest.mark.parametrize("dtype,causal", [(torch.bfloat16, False), (torch.bfloat16, True), (torch.float16, False),
                                          (torch.float16, True)], ids=["bf16-full", "bf16-causal", "fp16-full",
                                                                        "fp16-causal"])
def test_single_term_ds_where_dq_cancels(dtype, causal):
    """Keys sharing a large component: the kernel's two-term dS stays inside the bound; a single
    rounded dS is outside it in bf16 and in fp16 under the causal mask. (In fp16 without the mask
    its error is of the size of the bound's Delta term, the stored O's rounding, so the bound cannot
    tell them apart there.)"""
    n, d = 256, 64
    scale = float(np.float32(d ** -0.5))
    q, k, v, do = _inputs(n, d, dtype, seed=7 + causal, shared=20.0)
    exact = oracle.head_bwd_ref(q, k, v, do, causal=causal, scale=scale)
    got, o16, lse16 = _emulate(q, k, v, do, causal, scale, dtype)
    bq, _, _ = gb.head_bwd_bound(q, k, v, do, o16, lse16, causal=causal, scale=scale, dtype=dtype, dq_only=True)
    assert gb.bound_ratio(got[0], exact[0], bq) <= 1.0
    single, _, _ = _emulate(q, k, v, do, causal, scale, dtype, two_term=False)
    if dtype == torch.bfloat16 or causal:
        assert gb.bound_ratio(single[0], exact[0], bq) > 1.0, "a single-term dS passes the dQ bound"


def test_floor_near_zero_covers_a_flushed_probability():
    """bf16: a key whose probabilities lie far below fp32's normal range (score 96 below the row
    maximum, P about 2e-42) has exact dK and dV of about 1e-43; hardware that flushes such an fp32
    probability to zero stores 0. The bound's absolute floors near zero (eta and f) must cover that
    and be what covers it: without them the same result is outside the bound."""
    dtype = torch.bfloat16
    n, d, scale = 8, 16, 0.25
    q = np.zeros((n, d))
    q[:, 0] = 1.0
    k = np.zeros((n, d))
    k[1, 0] = -384.0  # scores 96 below the others
    rng = np.random.default_rng(3)
    v = _rnd(rng.standard_normal((n, d)), dtype)
    do = _rnd(rng.standard_normal((n, d)), dtype)
    exact = oracle.head_bwd_ref(q, k, v, do, causal=False, scale=scale)
    assert 0 < np.max(np.abs(exact[1][1])) < 1e-40 and 0 < np.max(np.abs(exact[2][1])) < 1e-40
    o, lse = oracle.attention_ref(q[None, None], k[None, None], v[None, None], causal=False, scale=scale)
    o16 = _rnd(o[0, 0], dtype)
    lse16 = lse[0, 0].astype(np.float32).astype(np.float64)
    p = oracle.attention_bwd.softmax_rows(q, k, np.arange(n), False, scale)
    p_kernel = np.where(p < 2.0 ** -126, 0.0, p)  # flushed to zero
    ds = p_kernel * (do @ v.T - np.sum(o16 * do, axis=1)[:, None])
    got_dk = _rnd(scale * (_rnd(ds, dtype).T @ q), dtype)
    got_dv = _rnd(_rnd(p_kernel, dtype).T @ do, dtype)
    assert not got_dk[1].any() and not got_dv[1].any()
    _, bk, bv = gb.head_bwd_bound(q, k, v, do, o16, lse16, causal=False, scale=scale, dtype=dtype)
    bk, bv = gb.finish_kv(bk, bv, exact[1], exact[2], dtype)
    assert gb.bound_ratio(got_dk, exact[1], bk) <= 1.0 and gb.bound_ratio(got_dv, exact[2], bv) <= 1.0
    saved = gb.SUBNORMAL_HALF[dtype], gb.FP32_FLUSH
    try:
        gb.SUBNORMAL_HALF[dtype], gb.FP32_FLUSH = 0.0, 0.0
        _, bk0, bv0 = gb.head_bwd_bound(q, k, v, do, o16, lse16, causal=False, scale=scale, dtype=dtype)
        bk0, bv0 = gb.finish_kv(bk0, bv0, exact[1], exact[2], dtype)
    finally:
        gb.SUBNORMAL_HALF[dtype], gb.FP32_FLUSH = saved
    assert gb.bound_ratio(got_dk, exact[1], bk0) > 1.0 and gb.bound_ratio(got_dv, exact[2], bv0) > 1.0
