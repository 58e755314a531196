"""GPU parity under score patterns that stress the online softmax, forward and backward, against
the float64 oracles with the same tolerances as the other parity tests.

* Rising scores: every key tile's scores exceed the previous tile's by more than the kernel's
  rescale headroom, so the running maximum grows (and the accumulator is rescaled) on every tile.
* Falling scores: the first tile holds every row's maximum and later tiles contribute almost
  nothing, the case where a stale maximum must not lose precision.
* Very peaked rows: Q scaled by 30, so each row's weight sits on a handful of keys.
* A single key/value head shared by 32 query heads (MQA) at D = 128.
* One spiking key: every score near 0 except key 96's, which sits J (log2 units) above the first
  tile's maximum. The forward's fast softmax path keeps a tile's probabilities without taking its
  maximum while a lane's sum of them stays at most 2^14. J = 12.5 keeps every row below that
  bound (a probability of about 2^12.5 kept, inside fp16's range), J = 15.5 puts every row above
  it (the tile is scored again and the maximum raised), and at J = 13.8 the first tile's noise
  puts some rows on each side.
The structured inputs are built in float32 and rounded to the 16-bit dtype once; the oracle sees
the same rounded tensors. In the monotone cases every key shares a large component, which makes dQ
a cancelling sum; all three gradients are held to the usual tolerance there, against the exact
gradient for the forward's stored 16-bit O (which Delta is formed from).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity_util as pu
from tests.test_bwd_parity import _dout, _grad_ratio

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import scaled_dot_product_fa2_amd as fa
    return fa


def _monotone(N, D, dtype, rising: bool, seed: int):
    """Q rows all a * e0 plus noise; key j has a component beta * j (rising) or beta * (N - j)
    (falling) along e0 plus noise, so the scores move by a * beta * scale per key."""
    g = torch.Generator().manual_seed(seed)
    a, beta = 20.0, 0.05
    q = 0.1 * torch.randn(1, 2, N, D, generator=g)
    q[..., 0] += a
    k = 0.1 * torch.randn(1, 2, N, D, generator=g)
    pos = torch.arange(N, dtype=torch.float32)
    k[..., 0] += beta * (pos if rising else (N - pos))
    v = torch.randn(1, 2, N, D, generator=g)
    return q.to(dtype), k.to(dtype), v.to(dtype)


@pytest.mark.parametrize("rising", [True, False], ids=["rising", "falling"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_monotone_scores_forward_and_backward(rising, causal, dtype):
    N, D = 520, 64
    print(f"[case] monotone rising={rising} causal={causal} {dtype}", flush=True)
    fa = _fa()
    q, k, v = _monotone(N, D, dtype, rising, seed=3000 + 2 * rising + causal)
    scale = 1.0 / math.sqrt(D)
    # per 64-key tile the scaled scores rise by a * beta * 64 * scale * log2(e) ~ 11.5 > 8 (log2 units)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal)
    torch.cuda.synchronize()
    pu.full_check(qd, kd, vd, o, lse, causal, scale, f"monotone rising={rising}")
    do = _dout(1, 2, N, D, dtype, 3100)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, lse, do.to(DEV), causal=causal)
    torch.cuda.synchronize()
    sc = pu.f32_scale(scale)
    q64, k64, v64, do64 = (pu.to_f64(t) for t in (q, k, v, do))
    rq, rk, rv = oracle.attention_bwd_ref(q64, k64, v64, do64, causal=causal, scale=sc)
    # The backward's input O is the forward's 16-bit output, and Delta = rowsum(O * dO) is formed
    # from it. With every key sharing a large component, dQ = dS K amplifies that half-ulp
    # difference (sum_j dS_ij = -Delta error, times the common component) beyond the rounding
    # tolerance, so the reference is the exact gradient for the stored O:
    #   dS' = dS - scale * P * (Delta16 - Delta)  =>  dQ' = dQ - scale * d * (P K),  dK' = dK - scale * P^T (d * Q)
    # with d = Delta16 - Delta; P K is the oracle forward with V := K, P^T X the oracle's dV for dO := X.
    o_exact, _ = oracle.attention_ref(q64, k64, v64, causal=causal, scale=sc)
    d = np.sum(pu.to_f64(o) * do64, axis=-1) - np.sum(o_exact * do64, axis=-1)
    pk, _ = oracle.attention_ref(q64, k64, k64, causal=causal, scale=sc)
    _, _, ptdq = oracle.attention_bwd_ref(q64, k64, k64, d[..., None] * q64, causal=causal, scale=sc)
    ref = (rq - sc * d[..., None] * pk, rk - sc * ptdq, rv)
    floor = 1e-3 * float(np.sqrt(np.mean(do64 ** 2)))
    for name, got, r in zip(("dk", "dv"), (dk, dv), ref[1:]):
        g = pu.to_f64(got)
        assert np.all(np.isfinite(g)), f"non-finite {name}"
        ratio = _grad_ratio(g, r, dtype, floor=floor)
        assert ratio <= 1.0, f"{name}: gradient error ratio {ratio:.3f}"
    # dQ = scale * sum_j dS_ij k_j, where with every key sharing a large component the terms cancel to a
    # small result: one rounding of dS to the dtype would dominate it, and the kernel feeds the dQ
    # product dS as two dtype terms (rounded value and rounded remainder) so that it does not.
    ratio = _grad_ratio(pu.to_f64(dq), ref[0], dtype, floor=floor)
    print(f"[result] monotone rising={rising} causal={causal} {dtype}: dq error ratio {ratio:.3f}", flush=True)
    assert ratio <= 1.0, f"dq: gradient error ratio {ratio:.3f}"


@pytest.mark.parametrize("causal", [False, True])
def test_very_peaked_rows(causal):
    print(f"[case] Q x 30 causal={causal}", flush=True)
    fa = _fa()
    q, k, v = workloads.make_random(2, 4, 2, 333, 333, 128, torch.bfloat16, seed=3200 + causal, q_mult=30.0)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal)
    torch.cuda.synchronize()
    pu.full_check(qd, kd, vd, o, lse, causal, 1.0 / math.sqrt(128), "Q x 30")


@pytest.mark.parametrize("causal", [False, True])
def test_mqa_32_heads(causal):
    print(f"[case] MQA Hq=32 Hkv=1 causal={causal}", flush=True)
    fa = _fa()
    q, k, v = workloads.make_random(1, 32, 1, 300, 300, 128, torch.bfloat16, seed=3300 + causal)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal)
    torch.cuda.synchronize()
    pu.full_check(qd, kd, vd, o, lse, causal, 1.0 / math.sqrt(128), "MQA 32:1")
    do = _dout(1, 32, 300, 128, torch.bfloat16, 3301)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, lse, do.to(DEV), causal=causal)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd_ref(pu.to_f64(q), pu.to_f64(k), pu.to_f64(v), pu.to_f64(do), causal=causal,
                                   scale=pu.f32_scale(1.0 / math.sqrt(128)))
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        ratio = _grad_ratio(pu.to_f64(got), r, torch.bfloat16)
        assert ratio <= 1.0, f"{name}: gradient error ratio {ratio:.3f}"


@pytest.mark.parametrize("jump", [6.0, 12.5, 13.8, 15.5, 40.0])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_spiking_key_around_fast_path_bound(jump, D, dtype, causal):
    print(f"[case] spike J={jump} D={D} {dtype} causal={causal}", flush=True)
    fa = _fa()
    N, scale = 200, 1.0 / math.sqrt(D)
    g = torch.Generator().manual_seed(3400 + int(jump * 10) + D + causal)
    q = 0.1 * torch.randn(1, 2, N, D, generator=g)
    q[..., 0] += 1.0 / scale  # scale * q . k along e0 is then k's e0 component
    k = 0.1 * torch.randn(1, 2, N, D, generator=g)
    k[:, :, 96, 0] += jump / math.log2(math.e)
    v = torch.randn(1, 2, N, D, generator=g)
    qd, kd, vd = (t.to(dtype).to(DEV) for t in (q, k, v))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal)
    torch.cuda.synchronize()
    pu.full_check(qd, kd, vd, o, lse, causal, scale, f"spike J={jump} D={D}")
