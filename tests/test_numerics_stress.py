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
a cancelling sum; the gradients are held to the same elementwise error bound as everywhere else
(tests/grad_bound.py).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity_util as pu
from tests import grad_bound as gb
from tests.test_bwd_parity import _dout, assert_within_bound

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
    refs = oracle.attention_bwd_ref(q64, k64, v64, do64, causal=causal, scale=sc)
    # With every key sharing a large component dQ = scale sum_j dS_ij k_j is a cancelling sum: one
    # rounding of dS to the dtype would dominate it (the kernel feeds dS to the dQ product as two
    # dtype terms), and so does Delta's use of the stored 16-bit O, which the bound accounts for.
    bounds = gb.attention_bwd_bound(q64, k64, v64, do64, o, lse, refs[1], refs[2], causal=causal, scale=sc,
                                    dtype=dtype)
    assert_within_bound((dq, dk, dv), refs, bounds, f"monotone rising={rising} causal={causal} {dtype}")


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
    sc = pu.f32_scale(1.0 / math.sqrt(128))
    refs = oracle.attention_bwd_ref(pu.to_f64(q), pu.to_f64(k), pu.to_f64(v), pu.to_f64(do), causal=causal, scale=sc)
    bounds = gb.attention_bwd_bound(q, k, v, do, o, lse, refs[1], refs[2], causal=causal, scale=sc,
                                    dtype=torch.bfloat16)
    assert_within_bound((dq, dk, dv), refs, bounds, f"MQA 32:1 causal={causal}")


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
