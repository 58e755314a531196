"""GPU parity of the packed variable-length backward (fa_bwd_varlen) against the float64 backward
oracle: every gradient element within the elementwise error bound of the dense backward
(tests/grad_bound.py), formed per sequence (each sequence is its own attention problem). The tokens
of a sequence without queries get dK = dV = 0 exactly, those of a sequence without keys dQ = 0; one
packed sequence must reproduce the dense backward bitwise."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.parity_util import f32_scale, to_f64
from tests import grad_bound as gb
from tests.test_varlen_parity import _packed

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import scaled_dot_product_fa2_amd as fa
    return fa


def _check(lens_q, lens_k, Hq, Hkv, D, dtype, causal, seed):
    print(f"[case] varlen bwd q{lens_q} k{lens_k} Hq{Hq} Hkv{Hkv} D{D} {dtype} causal={causal}", flush=True)
    fa = _fa()
    q, k, v, cq, ck = _packed(lens_q, lens_k, Hq, Hkv, D, dtype, seed)
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(q.shape, generator=g).to(dtype)
    qd, kd, vd, dod, cqd, ckd = (t.to(DEV) for t in (q, k, v, do, cq, ck))
    mq, mk = max(max(lens_q), 1), max(max(lens_k), 1)
    o, lse = fa.fa_fwd_varlen(qd, kd, vd, cqd, ckd, mq, mk, causal=causal)
    # NaN-filled outputs: every token belongs to a sequence, so every element must be written
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (qd, kd, vd))
    fa.fa_bwd_varlen(qd, kd, vd, o, lse, dod, cqd, ckd, mq, mk, causal=causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_varlen_bwd_ref(to_f64(q), to_f64(k), to_f64(v), to_f64(do), cq.numpy(),
                                                 ck.numpy(), causal=causal, scale=f32_scale(1.0 / np.sqrt(D)))
    gq, gk, gv = to_f64(dq), to_f64(dk), to_f64(dv)
    for name, t in (("dq", gq), ("dk", gk), ("dv", gv)):
        assert np.all(np.isfinite(t)), f"non-finite {name}"
    cqn, ckn = cq.numpy(), ck.numpy()
    bq, bk, bv = gb.varlen_bwd_bound(q, k, v, do, o, lse, cqn, ckn, rk, rv, causal=causal,
                                     scale=f32_scale(1.0 / np.sqrt(D)), dtype=dtype)
    worst = 0.0
    for b in range(len(lens_q)):
        q0, q1, k0, k1 = int(cqn[b]), int(cqn[b + 1]), int(ckn[b]), int(ckn[b + 1])
        if q1 == q0 or k1 == k0:
            # no attention in this sequence: its gradients are exactly zero
            assert np.all(gq[q0:q1] == 0) and np.all(gk[k0:k1] == 0) and np.all(gv[k0:k1] == 0), f"sequence {b}"
            continue
        for name, got, ref, bnd in (("dq", gq[q0:q1], rq[q0:q1], bq[q0:q1]), ("dk", gk[k0:k1], rk[k0:k1], bk[k0:k1]),
                                    ("dv", gv[k0:k1], rv[k0:k1], bv[k0:k1])):
            r = gb.bound_ratio(got, ref, bnd)
            assert r <= 1.0, f"sequence {b} ({q1 - q0} x {k1 - k0}) {name}: error / bound {r:.3f}"
            worst = max(worst, r)
    print(f"[result] varlen bwd: worst gradient error / bound {worst:.4f}", flush=True)
    return worst


CASES = [
    ([128, 1, 300, 77, 0, 64], [128, 1, 300, 77, 5, 64]),
    ([33, 200, 129], [500, 17, 129]),
    ([5, 0, 70], [0, 9, 200]),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_varlen_bwd_mixed_lengths(case, causal):
    lens_q, lens_k = CASES[case]
    _check(lens_q, lens_k, 4, 2, 128, torch.bfloat16, causal, 2000 + case)


@pytest.mark.parametrize("D", [16, 32, 64, 256])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_varlen_bwd_head_dims(D, dtype):
    _check([90, 257, 3], [90, 257, 40], 2, 1, D, dtype, True, 2100 + D)


def test_varlen_bwd_one_sequence_matches_dense():
    """A single packed sequence reproduces fa_bwd on the same data bitwise, both masks."""
    print("[case] varlen bwd one sequence vs dense", flush=True)
    fa = _fa()
    q, k, v, cq, ck = _packed([777], [777], 8, 2, 128, torch.bfloat16, 2200)
    g = torch.Generator().manual_seed(2201)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    qd, kd, vd, dod, cqd, ckd = (t.to(DEV) for t in (q, k, v, do, cq, ck))
    for causal in (False, True):
        o, lse = fa.fa_fwd_varlen(qd, kd, vd, cqd, ckd, 777, 777, causal=causal)
        gp = fa.fa_bwd_varlen(qd, kd, vd, o, lse, dod, cqd, ckd, 777, 777, causal=causal)
        bnsd = [t.permute(1, 0, 2)[None] for t in (qd, kd, vd, dod)]
        od, ld = fa.fa_fwd(bnsd[0], bnsd[1], bnsd[2], causal=causal)
        gd = fa.fa_bwd(bnsd[0], bnsd[1], bnsd[2], od, ld, bnsd[3], causal=causal)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), gp, gd):
            assert torch.equal(a, b[0].permute(1, 0, 2)), f"{name} causal={causal}"


def test_varlen_bwd_many_sequences():
    """64 sequences of 1..400 tokens, GQA 4, causal, fp16 D=64."""
    rng = np.random.default_rng(2300)
    lens = [int(x) for x in rng.integers(1, 400, size=64)]
    _check(lens, lens, 8, 2, 64, torch.float16, True, 2301)
