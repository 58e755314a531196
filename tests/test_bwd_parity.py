"""GPU parity of the HIP backward (fa_bwd) against the float64 backward oracle.

Every case runs the HIP forward for O and LSE, then the HIP backward, and compares dQ, dK, dV
element by element with the oracle's gradients of the same 16-bit inputs (the oracle uses the
exact forward, not the kernel's O).

Tolerance: the elementwise first-order error bound of tests/grad_bound.py, derived from the
roundings the kernel performs (P and dS rounded to the dtype before their products, dS as two
terms in dQ, Delta from the stored O, the forward's LSE, fp32 arithmetic, the final store); it
carries no empirical constant. Each case prints its worst error / bound ratio per gradient.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import grad_bound as gb
from tests.parity_util import f32_scale, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import scaled_dot_product_fa2_amd as fa
    return fa


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _dout(B, Hq, Nq, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(B, Hq, Nq, D, generator=g).to(dtype)


def assert_within_bound(grads, refs, bounds, what=""):
    """Every element of (dq, dk, dv) within its error bound; returns and prints the worst ratios."""
    worst = {}
    for name, got, ref, bound in zip(("dq", "dk", "dv"), grads, refs, bounds):
        g = to_f64(got)
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        worst[name] = round(gb.bound_ratio(g, ref, bound), 4)
    print(f"[result] {what}: gradient error / bound {worst}", flush=True)
    assert max(worst.values()) <= 1.0, f"{what}: gradient error ratios {worst}"
    return worst


def _check(q, k, v, do, causal, scale=None, what="", layout=None):
    fa = _fa()
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    if layout is not None:
        qd, kd, vd, dod = layout(qd, kd, vd, dod)
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    s = f32_scale(scale if scale is not None else 1.0 / np.sqrt(q.shape[-1]))
    refs = oracle.attention_bwd_ref(to_f64(q), to_f64(k), to_f64(v), to_f64(do), causal=causal, scale=s)
    bounds = gb.attention_bwd_bound(q, k, v, do, o, lse, refs[1], refs[2], causal=causal, scale=s, dtype=q.dtype)
    return assert_within_bound((dq, dk, dv), refs, bounds, what)


SWEEP = [(D, dt, c) for D in (16, 32, 64, 128, 256) for dt in (torch.bfloat16, torch.float16) for c in (False, True)]


@pytest.mark.parametrize("D,dtype,causal", SWEEP,
                         ids=[f"d{D}-{'bf16' if dt == torch.bfloat16 else 'fp16'}-{'causal' if c else 'full'}"
                              for D, dt, c in SWEEP])
def test_bwd_sweep_ragged(D, dtype, causal):
    """Several query/key tiles with a ragged tail (150 rows), GQA group of 2."""
    _announce(f"bwd sweep D={D} {dtype} causal={causal}")
    q, k, v = workloads.make_random(1, 4, 2, 150, 150, D, dtype, seed=300 + D)
    _check(q, k, v, _dout(1, 4, 150, D, dtype, 301 + D), causal, what=f"D{D}")


CROSS = [(100, 230), (230, 100), (1, 77), (77, 1), (129, 129)]


@pytest.mark.parametrize("Nq,Nkv", CROSS, ids=[f"{a}x{b}" for a, b in CROSS])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_bwd_unequal_lengths(Nq, Nkv, causal, D):
    # D = 128 runs the dK/dV form with K and V in LDS; causal 100 x 230 leaves it a key block that
    # no query row sees (no tile copied or streamed, zero gradients written after the exchange)
    _announce(f"bwd lengths {Nq}x{Nkv} causal={causal} D={D}")
    q, k, v = workloads.make_random(2, 4, 1, Nq, Nkv, D, torch.bfloat16, seed=Nq * 7 + Nkv)
    _check(q, k, v, _dout(2, 4, Nq, D, torch.bfloat16, Nq + Nkv), causal, what=f"{Nq}x{Nkv} D{D}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 1), (6, 3)], ids=["mha", "mqa", "gqa2"])
def test_bwd_head_groups(Hq, Hkv):
    _announce(f"bwd heads {Hq}/{Hkv}")
    q, k, v = workloads.make_random(1, Hq, Hkv, 200, 200, 128, torch.bfloat16, seed=Hq * 10 + Hkv)
    _check(q, k, v, _dout(1, Hq, 200, 128, torch.bfloat16, 5), True, what=f"{Hq}/{Hkv}")


def test_bwd_custom_scale():
    _announce("bwd custom scale")
    q, k, v = workloads.make_random(1, 2, 2, 190, 190, 64, torch.float16, seed=41)
    _check(q, k, v, _dout(1, 2, 190, 64, torch.float16, 42), False, scale=0.3, what="scale 0.3")


def test_bwd_strided_layouts():
    """Q, K, V, O and dO stored (B, N, H, D) and viewed as BNSD; gradients into BSND views too."""
    _announce("bwd strided layouts")
    fa = _fa()
    B, H, N, D = 2, 4, 160, 64
    q, k, v = workloads.make_random(B, H, H, N, N, D, torch.bfloat16, seed=51)
    do = _dout(B, H, N, D, torch.bfloat16, 52)

    def bsnd(t):
        return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)

    qd, kd, vd, dod = (bsnd(t.to(DEV)) for t in (q, k, v, do))
    o = bsnd(torch.empty(B, H, N, D, dtype=torch.bfloat16, device=DEV))
    lse = torch.empty(B, H, N, dtype=torch.float32, device=DEV)
    fa.fa_fwd(qd, kd, vd, causal=True, out=o, lse=lse)
    dq, dk, dv = (bsnd(torch.empty(B, H, N, D, dtype=torch.bfloat16, device=DEV)) for _ in range(3))
    fa.fa_bwd(qd, kd, vd, o, lse, dod, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    sc = f32_scale(1.0 / np.sqrt(D))
    refs = oracle.attention_bwd_ref(to_f64(q), to_f64(k), to_f64(v), to_f64(do), causal=True, scale=sc)
    bounds = gb.attention_bwd_bound(q, k, v, do, o, lse, refs[1], refs[2], causal=True, scale=sc, dtype=q.dtype)
    assert_within_bound((dq, dk, dv), refs, bounds, "strided layouts")


def test_bwd_deterministic_and_fully_written():
    """Outputs pre-filled with NaN are fully overwritten, and repeated calls are bitwise equal."""
    _announce("bwd determinism")
    fa = _fa()
    q, k, v = (t.to(DEV) for t in workloads.make_random(2, 4, 2, 333, 333, 128, torch.bfloat16, seed=61))
    do = _dout(2, 4, 333, 128, torch.bfloat16, 62).to(DEV)
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    outs = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    fa.fa_bwd(q, k, v, o, lse, do, causal=True, dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.synchronize()
    assert all(torch.isfinite(t).all() for t in outs)
    for _ in range(2):
        again = fa.fa_bwd(q, k, v, o, lse, do, causal=True)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(outs, again))


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_workload_b4h16n1024d128_heads(causal):
    """The benchmark shape at full size; three (batch, head) pairs compared in full with the oracle
    (every gradient of those heads), the rest by the sum identities below."""
    _announce(f"bwd b4h16n1024d128 causal={causal}")
    fa = _fa()
    w = workloads.WORKLOADS["b4h16n1024d128"]
    q, k, v = workloads.make_inputs(w)
    do = _dout(w.B, w.Hq, w.Nq, w.D, w.dtype, 71)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, lse, dod, causal=causal)
    torch.cuda.synchronize()
    sc = f32_scale(w.scale)
    for b, h in ((0, 0), (1, 7), (3, 15)):
        # one query head per key/value head here, so the head's terms are the whole dK and dV
        refs = oracle.head_bwd_ref(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), to_f64(do[b, h]),
                                   causal=causal, scale=sc)
        bq, bk, bv = gb.head_bwd_bound(q[b, h], k[b, h], v[b, h], do[b, h], o[b, h], lse[b, h], causal=causal,
                                       scale=sc, dtype=w.dtype)
        bk, bv = gb.finish_kv(bk, bv, refs[1], refs[2], w.dtype)
        assert_within_bound((dq[b, h], dk[b, h], dv[b, h]), refs, (bq, bk, bv), f"b4h16n1024d128 (b={b}, h={h})")
    _sum_identities(dk, dv, do, w.Hq // w.Hkv, w.dtype)


def _sum_identities(dk, dv, do, G, dtype):
    """Every row of dS sums to zero, so sum_j dK_j = 0; the softmax weights sum to one, so
    sum_j dV_j equals the sum of the group's dO rows. A sanity check over every head of a workload
    too large to bound element by element: compared against the magnitude of the summed gradients
    with a margin of a few dtype ulps (the elementwise bound is applied to the sampled heads)."""
    dk64, dv64, do64 = (t.to(dk.device, torch.float64) for t in (dk, dv, do))
    B, Hkv = dk.shape[0], dk.shape[1]
    tol = 3e-2 if dtype == torch.bfloat16 else 6e-3
    ksum = dk64.sum(dim=2)
    kscale = dk64.abs().sum(dim=2)
    assert torch.all(ksum.abs() <= tol * kscale + 1e-6), f"sum_j dK_j: {(ksum.abs() / kscale).max().item():.3e}"
    want = do64.reshape(B, Hkv, G, *do64.shape[2:]).sum(dim=(2, 3))
    got = dv64.sum(dim=2)
    scale = do64.abs().reshape(B, Hkv, G, *do64.shape[2:]).sum(dim=(2, 3))
    assert torch.all((got - want).abs() <= tol * scale + 1e-6), \
        f"sum_j dV_j: {((got - want).abs() / scale).max().item():.3e}"


def test_bwd_workload_gqa16k_sampled():
    """The 16k-token GQA workload: dQ on sampled rows against the oracle (each row needs only its
    own scores), dK and dV through the sum identities."""
    _announce("bwd gqa_b1h32kv8n16384d128 sampled")
    fa = _fa()
    w = workloads.WORKLOADS["gqa_b1h32kv8n16384d128"]
    q, k, v = workloads.make_inputs(w)
    do = _dout(w.B, w.Hq, w.Nq, w.D, w.dtype, 81)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=True)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, lse, dod, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(82)
    q64, k64, v64, do64 = (to_f64(t) for t in (q, k, v, do))
    sc = f32_scale(w.scale)
    o64, lse64 = to_f64(o), to_f64(lse)
    G = w.Hq // w.Hkv
    for h in (0, 13, 31):
        rows = sorted({0, 1, 63, 64, 127, 128, w.Nq - 1, *map(int, rng.integers(0, w.Nq, 5))})
        ref = oracle.dq_rows(q64, k64, v64, do64, 0, h, rows, causal=True, scale=sc)
        bq, _, _ = gb.head_bwd_bound(q64[0, h], k64[0, h // G], v64[0, h // G], do64[0, h], o64[0, h], lse64[0, h],
                                     causal=True, scale=sc, dtype=w.dtype, rows=rows, dq_only=True)
        ratio = gb.bound_ratio(to_f64(dq[0, h])[rows], ref, bq)
        print(f"[result] gqa16k h={h}: sampled dq rows, error / bound {ratio:.4f}", flush=True)
        assert ratio <= 1.0, f"h={h}: dq ratio {ratio:.3f}"
    _sum_identities(dk, dv, do.to(DEV), w.Hq // w.Hkv, w.dtype)
