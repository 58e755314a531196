"""GPU parity of the HIP attention forward against the float64 oracle.

Every case compares every output element with the oracle, the five named
workloads included (the three large ones through the pooled oracle on the host
cores). Every case prints its name before it runs.
"""
import math

import numpy as np
import pytest
import torch

from tests import parity_util as pu
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import scaled_dot_product_fa2_amd as fa
    return fa


def _run(q, k, v, causal, scale=None):
    fa = _fa()
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return q, k, v, o, lse


def _announce(msg):
    print(f"[case] {msg}", flush=True)


SWEEP = []
for D in (16, 32, 64, 128, 256):
    for dtype in (torch.float16, torch.bfloat16):
        for causal in (False, True):
            SWEEP.append((D, dtype, causal))


@pytest.mark.parametrize("D,dtype,causal", SWEEP,
                         ids=[f"d{d}-{str(t).split('.')[-1]}-{'causal' if c else 'full'}" for d, t, c in SWEEP])
def test_sweep_ragged(D, dtype, causal):
    """Several tiles plus a ragged tail in both sequence dims, GQA group 2."""
    B, Hq, Hkv, N = 2, 4, 2, 200
    _announce(f"sweep D={D} {dtype} causal={causal} B={B} Hq={Hq} Hkv={Hkv} N={N}")
    q, k, v = workloads.make_random(B, Hq, Hkv, N, N, D, dtype, seed=100 + D)
    q, k, v, o, lse = _run(q, k, v, causal)
    pu.full_check(q, k, v, o, lse, causal, 1.0 / math.sqrt(D), f"sweep D={D}")


GQA = [(8, 1), (8, 2), (8, 4), (8, 8), (6, 3)]


@pytest.mark.parametrize("Hq,Hkv", GQA, ids=[f"hq{a}-hkv{b}" for a, b in GQA])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_groups(Hq, Hkv, causal):
    _announce(f"gqa Hq={Hq} Hkv={Hkv} causal={causal}")
    q, k, v = workloads.make_random(1, Hq, Hkv, 256, 256, 64, torch.bfloat16, seed=7 + Hq * 10 + Hkv)
    q, k, v, o, lse = _run(q, k, v, causal)
    pu.full_check(q, k, v, o, lse, causal, 1 / 8, f"gqa {Hq}/{Hkv}")


CROSS = [(1, 1), (1, 300), (77, 1), (64, 640), (640, 64), (129, 257), (257, 129), (1000, 333)]


@pytest.mark.parametrize("Nq,Nkv", CROSS, ids=[f"{a}x{b}" for a, b in CROSS])
@pytest.mark.parametrize("causal", [False, True])
def test_unequal_lengths(Nq, Nkv, causal):
    """Nq != Nkv and sizes that are not tile multiples; the causal mask is top-left (key j <= row i)."""
    _announce(f"lengths Nq={Nq} Nkv={Nkv} causal={causal}")
    q, k, v = workloads.make_random(1, 2, 1, Nq, Nkv, 128, torch.float16, seed=Nq * 7 + Nkv)
    q, k, v, o, lse = _run(q, k, v, causal)
    pu.full_check(q, k, v, o, lse, causal, 1 / math.sqrt(128), f"lengths {Nq}x{Nkv}")


def test_custom_scale_and_peaked_rows():
    _announce("custom scale 0.5, Q x 8")
    q, k, v = workloads.make_random(1, 2, 2, 300, 300, 64, torch.bfloat16, seed=99, q_mult=8.0)
    for causal in (False, True):
        qd, kd, vd, o, lse = _run(q, k, v, causal, scale=0.5)
        pu.full_check(qd, kd, vd, o, lse, causal, 0.5, "peaked")


@pytest.mark.parametrize("layout", ["bsnd_q", "bsnd_kv", "bsnd_all"])
def test_strided_layouts(layout):
    """BSND storage viewed as BNSD, for Q, for K/V, and for all of Q/K/V/O."""
    _announce(f"strided {layout}")
    q, k, v = workloads.make_random(2, 4, 4, 192, 192, 64, torch.float16, seed=31,
                                    kv_layout="bsnd" if layout != "bsnd_q" else "bnsd",
                                    q_layout="bsnd" if layout != "bsnd_kv" else "bnsd")
    fa = _fa()
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    assert not (qd.is_contiguous() and kd.is_contiguous())
    out = None
    if layout == "bsnd_all":
        out = torch.empty(2, 192, 4, 64, dtype=q.dtype, device=DEV).permute(0, 2, 1, 3)
    for causal in (False, True):
        o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, out=out)
        torch.cuda.synchronize()
        pu.full_check(qd, kd, vd, o, lse, causal, 1 / 8, f"strided {layout}")
        o2, lse2 = fa.fa_fwd(qd.contiguous(), kd.contiguous(), vd.contiguous(), causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o.contiguous(), o2) and torch.equal(lse, lse2), "stride changes the result"


# ---------------------------------------------------------------------------------------------
# The five named workloads, at their full sizes.

def _workload_case(name, causal):
    w = workloads.WORKLOADS[name]
    _announce(f"workload {name} causal={causal}")
    q, k, v = workloads.make_inputs(w)
    q, k, v, o, lse = _run(q, k, v, causal)
    return w, q, k, v, o, lse


def test_workload_tiny_full():
    for causal in (False, True):
        w, q, k, v, o, lse = _workload_case("tiny", causal)
        r, e = pu.full_check(q, k, v, o, lse, causal, w.scale, f"tiny causal={causal}")
        print(f"[result] tiny causal={causal}: every element, worst O error ratio {r:.3f}, worst LSE error {e:.2e}",
              flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_workload_b4h16n1024d128_full(causal):
    w, q, k, v, o, lse = _workload_case("b4h16n1024d128", causal)
    r, e = pu.full_check(q, k, v, o, lse, causal, w.scale, f"b4h16n1024d128 causal={causal}")
    print(f"[result] b4h16n1024d128 causal={causal}: every element, worst O error ratio {r:.3f}, "
          f"worst LSE error {e:.2e}", flush=True)


def _heads(w, rng, n):
    hs = {(0, 0), (w.B - 1, w.Hq - 1)}
    while len(hs) < n:
        hs.add((int(rng.integers(0, w.B)), int(rng.integers(0, w.Hq))))
    return sorted(hs)


@pytest.mark.parametrize("name", ["z128h8n1024d64_strided", "b2h16n4096d256_peaked", "gqa_b1h32kv8n16384d128"])
def test_workload_full(name):
    """Every O and LSE element of the three large workloads against the float64 oracle, which runs one
    (batch, head) per task on the host cores. Sampled rows (first, last, tile edges, random) of six heads
    are compared first as a quick pre-check."""
    w = workloads.WORKLOADS[name]
    for causal in w.causal_modes:
        w, q, k, v, o, lse = _workload_case(name, causal)
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        rng = np.random.default_rng(w.seed)
        rows = pu.sample_rows(w.Nq, 128, rng)
        pu.sampled_check(q, k, v, o, lse, causal, w.scale, _heads(w, rng, 6), rows, name)
        r, e = pu.full_check_pool(q, k, v, o, lse, causal, w.scale, name)
        print(f"[result] {name} causal={causal}: every element, worst O error ratio {r:.3f}, "
              f"worst LSE error {e:.2e}", flush=True)


# More items than resident workgroups under the causal mask: each XCD lists its items unit by unit
# (longest first within a unit) and every workgroup runs several of them.
MANY_ITEMS = [(16, 16, 16, 520, 128, torch.bfloat16), (8, 16, 4, 1000, 64, torch.float16)]


@pytest.mark.parametrize("B,Hq,Hkv,N,D,dtype", MANY_ITEMS,
                         ids=[f"b{b}h{hq}kv{hkv}n{n}d{d}" for b, hq, hkv, n, d, _ in MANY_ITEMS])
def test_causal_many_items_per_workgroup(B, Hq, Hkv, N, D, dtype):
    _announce(f"causal, many items per workgroup: B={B} Hq={Hq} Hkv={Hkv} N={N} D={D} {dtype}")
    fa = _fa()
    plan = fa.fa_fwd_plan(B, Hq, Hkv, N, N, D, True, 1 if dtype == torch.bfloat16 else 0)
    assert B * Hq * ((N + plan["block_q"] - 1) // plan["block_q"]) > plan["grid"]
    q, k, v = workloads.make_random(B, Hq, Hkv, N, N, D, dtype, seed=5100 + D)
    q, k, v, o, lse = _run(q, k, v, True)
    pu.full_check(q, k, v, o, lse, True, 1.0 / math.sqrt(D), f"many items b{B} h{Hq}/{Hkv} n{N} d{D}")
