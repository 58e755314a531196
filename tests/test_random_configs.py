"""Seeded random configurations: every axis of the forward and the backward at once.

The other parity tests vary one axis at a time (head dim, dtype, head group, lengths, mask,
storage layout, scale). Here each case draws all of them together from a seeded generator, so
their interactions -- a D = 16 head with a group of three in BSND storage under a sliding window
with Nq != Nkv, say -- are compared element by element with the float64 oracles too: O and LSE
within the forward tolerances, dQ, dK and dV within the derived error bound of tests/grad_bound.py.
Packed variable-length sequences are drawn the same way (sequence count, query and key lengths with
empty sequences among them, head dim, dtype, group, mask) and go through the varlen entry points.
The case list is fixed by the seed; each case prints its draw before it runs.

Wider draws are opt-in: FA_RANDOM_SWEEP=<n> in the environment adds, per family, n forward and
n/2 backward cases with longer sequences (up to 2 000 rows), with batches and head counts that
give the persistent schedule several rounds, and with extreme scores (Q x 8 to x 32, scales up to
1.5), plus n/4 forward and n/8 backward packed batches of up to 24 sequences of up to 4 000 tokens.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import grad_bound as gb
from tests.parity_util import LSE_ATOL, O_TOL, f32_scale, o_ratio, to_f64
from tests.test_bwd_parity import assert_within_bound

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _draw_cases(n: int, seed: int):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 3]))
        mask = str(rng.choice(["full", "causal", "window"]))
        cases.append(dict(
            D=int(rng.choice([16, 32, 64, 128, 256])),
            dtype=[torch.bfloat16, torch.float16][int(rng.integers(2))],
            B=int(rng.integers(1, 3)), Hkv=hkv, Hq=hkv * int(rng.choice([1, 2, 3, 4])),
            Nq=int(rng.integers(1, 330)), Nkv=int(rng.integers(1, 330)),
            mask=mask,
            # window sides: -1 is unbounded; a finite side is anything from 0 to beyond the sequence
            left=int(rng.integers(-1, 200)), right=int(rng.integers(-1, 60)),
            q_layout=str(rng.choice(["bnsd", "bsnd"])), kv_layout=str(rng.choice(["bnsd", "bsnd"])),
            scale=None if rng.random() < 0.5 else float(rng.uniform(0.03, 0.4)),
            q_mult=float(rng.choice([1.0, 1.0, 4.0])),
            seed=seed * 1000 + i))
    return cases


FWD = _draw_cases(32, 17)
BWD = _draw_cases(16, 29)


def _id(c):
    dt = "bf16" if c["dtype"] == torch.bfloat16 else "fp16"
    m = c["mask"] if c["mask"] != "window" else f"w{c['left']}_{c['right']}"
    return f"d{c['D']}-{dt}-b{c['B']}h{c['Hq']}kv{c['Hkv']}-{c['Nq']}x{c['Nkv']}-{m}-{c['q_layout']}{c['kv_layout']}"


def _inputs(c):
    q, k, v = workloads.make_random(c["B"], c["Hq"], c["Hkv"], c["Nq"], c["Nkv"], c["D"], c["dtype"], seed=c["seed"],
                                    q_mult=c["q_mult"], kv_layout=c["kv_layout"], q_layout=c["q_layout"])
    return q, k, v


def _window(c):
    if c["mask"] != "window":
        return None
    return (None if c["left"] < 0 else c["left"], None if c["right"] < 0 else c["right"])


def _forward(fa, c, qd, kd, vd):
    if c["mask"] == "window":
        return fa.fa_fwd_window(qd, kd, vd, window_left=c["left"], window_right=c["right"], scale=c["scale"])
    return fa.fa_fwd(qd, kd, vd, causal=c["mask"] == "causal", scale=c["scale"])


@pytest.mark.parametrize("c", FWD, ids=[_id(c) for c in FWD])
def test_random_forward(c):
    import scaled_dot_product_fa2_amd as fa
    print(f"[case] forward {_id(c)} scale={c['scale']} q_mult={c['q_mult']} seed={c['seed']}", flush=True)
    q, k, v = _inputs(c)
    o, lse = _forward(fa, c, q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    s = f32_scale(c["scale"] if c["scale"] is not None else 1.0 / np.sqrt(c["D"]))
    o_ref, l_ref = oracle.attention_ref(to_f64(q), to_f64(k), to_f64(v), causal=c["mask"] == "causal", scale=s,
                                        window=_window(c))
    og, lg = to_f64(o), to_f64(lse)
    assert np.all(np.isfinite(og)), "non-finite O"
    ratio = o_ratio(og, o_ref, c["dtype"])
    empty = np.isneginf(l_ref)  # rows whose window holds no key: O = 0, LSE = -inf
    assert np.array_equal(np.isneginf(lg), empty), "LSE = -inf exactly on the rows without keys"
    lerr = float(np.max(np.abs(lg[~empty] - l_ref[~empty]))) if (~empty).any() else 0.0
    print(f"[result] forward {_id(c)}: O error ratio {ratio:.3f}, LSE error {lerr:.2e}", flush=True)
    assert ratio <= 1.0, f"O error ratio {ratio:.3f} > 1 ({O_TOL[c['dtype']]})"
    assert lerr <= LSE_ATOL, f"LSE error {lerr:.2e}"


@pytest.mark.parametrize("c", BWD, ids=[_id(c) for c in BWD])
def test_random_backward(c):
    import scaled_dot_product_fa2_amd as fa
    print(f"[case] backward {_id(c)} scale={c['scale']} q_mult={c['q_mult']} seed={c['seed']}", flush=True)
    q, k, v = _inputs(c)
    g = torch.Generator().manual_seed(c["seed"] + 1)
    do = torch.randn(c["B"], c["Hq"], c["Nq"], c["D"], generator=g).to(c["dtype"])
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = _forward(fa, c, qd, kd, vd)
    win = None if c["mask"] != "window" else (c["left"], c["right"])
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, lse, dod, causal=c["mask"] == "causal", scale=c["scale"], window=win)
    torch.cuda.synchronize()
    s = f32_scale(c["scale"] if c["scale"] is not None else 1.0 / np.sqrt(c["D"]))
    causal = c["mask"] == "causal"
    refs = oracle.attention_bwd_ref(to_f64(q), to_f64(k), to_f64(v), to_f64(do), causal=causal, scale=s,
                                    window=_window(c))
    bounds = gb.attention_bwd_bound(q, k, v, do, o, lse, refs[1], refs[2], causal=causal, scale=s, dtype=c["dtype"],
                                    window=_window(c))
    assert_within_bound((dq, dk, dv), refs, bounds, f"backward {_id(c)}")


# Drawn cases kept because they once failed:
#  * an fp16 window case whose dQ missed its bound by 5 % where the two dtype terms of one large dS
#    were converted from different roundings of it (one dS next to an fp16 rounding midpoint;
#    tests/test_isa.py checks the generated code for the cause);
#  * a bf16 causal case with Nkv > Nq and peaked rows, where the exact dK and dV of the last row's
#    diagonal key are about 1e-42 and the kernel stores 0 (below bf16's smallest subnormal), and a
#    bf16 D = 256 window case with five query rows whose exact dK of one key is 2.7e-37 and comes
#    out 0 (its probabilities lie below fp32's smallest normal): the bound had no absolute floor
#    near zero for bf16 and none for a flushed probability (tests/grad_bound.py, eta and f).
REGRESSION = [dict(D=32, dtype=torch.float16, B=1, Hkv=2, Hq=8, Nq=105, Nkv=181, mask="window", left=84, right=47,
                   q_layout="bsnd", kv_layout="bsnd", scale=0.27857336768124596, q_mult=4.0, seed=7002062),
              dict(D=128, dtype=torch.bfloat16, B=2, Hkv=2, Hq=2, Nq=572, Nkv=1168, mask="causal", left=61, right=179,
                   q_layout="bsnd", kv_layout="bsnd", scale=0.3699197098836212, q_mult=4.0, seed=8002222),
              dict(D=256, dtype=torch.bfloat16, B=1, Hkv=1, Hq=1, Nq=5, Nkv=105, mask="window", left=196, right=55,
                   q_layout="bnsd", kv_layout="bsnd", scale=0.3631942927492421, q_mult=4.0, seed=9002454)]


@pytest.mark.parametrize("c", REGRESSION, ids=[_id(c) for c in REGRESSION])
def test_backward_regression(c):
    test_random_backward(c)


# Opt-in wider draws (FA_RANDOM_SWEEP=<n>): families "long", "rounds" and "scores", each seeded on its own.
N_WIDE = int(os.environ.get("FA_RANDOM_SWEEP", "0"))


def _draw_wide(n: int, seed: int, family: str, backward: bool):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(rng.choice([16, 32, 64, 128, 256]))
        dtype = [torch.bfloat16, torch.float16][int(rng.integers(2))]
        mask = str(rng.choice(["full", "causal", "window"]))
        if family == "rounds":  # enough items for several rounds of the persistent grid
            hkv = int(rng.choice([1, 2, 4, 8]))
            B, Hq, hi = int(rng.integers(1, 9)), hkv * int(rng.choice([1, 2, 4])), 1100
            if backward:  # keep the host-side bound affordable
                B, g = min(B, 2), Hq // hkv
                hkv = min(hkv, 2)
                Hq = hkv * g
        else:
            hkv = int(rng.choice([1, 2, 3]))
            B, Hq = int(rng.integers(1, 3)), hkv * int(rng.choice([1, 2, 3, 4]))
            hi = (1200 if backward else 2000) if family == "long" and rng.random() < 0.35 else 330
        q_mult = float(rng.choice([8.0, 16.0, 32.0])) if family == "scores" else float(rng.choice([1.0, 1.0, 4.0]))
        if family == "scores":
            scale = float(rng.uniform(0.3, 1.5)) if rng.random() < 0.7 else None
        else:
            scale = None if rng.random() < 0.5 else float(rng.uniform(0.03, 0.4))
        cases.append(dict(D=D, dtype=dtype, B=B, Hkv=hkv, Hq=Hq, Nq=int(rng.integers(1, hi)),
                          Nkv=int(rng.integers(1, hi)), mask=mask, left=int(rng.integers(-1, 600)),
                          right=int(rng.integers(-1, 200)), q_layout=str(rng.choice(["bnsd", "bsnd"])),
                          kv_layout=str(rng.choice(["bnsd", "bsnd"])), scale=scale, q_mult=q_mult,
                          seed=seed * 1000 + i))
    return cases


WIDE_FWD = [c for k, fam in enumerate(("long", "rounds", "scores")) for c in _draw_wide(N_WIDE, 50 + 2 * k, fam, False)]
WIDE_BWD = [c for k, fam in enumerate(("long", "rounds", "scores"))
            for c in _draw_wide(N_WIDE // 2, 51 + 2 * k, fam, True)]


if N_WIDE:  # defined only when asked for, so that the default suite collects no empty parameter sets
    @pytest.mark.parametrize("c", WIDE_FWD, ids=[_id(c) for c in WIDE_FWD])
    def test_wide_forward(c):
        test_random_forward(c)

    @pytest.mark.parametrize("c", WIDE_BWD, ids=[_id(c) for c in WIDE_BWD])
    def test_wide_backward(c):
        test_random_backward(c)


# Packed variable-length sequences: a random number of sequences with random query and key lengths
# (empty ones included), head dim, dtype, head group and mask, through the varlen entry points.
def _draw_varlen(n: int, seed: int):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        nseq = int(rng.integers(1, 7))
        lens_q = [int(x) if rng.random() > 0.12 else 0 for x in rng.integers(1, 300, nseq)]
        lens_k = [int(x) if rng.random() > 0.12 else 0 for x in rng.integers(1, 300, nseq)]
        if sum(lens_q) == 0:
            lens_q[0] = int(rng.integers(1, 100))
        if sum(lens_k) == 0:
            lens_k[-1] = int(rng.integers(1, 100))
        hkv = int(rng.choice([1, 2]))
        cases.append(dict(lens_q=lens_q, lens_k=lens_k, Hkv=hkv, Hq=hkv * int(rng.choice([1, 2, 4])),
                          D=int(rng.choice([16, 32, 64, 128, 256])),
                          dtype=[torch.bfloat16, torch.float16][int(rng.integers(2))],
                          causal=bool(rng.integers(2)), seed=seed * 1000 + i))
    return cases


def _draw_varlen_wide(n: int, seed: int, backward: bool):
    """Up to 24 sequences of up to 4 000 tokens (backward: 8 of up to 1 200), empty ones among them."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        nseq = int(rng.integers(1, 25))
        hi = int(rng.choice([300, 1500, 4000]))
        lens_q = [int(x) if rng.random() > 0.1 else 0 for x in rng.integers(1, hi, nseq)]
        lens_k = [int(x) if rng.random() > 0.1 else 0 for x in rng.integers(1, hi, nseq)]
        if rng.random() < 0.5:
            lens_k = list(lens_q)
        hkv = int(rng.choice([1, 2, 4]))
        Hq = hkv * int(rng.choice([1, 2, 4]))
        if backward:
            lens_q, lens_k = [min(x, 1200) for x in lens_q][:8], [min(x, 1200) for x in lens_k][:8]
            Hq, hkv = min(Hq, 4), min(hkv, 2)
            Hq -= Hq % hkv
        if sum(lens_q) == 0:
            lens_q[0] = 5
        if sum(lens_k) == 0:
            lens_k[-1] = 7
        cases.append(dict(lens_q=lens_q, lens_k=lens_k, Hkv=hkv, Hq=Hq, D=int(rng.choice([16, 32, 64, 128, 256])),
                          dtype=[torch.bfloat16, torch.float16][int(rng.integers(2))],
                          causal=bool(rng.integers(2)), seed=seed * 1000 + i))
    return cases


VL_FWD = _draw_varlen(16, 41) + _draw_varlen_wide(N_WIDE // 4, 61, False)
VL_BWD = _draw_varlen(8, 43) + _draw_varlen_wide(N_WIDE // 8, 63, True)


def _vl_id(c):
    dt = "bf16" if c["dtype"] == torch.bfloat16 else "fp16"
    return f"d{c['D']}-{dt}-h{c['Hq']}kv{c['Hkv']}-{len(c['lens_q'])}seq-{'causal' if c['causal'] else 'full'}"


@pytest.mark.parametrize("c", VL_FWD, ids=[_vl_id(c) for c in VL_FWD])
def test_random_varlen_forward(c):
    from tests import test_varlen_parity as vp
    r = vp._check(c["lens_q"], c["lens_k"], c["Hq"], c["Hkv"], c["D"], c["dtype"], c["causal"], c["seed"])
    print(f"[result] varlen forward {_vl_id(c)}: O error ratio {r:.3f}", flush=True)


@pytest.mark.parametrize("c", VL_BWD, ids=[_vl_id(c) for c in VL_BWD])
def test_random_varlen_backward(c):
    from tests import test_varlen_bwd_parity as vbp
    vbp._check(c["lens_q"], c["lens_k"], c["Hq"], c["Hkv"], c["D"], c["dtype"], c["causal"], c["seed"])
