"""GPU parity of the sliding-window forward (fa_fwd_window) against the float64 oracle's window
mask: every output element of every case, same tolerances as the causal and full forward. A row
whose window holds no key must come back as O = 0 and LSE = -inf."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity_util import O_TOL, LSE_ATOL, f32_scale, o_ratio, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import scaled_dot_product_fa2_amd as fa
    return fa


def _run(B, Hq, Hkv, Nq, Nkv, D, dtype, left, right, seed, scale=None):
    print(f"[case] window ({left},{right}) B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nkv{Nkv} D{D} {dtype}", flush=True)
    fa = _fa()
    q, k, v = workloads.make_random(B, Hq, Hkv, Nq, Nkv, D, dtype, seed=seed)
    o, lse = fa.fa_fwd_window(q.to(DEV), k.to(DEV), v.to(DEV), window_left=left, window_right=right, scale=scale)
    torch.cuda.synchronize()
    win = (None if left < 0 else left, None if right < 0 else right)
    s = f32_scale(scale) if scale is not None else None
    o_ref, l_ref = oracle.attention_ref(to_f64(q), to_f64(k), to_f64(v), causal=False, scale=s, window=win)
    og, lg = to_f64(o), to_f64(lse)
    assert np.all(np.isfinite(og)), "non-finite O"
    ratio = o_ratio(og, o_ref, dtype)
    assert ratio <= 1.0, f"O error ratio {ratio:.3f} > 1 ({O_TOL[dtype]})"
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lg), empty), "rows without keys must have LSE = -inf, and only they"
    if (~empty).any():
        err = np.max(np.abs(lg[~empty] - l_ref[~empty]))
        assert err <= LSE_ATOL, f"LSE error {err:.2e}"
    return ratio


WINDOWS = [(0, 0), (1, 0), (63, 0), (64, 0), (100, 0), (200, 17), (5, 130), (-1, 0), (-1, -1), (70, -1), (-1, 3)]


@pytest.mark.parametrize("left,right", WINDOWS, ids=[f"w{a}_{b}" for a, b in WINDOWS])
def test_window_shapes_d128(left, right):
    _run(1, 4, 2, 333, 333, 128, torch.bfloat16, left, right, seed=900 + left + 7 * right)


@pytest.mark.parametrize("D", [16, 32, 64, 256])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_window_head_dims(D, dtype):
    _run(2, 2, 1, 200, 200, D, dtype, 48, 8, seed=910 + D)


@pytest.mark.parametrize("Nq,Nkv,left,right", [(100, 300, 20, 20), (300, 100, 0, 0), (300, 100, 50, 0),
                                               (1, 500, 3, 7), (257, 257, 256, 256)])
def test_window_unequal_lengths_and_empty_rows(Nq, Nkv, left, right):
    """Rows past Nkv + left see nothing under a bounded left side (O = 0, LSE = -inf)."""
    _run(1, 2, 2, Nq, Nkv, 64, torch.float16, left, right, seed=920 + Nq + Nkv)


def test_window_matches_causal_and_full_entry_points():
    """(-1, 0) reproduces fa_fwd(causal=True) bitwise, and (-1, -1) fa_fwd(causal=False)."""
    fa = _fa()
    q, k, v = (t.to(DEV) for t in workloads.make_random(2, 8, 2, 500, 500, 128, torch.bfloat16, seed=930))
    for (left, right), causal in (((-1, 0), True), ((-1, -1), False)):
        ow, lw = fa.fa_fwd_window(q, k, v, window_left=left, window_right=right)
        oc, lc = fa.fa_fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(ow, oc) and torch.equal(lw, lc), f"window ({left},{right}) vs causal={causal}"


def test_window_long_sequence_sampled():
    """A 4096-window over 16384 tokens (GQA 4, bf16 D=128), sampled rows against the oracle."""
    fa = _fa()
    w = workloads.WORKLOADS["gqa_b1h32kv8n16384d128"]
    q, k, v = workloads.make_inputs(w)
    print("[case] window (4096, 0) over gqa_b1h32kv8n16384d128", flush=True)
    o, lse = fa.fa_fwd_window(q.to(DEV), k.to(DEV), v.to(DEV), window_left=4096, window_right=0)
    torch.cuda.synchronize()
    rows = [0, 1, 4095, 4096, 4097, 8191, 12000, 16383]
    for h in (0, 17):
        kvh = h // (w.Hq // w.Hkv)
        o_ref, l_ref = oracle.attention_rows(
            to_f64(q[0:1, h:h + 1]), to_f64(k[0:1, kvh:kvh + 1]), to_f64(v[0:1, kvh:kvh + 1]), 0, 0, rows,
            causal=False, scale=f32_scale(w.scale), window=(4096, 0))
        og = to_f64(o[0, h])[rows]
        assert o_ratio(og, o_ref, w.dtype) <= 1.0
        assert np.max(np.abs(to_f64(lse[0, h])[rows] - l_ref)) <= LSE_ATOL
