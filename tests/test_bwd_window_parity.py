"""GPU parity of the sliding-window backward (fa_bwd_window) against the float64 backward oracle's
window mask: every gradient element of every case, within the elementwise error bound of the
causal and full backward (tests/grad_bound.py, with the window's visible key set; the roundings are
the same, the window only removes terms). A query row whose window holds no key has a zero dQ row
and adds nothing to dK or dV."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity_util import f32_scale, to_f64
from tests import grad_bound as gb
from tests.test_bwd_parity import _dout, assert_within_bound

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import scaled_dot_product_fa2_amd as fa
    return fa


def _run(B, Hq, Hkv, Nq, Nkv, D, dtype, left, right, seed, scale=None):
    print(f"[case] bwd window ({left},{right}) B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nkv{Nkv} D{D} {dtype}", flush=True)
    fa = _fa()
    q, k, v = workloads.make_random(B, Hq, Hkv, Nq, Nkv, D, dtype, seed=seed)
    do = _dout(B, Hq, Nq, D, dtype, seed + 1)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_fwd_window(qd, kd, vd, window_left=left, window_right=right, scale=scale)
    # NaN-filled outputs: every element, the zero rows of empty windows included, must be written
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (qd, kd, vd))
    fa.fa_bwd(qd, kd, vd, o, lse, dod, scale=scale, window=(left, right), dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    win = (None if left < 0 else left, None if right < 0 else right)
    s = f32_scale(scale) if scale is not None else None
    if s is None:
        s = f32_scale(1.0 / np.sqrt(D))
    ref = oracle.attention_bwd_ref(to_f64(q), to_f64(k), to_f64(v), to_f64(do), causal=False, scale=s, window=win)
    bounds = gb.attention_bwd_bound(q, k, v, do, o, lse, ref[1], ref[2], causal=False, scale=s, dtype=dtype,
                                    window=win)
    worst = assert_within_bound((dq, dk, dv), ref, bounds, f"window ({left},{right}) D{D}")
    # a row whose window holds no key gets an exactly zero dQ row
    rows = np.arange(Nq)
    lo = np.maximum(0, rows - (Nq if left < 0 else left))
    hi = np.minimum(Nkv - 1, rows + (Nkv if right < 0 else right))
    empty = lo > hi
    assert np.all(to_f64(dq)[:, :, empty] == 0), "dQ of rows without keys must be zero"
    return worst


WINDOWS = [(0, 0), (1, 0), (63, 0), (64, 0), (100, 17), (5, 130), (-1, 3), (70, -1), (-1, -1)]


@pytest.mark.parametrize("left,right", WINDOWS, ids=[f"w{a}_{b}" for a, b in WINDOWS])
def test_bwd_window_shapes_d128(left, right):
    _run(1, 4, 2, 333, 333, 128, torch.bfloat16, left, right, seed=1900 + left + 7 * right)


@pytest.mark.parametrize("D", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_bwd_window_head_dims(D, dtype):
    _run(2, 2, 1, 200, 200, D, dtype, 48, 8, seed=1910 + D)


@pytest.mark.parametrize("Nq,Nkv,left,right", [(100, 300, 20, 20), (300, 100, 0, 0), (300, 100, 50, 0),
                                               (1, 500, 3, 7), (257, 257, 256, 256), (400, 90, 10, 200)])
def test_bwd_window_unequal_lengths_and_empty_rows(Nq, Nkv, left, right):
    """Rows past Nkv + left see no key under a bounded left side; keys far right of every row
    (Nkv > Nq + right) receive no gradient."""
    _run(1, 2, 2, Nq, Nkv, 64, torch.float16, left, right, seed=1920 + Nq + Nkv)


def test_bwd_window_custom_scale_gqa4():
    _run(1, 8, 2, 260, 260, 64, torch.bfloat16, 33, 33, seed=1931, scale=0.2)


def test_bwd_window_matches_causal_and_full_entry_points():
    """Window (-1, 0) gives fa_bwd(causal=True)'s gradients bitwise, (-1, -1) fa_bwd(causal=False)'s:
    the same tiles are visited in the same order and the extra masked terms are exact zeros."""
    print("[case] bwd window vs causal/full entry points", flush=True)
    fa = _fa()
    q, k, v = (t.to(DEV) for t in workloads.make_random(2, 8, 2, 500, 500, 128, torch.bfloat16, seed=1940))
    do = _dout(2, 8, 500, 128, torch.bfloat16, 1941).to(DEV)
    for (left, right), causal in (((-1, 0), True), ((-1, -1), False)):
        o, lse = fa.fa_fwd(q, k, v, causal=causal)
        gw = fa.fa_bwd(q, k, v, o, lse, do, window=(left, right))
        gc = fa.fa_bwd(q, k, v, o, lse, do, causal=causal)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), gw, gc):
            assert torch.equal(a, b), f"window ({left},{right}) vs causal={causal}: {name} differs"


def test_bwd_window_long_sequence_sampled():
    """A 1024-key causal window over 16384 tokens (GQA 4, bf16 D=128): dQ on sampled rows against the
    oracle restricted to each row's window, dK and dV of one key/value head in full against the
    oracle over the query rows that can see its keys."""
    print("[case] bwd window long sequence", flush=True)
    fa = _fa()
    w = workloads.WORKLOADS["gqa_b1h32kv8n16384d128"]
    left = 1024
    q, k, v = workloads.make_inputs(w)
    do = _dout(w.B, w.Hq, w.Nq, w.D, w.dtype, 1951)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_fwd_window(qd, kd, vd, window_left=left, window_right=0)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, lse, dod, window=(left, 0))
    torch.cuda.synchronize()
    sc = f32_scale(w.scale)
    rng = np.random.default_rng(1952)
    # keys 5000..5999 of kv head 3 are seen by query rows 5000..7023 of query heads 12..15
    k0, k1 = 5000, 6000
    r0, r1 = k0, k1 + left
    q64 = to_f64(q[:, :, r0:r1])
    do64 = to_f64(do[:, :, r0:r1])
    kv0 = r0 - left                      # keys the rows r0..r1 can see start here
    k64, v64 = to_f64(k[:, :, kv0:r1]), to_f64(v[:, :, kv0:r1])
    G = w.Hq // w.Hkv
    o64, lse64 = to_f64(o[:, :, r0:r1]), to_f64(lse[:, :, r0:r1])
    dk_ref = np.zeros((k1 - k0, w.D))
    dv_ref = np.zeros((k1 - k0, w.D))
    bk_sum = np.zeros((k1 - k0, w.D))
    bv_sum = np.zeros((k1 - k0, w.D))
    for h in range(3 * G, 4 * G):
        rq, rk, rv = _bwd_slice(q64[0, h], k64[0, 3], v64[0, 3], do64[0, h], left, sc)
        dk_ref += rk[k0 - kv0:k1 - kv0]
        dv_ref += rv[k0 - kv0:k1 - kv0]
        bq, bk, bv = gb.head_bwd_bound(q64[0, h], k64[0, 3], v64[0, 3], do64[0, h], o64[0, h], lse64[0, h],
                                       causal=False, scale=sc, dtype=w.dtype, window=(0, left))
        bk_sum += bk[k0 - kv0:k1 - kv0]
        bv_sum += bv[k0 - kv0:k1 - kv0]
        rows = sorted({0, 1, 511, 1023, r1 - r0 - 1, *map(int, rng.integers(0, r1 - r0, 6))})
        ratio = gb.bound_ratio(to_f64(dq[0, h, r0:r1])[rows], rq[rows], bq[rows])
        assert ratio <= 1.0, f"h={h}: dq rows, error / bound {ratio:.3f}"
    bk_sum, bv_sum = gb.finish_kv(bk_sum, bv_sum, dk_ref, dv_ref, w.dtype)
    for name, got, r, bnd in (("dk", dk[0, 3, k0:k1], dk_ref, bk_sum), ("dv", dv[0, 3, k0:k1], dv_ref, bv_sum)):
        ratio = gb.bound_ratio(to_f64(got), r, bnd)
        print(f"[result] window long sequence {name}: error / bound {ratio:.4f}", flush=True)
        assert ratio <= 1.0, f"{name}: error / bound {ratio:.3f}"


def _bwd_slice(qh, kh, vh, doh, left, scale):
    """Oracle gradients of a slice of query rows against the keys from ``left`` positions before its
    first row: key j of the slice sits ``left`` places earlier than row j, so row i sees keys
    i .. i + left, which is the oracle's window (0, left) on the sliced tensors."""
    return oracle.head_bwd_ref(qh, kh, vh, doh, causal=False, scale=scale, window=(0, left))
