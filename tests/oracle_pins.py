"""Checks that pin the float64 oracle to facts that do not come from the oracle itself.

Each pin takes an oracle module (anything exposing ``attention_ref`` and
``attention_rows``) and raises AssertionError when the module disagrees with
the fact it pins. The pins are run against the real oracle in
``test_oracle.py`` and against deliberately broken copies of it in
``test_oracle_mutants.py``, which shows that each plausible mistake is caught.

Sources of truth used here: closed forms of softmax attention, invariances of
the definition, pure-Python brute force on tiny inputs, and two independent
library routines (torch's float64 scaled_dot_product_attention on the CPU and
scipy's logsumexp).
"""
from __future__ import annotations

import math

import numpy as np
import torch
from scipy.special import logsumexp

TOL = 1e-11


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max rel err {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------------------------
# 1. Brute force on tiny inputs: pure-Python loops, math.fsum, no max subtraction.

def _brute(q, k, v, causal, scale):
    B, Hq, Nq, D = q.shape
    Hkv, Nkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    o = np.zeros((B, Hq, Nq, Dv))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(Nq):
                keys = [j for j in range(Nkv) if (not causal) or j <= i]
                s = {j: scale * math.fsum(float(q[b, h, i, d]) * float(k[b, g, j, d]) for d in range(D))
                     for j in keys}
                z = math.log(math.fsum(math.exp(s[j]) for j in keys))
                lse[b, h, i] = z
                for e in range(Dv):
                    o[b, h, i, e] = math.fsum(math.exp(s[j] - z) * float(v[b, g, j, e]) for j in keys)
    return o, lse


def pin_brute_force(mod):
    rng = _rng(11)
    cases = 0
    for Hq, Hkv in [(1, 1), (2, 1), (4, 2), (2, 2)]:
        for Nq, Nkv in [(1, 1), (3, 5), (6, 6), (9, 4), (5, 9)]:
            for D in (1, 3, 5):
                for causal in (False, True):
                    q = _rand(rng, 1, Hq, Nq, D)
                    k = _rand(rng, 1, Hkv, Nkv, D)
                    v = _rand(rng, 1, Hkv, Nkv, D + 1)
                    scale = 0.7
                    o, lse = mod.attention_ref(q, k, v, causal=causal, scale=scale)
                    ob, lb = _brute(q, k, v, causal, scale)
                    _close(o, ob, what=f"brute o Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} D={D} causal={causal}")
                    _close(lse, lb, what=f"brute lse Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} D={D} causal={causal}")
                    cases += 1
    assert cases == 120


# ---------------------------------------------------------------------------------------------
# 2. Library routine: torch scaled_dot_product_attention in float64 on the CPU. Its causal mask is
#    a lower triangle anchored at the top-left corner, the reading the oracle takes.

def pin_sdpa_float64(mod):
    rng = _rng(12)
    shapes = [
        (2, 4, 4, 33, 33, 16, False, None), (2, 4, 4, 33, 33, 16, True, None),
        (1, 8, 2, 40, 40, 32, True, 0.3), (1, 8, 1, 17, 29, 8, False, 0.5),
        (1, 6, 3, 24, 50, 64, True, None), (1, 4, 4, 50, 24, 16, True, 1.25),
        (3, 2, 1, 7, 130, 128, False, None),
    ]
    for B, Hq, Hkv, Nq, Nkv, D, causal, scale in shapes:
        q = _rand(rng, B, Hq, Nq, D)
        k = _rand(rng, B, Hkv, Nkv, D)
        v = _rand(rng, B, Hkv, Nkv, D)
        o, _ = mod.attention_ref(q, k, v, causal=causal, scale=scale)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal,
            scale=scale, enable_gqa=(Hq != Hkv)).numpy()
        _close(o, ref, tol=1e-10, what=f"sdpa {B,Hq,Hkv,Nq,Nkv,D,causal,scale}")


# ---------------------------------------------------------------------------------------------
# 3. Library routine: scipy logsumexp of the masked scaled scores (scores by einsum in float64).

def pin_lse_scipy(mod):
    rng = _rng(13)
    for B, Hq, Hkv, Nq, Nkv, D, causal, scale in [(2, 4, 2, 31, 31, 32, True, 0.2),
                                                   (1, 3, 1, 12, 45, 16, False, 0.9),
                                                   (1, 2, 2, 45, 12, 8, True, 1.7)]:
        q = _rand(rng, B, Hq, Nq, D) * 2.0
        k = _rand(rng, B, Hkv, Nkv, D)
        v = _rand(rng, B, Hkv, Nkv, D)
        _, lse = mod.attention_ref(q, k, v, causal=causal, scale=scale)
        kk = np.repeat(k, Hq // Hkv, axis=1)
        s = scale * np.einsum("bhid,bhjd->bhij", q, kk)
        if causal:
            s = np.where(np.tril(np.ones((Nq, Nkv), dtype=bool)), s, -np.inf)
        _close(lse, logsumexp(s, axis=-1), what="lse vs scipy logsumexp")


# ---------------------------------------------------------------------------------------------
# 4. Closed forms.

def pin_single_key(mod):
    """One key: every row attends only to it, so o = v_0 and lse = scale * q.k_0."""
    rng = _rng(14)
    for causal in (False, True):
        q = _rand(rng, 2, 4, 9, 16)
        k = _rand(rng, 2, 2, 1, 16)
        v = _rand(rng, 2, 2, 1, 16)
        o, lse = mod.attention_ref(q, k, v, causal=causal, scale=0.25)
        kk = np.repeat(k, 2, axis=1)
        vv = np.repeat(v, 2, axis=1)
        _close(o, np.broadcast_to(vv, o.shape), what="single key o")
        _close(lse, 0.25 * np.sum(q * kk, axis=-1), what="single key lse")


def pin_zero_query(mod):
    """Q = 0: uniform weights. Non-causal: o = mean of all V rows, lse = ln Nkv.
    Causal: o_i = mean of V rows 0..i, lse_i = ln(i + 1)."""
    rng = _rng(15)
    B, Hq, Hkv, N, D = 2, 4, 2, 37, 8
    q = np.zeros((B, Hq, N, D))
    k = _rand(rng, B, Hkv, N, D)
    v = _rand(rng, B, Hkv, N, D)
    vv = np.repeat(v, Hq // Hkv, axis=1)
    o, lse = mod.attention_ref(q, k, v, causal=False, scale=0.3)
    _close(o, np.broadcast_to(vv.mean(axis=2, keepdims=True), o.shape), what="Q=0 non-causal o")
    _close(lse, np.full(lse.shape, math.log(N)), what="Q=0 non-causal lse")
    o, lse = mod.attention_ref(q, k, v, causal=True, scale=0.3)
    cum = np.cumsum(vv, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    _close(o, cum, what="Q=0 causal o")
    _close(lse, np.broadcast_to(np.log(np.arange(1, N + 1)), lse.shape), what="Q=0 causal lse")


def pin_first_causal_row(mod):
    """Causal row 0 sees only key 0: o_0 = v_0 and lse_0 = scale * q_0.k_0."""
    rng = _rng(16)
    q = _rand(rng, 2, 6, 20, 32)
    k = _rand(rng, 2, 3, 20, 32)
    v = _rand(rng, 2, 3, 20, 32)
    o, lse = mod.attention_ref(q, k, v, causal=True, scale=0.4)
    kk = np.repeat(k, 2, axis=1)
    vv = np.repeat(v, 2, axis=1)
    _close(o[:, :, 0], vv[:, :, 0], what="first causal row o")
    _close(lse[:, :, 0], 0.4 * np.sum(q[:, :, 0] * kk[:, :, 0], axis=-1), what="first causal row lse")


def pin_default_scale(mod):
    """Without an explicit scale the scores are scaled by 1/sqrt(D)."""
    rng = _rng(17)
    q = _rand(rng, 1, 2, 10, 16)
    k = _rand(rng, 1, 2, 10, 16)
    v = _rand(rng, 1, 2, 10, 16)
    o1, l1 = mod.attention_ref(q, k, v, causal=False)
    o2, l2 = mod.attention_ref(q, k, v, causal=False, scale=0.25)
    _close(o1, o2, what="default scale o")
    _close(l1, l2, what="default scale lse")


def pin_scale_moves_to_q(mod):
    """scale enters only through s = scale * q.k: (2q, s) equals (q, 2s)."""
    rng = _rng(18)
    q = _rand(rng, 1, 2, 12, 8)
    k = _rand(rng, 1, 1, 15, 8)
    v = _rand(rng, 1, 1, 15, 8)
    for causal in (False, True):
        o1, l1 = mod.attention_ref(2.0 * q, k, v, causal=causal, scale=0.3)
        o2, l2 = mod.attention_ref(q, k, v, causal=causal, scale=0.6)
        _close(o1, o2, what="scale o")
        _close(l1, l2, what="scale lse")
        o3, l3 = mod.attention_ref(q, k, v, causal=causal, scale=0.3)
        assert np.max(np.abs(l3 - l2)) > 1e-3, "changing the scale must change the result"


# ---------------------------------------------------------------------------------------------
# 5. Invariants of the definition.

def pin_convex_rows(mod):
    """Each output row is a convex combination of the visible V rows: within their per-column
    range, and a V of all ones maps to all ones."""
    rng = _rng(19)
    q = _rand(rng, 1, 2, 25, 16) * 3
    k = _rand(rng, 1, 2, 25, 16)
    v = _rand(rng, 1, 2, 25, 16)
    for causal in (False, True):
        o, _ = mod.attention_ref(q, k, v, causal=causal, scale=0.5)
        for i in range(25):
            vis = v[:, :, : i + 1] if causal else v
            assert np.all(o[:, :, i] <= vis.max(axis=2) + 1e-12)
            assert np.all(o[:, :, i] >= vis.min(axis=2) - 1e-12)
        o1, _ = mod.attention_ref(q, k, np.ones_like(v), causal=causal, scale=0.5)
        _close(o1, np.ones_like(o1), what="weights sum to one")


def pin_affine_v(mod):
    """V -> a V + 1 c^T gives O -> a O + 1 c^T and leaves lse unchanged."""
    rng = _rng(20)
    q = _rand(rng, 2, 2, 14, 8)
    k = _rand(rng, 2, 2, 19, 8)
    v = _rand(rng, 2, 2, 19, 8)
    c = _rand(rng, 8)
    for causal in (False, True):
        o, lse = mod.attention_ref(q, k, v, causal=causal, scale=0.45)
        o2, lse2 = mod.attention_ref(q, k, -1.5 * v + c, causal=causal, scale=0.45)
        _close(o2, -1.5 * o + c, what="affine v o")
        _close(lse2, lse, what="affine v lse")


def pin_key_shift(mod):
    """Adding the same vector u to every key adds scale*q_i.u to every score of row i:
    O is unchanged and lse_i grows by exactly scale*q_i.u."""
    rng = _rng(21)
    q = _rand(rng, 1, 4, 16, 8)
    k = _rand(rng, 1, 2, 16, 8)
    v = _rand(rng, 1, 2, 16, 8)
    u = _rand(rng, 8)
    for causal in (False, True):
        o, lse = mod.attention_ref(q, k, v, causal=causal, scale=0.6)
        o2, lse2 = mod.attention_ref(q, k + u, v, causal=causal, scale=0.6)
        _close(o2, o, what="key shift o")
        _close(lse2, lse + 0.6 * (q @ u), what="key shift lse")


def pin_gqa_is_repeated_mha(mod):
    """Grouped heads equal ordinary multi-head attention with each K/V head repeated for its
    group of consecutive query heads."""
    rng = _rng(22)
    for Hq, Hkv in [(8, 2), (6, 3), (4, 1)]:
        q = _rand(rng, 2, Hq, 11, 16)
        k = _rand(rng, 2, Hkv, 13, 16)
        v = _rand(rng, 2, Hkv, 13, 16)
        for causal in (False, True):
            o, lse = mod.attention_ref(q, k, v, causal=causal, scale=0.3)
            G = Hq // Hkv
            o2, lse2 = mod.attention_ref(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1),
                                         causal=causal, scale=0.3)
            _close(o, o2, what="gqa o")
            _close(lse, lse2, what="gqa lse")
    # and it is not the same as pairing query head h with K/V head h % Hkv
    q = _rand(rng, 1, 4, 6, 8)
    k = _rand(rng, 1, 2, 6, 8)
    v = _rand(rng, 1, 2, 6, 8)
    o, _ = mod.attention_ref(q, k, v, causal=False, scale=0.3)
    o_alt, _ = mod.attention_ref(q, np.tile(k, (1, 2, 1, 1)), np.tile(v, (1, 2, 1, 1)), causal=False,
                                 scale=0.3)
    assert np.max(np.abs(o - o_alt)) > 1e-3


def pin_causal_prefix(mod):
    """Causal row i equals non-causal attention of that query over keys 0..i."""
    rng = _rng(23)
    q = _rand(rng, 1, 2, 12, 8)
    k = _rand(rng, 1, 2, 12, 8)
    v = _rand(rng, 1, 2, 12, 8)
    o, lse = mod.attention_ref(q, k, v, causal=True, scale=0.8)
    for i in range(12):
        oi, li = mod.attention_ref(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], causal=False, scale=0.8)
        _close(o[:, :, i:i + 1], oi, what=f"causal prefix o row {i}")
        _close(lse[:, :, i:i + 1], li, what=f"causal prefix lse row {i}")


def pin_key_permutation(mod):
    """Non-causal attention does not depend on the order of the (key, value) pairs."""
    rng = _rng(24)
    q = _rand(rng, 2, 2, 9, 8)
    k = _rand(rng, 2, 2, 21, 8)
    v = _rand(rng, 2, 2, 21, 8)
    perm = rng.permutation(21)
    o, lse = mod.attention_ref(q, k, v, causal=False, scale=0.5)
    o2, lse2 = mod.attention_ref(q, k[:, :, perm], v[:, :, perm], causal=False, scale=0.5)
    _close(o2, o, what="perm o")
    _close(lse2, lse, what="perm lse")


def pin_two_block_merge(mod):
    """Splitting the keys in two blocks and merging the partial results with the weights
    exp(lse_part - lse) reproduces the full result; lse = ln(e^lse1 + e^lse2)."""
    rng = _rng(25)
    q = _rand(rng, 1, 3, 10, 16) * 2
    k = _rand(rng, 1, 3, 30, 16)
    v = _rand(rng, 1, 3, 30, 16)
    o, lse = mod.attention_ref(q, k, v, causal=False, scale=0.35)
    o1, l1 = mod.attention_ref(q, k[:, :, :13], v[:, :, :13], causal=False, scale=0.35)
    o2, l2 = mod.attention_ref(q, k[:, :, 13:], v[:, :, 13:], causal=False, scale=0.35)
    lm = np.logaddexp(l1, l2)
    _close(lm, lse, what="merge lse")
    _close(np.exp(l1 - lm)[..., None] * o1 + np.exp(l2 - lm)[..., None] * o2, o, what="merge o")


def pin_strided_views(mod):
    """A (B, N, H, D) storage viewed as (B, H, N, D) gives the same result as a contiguous copy."""
    rng = _rng(26)
    k_bsnd = _rand(rng, 2, 17, 2, 8)
    v_bsnd = _rand(rng, 2, 17, 2, 8)
    q = _rand(rng, 2, 4, 17, 8)
    k = k_bsnd.transpose(0, 2, 1, 3)
    v = v_bsnd.transpose(0, 2, 1, 3)
    for causal in (False, True):
        o, lse = mod.attention_ref(q, k, v, causal=causal, scale=0.5)
        o2, lse2 = mod.attention_ref(q, np.ascontiguousarray(k), np.ascontiguousarray(v), causal=causal, scale=0.5)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def pin_rows_agree(mod):
    """attention_rows (used for sampled checks of large shapes) equals the full computation."""
    rng = _rng(27)
    q = _rand(rng, 2, 4, 40, 16)
    k = _rand(rng, 2, 2, 40, 16)
    v = _rand(rng, 2, 2, 40, 16)
    for causal in (False, True):
        o, lse = mod.attention_ref(q, k, v, causal=causal, scale=0.3)
        for b, h in [(0, 0), (1, 3), (0, 2)]:
            rows = [0, 5, 17, 39]
            orow, lrow = mod.attention_rows(q, k, v, b, h, rows, causal=causal, scale=0.3)
            _close(orow, o[b, h, rows], what="rows o")
            _close(lrow, lse[b, h, rows], what="rows lse")


def pin_large_scores(mod):
    """Rows whose score ranges differ by far more than float64's exponent range: each row must be
    shifted by its own maximum. Keys are one-hot, so the scores are read off directly: a zero
    query gives uniform weights (o = mean V, lse = ln 4); a query of 2000 along key 2 puts all
    weight on value row 2 with lse = 2000 (the other keys add e^-2000, below double precision)."""
    k = np.eye(4)[None, None]
    v = _rand(_rng(28), 1, 1, 4, 3)
    q = np.zeros((1, 1, 3, 4))
    q[0, 0, 1, 2] = 2000.0
    q[0, 0, 2, 0] = -1500.0  # key 0 scores -1500, the others 0: uniform over keys 1..3
    o, lse = mod.attention_ref(q, k, v, causal=False, scale=1.0)
    _close(o[0, 0, 0], v[0, 0].mean(axis=0), what="large scores, zero row o")
    _close(lse[0, 0, 0], math.log(4.0), what="large scores, zero row lse")
    _close(o[0, 0, 1], v[0, 0, 2], what="large scores, peaked row o")
    _close(lse[0, 0, 1], 2000.0, what="large scores, peaked row lse")
    _close(o[0, 0, 2], v[0, 0, 1:].mean(axis=0), what="large scores, negative row o")
    _close(lse[0, 0, 2], math.log(3.0), what="large scores, negative row lse")


# ---------------------------------------------------------------------------------------------
# Sliding windows: row i sees keys i - left .. i + right (None = unbounded on that side).

def _brute_window(q, k, v, left, right, scale):
    B, Hq, Nq, D = q.shape
    Hkv, Nkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    o = np.zeros((B, Hq, Nq, Dv))
    lse = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(Nq):
                keys = [j for j in range(Nkv) if (left is None or j >= i - left) and (right is None or j <= i + right)]
                if not keys:
                    continue
                s = {j: scale * math.fsum(float(q[b, h, i, d]) * float(k[b, g, j, d]) for d in range(D)) for j in keys}
                z = math.log(math.fsum(math.exp(s[j]) for j in keys))
                lse[b, h, i] = z
                for e in range(Dv):
                    o[b, h, i, e] = math.fsum(math.exp(s[j] - z) * float(v[b, g, j, e]) for j in keys)
    return o, lse


def _close_lse(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert np.array_equal(np.isneginf(a), np.isneginf(b)), f"{what}: -inf pattern differs"
    fin = ~np.isneginf(b)
    _close(a[fin], b[fin], what=what)


def pin_window_brute_force(mod):
    rng = _rng(31)
    for Hq, Hkv in [(1, 1), (2, 1)]:
        for Nq, Nkv in [(6, 6), (7, 4), (4, 9)]:
            for left, right in [(0, 0), (1, 0), (2, 1), (None, 1), (1, None), (3, 2), (0, None)]:
                q = _rand(rng, 1, Hq, Nq, 3)
                k = _rand(rng, 1, Hkv, Nkv, 3)
                v = _rand(rng, 1, Hkv, Nkv, 4)
                o, lse = mod.attention_ref(q, k, v, causal=False, scale=0.8, window=(left, right))
                ob, lb = _brute_window(q, k, v, left, right, 0.8)
                what = f"window brute Hq={Hq} Nq={Nq} Nkv={Nkv} window=({left},{right})"
                _close(o, ob, what=what + " o")
                _close_lse(lse, lb, what=what + " lse")


def pin_window_sdpa_bool_mask(mod):
    """torch float64 SDPA with an explicit boolean band mask (windows that leave no row empty)."""
    rng = _rng(32)
    for Nq, Nkv, left, right in [(20, 20, 5, 0), (20, 20, 3, 4), (16, 30, 7, 7), (30, 16, None, 2)]:
        q = _rand(rng, 1, 4, Nq, 8)
        k = _rand(rng, 1, 2, Nkv, 8)
        v = _rand(rng, 1, 2, Nkv, 8)
        o, _ = mod.attention_ref(q, k, v, causal=False, scale=0.4, window=(left, right))
        i = np.arange(Nq)[:, None]
        j = np.arange(Nkv)[None, :]
        band = np.ones((Nq, Nkv), dtype=bool)
        if left is not None:
            band &= j >= i - left
        if right is not None:
            band &= j <= i + right
        assert band.any(axis=1).all()
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=torch.from_numpy(band),
            scale=0.4, enable_gqa=True).numpy()
        _close(o, ref, tol=1e-10, what=f"window sdpa ({left},{right})")


def pin_window_special_cases(mod):
    rng = _rng(33)
    q = _rand(rng, 1, 2, 9, 4)
    k = _rand(rng, 1, 2, 9, 4)
    v = _rand(rng, 1, 2, 9, 5)
    # (unbounded, 0) is the causal mask; (unbounded, unbounded) is no mask
    oc, lc = mod.attention_ref(q, k, v, causal=True, scale=0.6)
    ow, lw = mod.attention_ref(q, k, v, causal=False, scale=0.6, window=(None, 0))
    _close(ow, oc, what="window (None, 0) o")
    _close(lw, lc, what="window (None, 0) lse")
    of, lf = mod.attention_ref(q, k, v, causal=False, scale=0.6)
    ou, lu = mod.attention_ref(q, k, v, causal=False, scale=0.6, window=(None, None))
    _close(ou, of, what="window (None, None) o")
    _close(lu, lf, what="window (None, None) lse")
    # (0, 0): each row sees only its own position, so o_i = v_i and lse_i = scale * q_i . k_i;
    # rows past the last key see nothing: o = 0, lse = -inf
    qq = _rand(rng, 1, 1, 7, 4)
    kk = _rand(rng, 1, 1, 5, 4)
    vv = _rand(rng, 1, 1, 5, 3)
    o0, l0 = mod.attention_ref(qq, kk, vv, causal=False, scale=0.5, window=(0, 0))
    _close(o0[0, 0, :5], vv[0, 0], what="window (0, 0) o")
    _close(l0[0, 0, :5], 0.5 * np.sum(qq[0, 0, :5] * kk[0, 0], axis=1), what="window (0, 0) lse")
    assert np.all(o0[0, 0, 5:] == 0.0) and np.all(np.isneginf(l0[0, 0, 5:])), "empty rows: o = 0, lse = -inf"
    # the sampled-rows entry point agrees with the full computation under a window
    rows = [0, 4, 8]
    o_r, l_r = mod.attention_rows(q, k, v, 0, 1, rows, causal=False, scale=0.6, window=(2, 1))
    o_a, l_a = mod.attention_ref(q, k, v, causal=False, scale=0.6, window=(2, 1))
    _close(o_r, o_a[0, 1, rows], what="window rows o")
    _close(l_r, l_a[0, 1, rows], what="window rows lse")


# ---------------------------------------------------------------------------------------------
# Packed variable-length sequences (CSR offsets).

def pin_varlen_against_masked_sdpa(mod):
    """Packed sequences = one padded batch whose padding keys are masked out, computed by torch
    float64 SDPA with a boolean mask (causal positions counted per sequence)."""
    rng = _rng(41)
    lens_q = [5, 1, 9, 0, 7]
    lens_k = [5, 4, 12, 3, 7]
    Hq, Hkv, D = 4, 2, 8
    cq = np.concatenate([[0], np.cumsum(lens_q)])
    ck = np.concatenate([[0], np.cumsum(lens_k)])
    q = _rand(rng, int(cq[-1]), Hq, D)
    k = _rand(rng, int(ck[-1]), Hkv, D)
    v = _rand(rng, int(ck[-1]), Hkv, D)
    for causal in (False, True):
        o, lse = mod.attention_varlen_ref(q, k, v, cq, ck, causal=causal, scale=0.45)
        for b in range(len(lens_q)):
            nq, nk = lens_q[b], lens_k[b]
            if nq == 0:
                continue
            qb = torch.from_numpy(q[cq[b]:cq[b + 1]].transpose(1, 0, 2).copy())[None]
            kb = torch.from_numpy(k[ck[b]:ck[b + 1]].transpose(1, 0, 2).copy())[None]
            vb = torch.from_numpy(v[ck[b]:ck[b + 1]].transpose(1, 0, 2).copy())[None]
            mask = torch.ones(nq, nk, dtype=torch.bool)
            if causal:
                mask = torch.tril(mask)
            ref = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask, scale=0.45,
                                                                   enable_gqa=True)[0].numpy().transpose(1, 0, 2)
            _close(o[cq[b]:cq[b + 1]], ref, tol=1e-10, what=f"varlen seq {b} causal={causal}")
            s = 0.45 * np.einsum("ihd,jhd->hij", q[cq[b]:cq[b + 1]], np.repeat(k[ck[b]:ck[b + 1]], Hq // Hkv, axis=1))
            if causal:
                s = np.where(np.tril(np.ones((nq, nk), dtype=bool)), s, -np.inf)
            _close(lse[:, cq[b]:cq[b + 1]], logsumexp(s, axis=-1), what=f"varlen lse seq {b}")


def pin_varlen_single_and_empty(mod):
    """One sequence is the dense computation; a sequence without keys gives o = 0, lse = -inf."""
    rng = _rng(42)
    q = _rand(rng, 11, 2, 4)
    k = _rand(rng, 13, 2, 4)
    v = _rand(rng, 13, 2, 4)
    o, lse = mod.attention_varlen_ref(q, k, v, [0, 11], [0, 13], causal=True, scale=0.7)
    od, ld = mod.attention_ref(q.transpose(1, 0, 2)[None], k.transpose(1, 0, 2)[None], v.transpose(1, 0, 2)[None],
                               causal=True, scale=0.7)
    _close(o, od[0].transpose(1, 0, 2), what="varlen single o")
    _close(lse, ld[0], what="varlen single lse")
    o2, l2 = mod.attention_varlen_ref(q, k, v, [0, 4, 11], [0, 13, 13], causal=False, scale=0.7)
    assert np.all(o2[4:] == 0.0) and np.all(np.isneginf(l2[:, 4:])), "rows of a key-less sequence"


ALL_PINS = [
    pin_brute_force, pin_sdpa_float64, pin_lse_scipy, pin_single_key, pin_zero_query,
    pin_first_causal_row, pin_default_scale, pin_scale_moves_to_q, pin_convex_rows, pin_affine_v,
    pin_key_shift, pin_gqa_is_repeated_mha, pin_causal_prefix, pin_key_permutation,
    pin_two_block_merge, pin_strided_views, pin_rows_agree, pin_large_scores,
    pin_window_brute_force, pin_window_sdpa_bool_mask, pin_window_special_cases,
    pin_varlen_against_masked_sdpa, pin_varlen_single_and_empty,
]
