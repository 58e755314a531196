"""Checks that pin the float64 backward oracle to facts that do not come from it.

Each pin takes a backward-oracle module (anything exposing ``attention_bwd_ref``,
``attention_varlen_bwd_ref`` and ``dq_rows``) and raises AssertionError when the module disagrees with the
fact it pins. They run against the real module in ``test_oracle_bwd.py`` and
against deliberately broken copies of it there too.

Sources of truth: central finite differences of the (separately pinned) float64
forward oracle, torch's float64 autograd through scaled_dot_product_attention on
the CPU, and identities of the softmax gradient: the rows of dS sum to zero (so
the dK rows of a head sum to zero), the softmax weights sum to one (so the dV
rows sum to the dO rows), a single key carries all the weight, grouped heads
are repeated heads, and the scale can move onto Q.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as fwd_oracle

TOL = 1e-11


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max rel err {err:.3e} > {tol:.1e}"


def _inputs(seed, B, Hq, Hkv, Nq, Nkv, D, Dv=None):
    rng = _rng(seed)
    Dv = D if Dv is None else Dv
    return (rng.standard_normal((B, Hq, Nq, D)), rng.standard_normal((B, Hkv, Nkv, D)),
            rng.standard_normal((B, Hkv, Nkv, Dv)), rng.standard_normal((B, Hq, Nq, Dv)))


# 1. Central finite differences of L = sum(dO * O) through the forward oracle.
def pin_bwd_finite_differences(mod):
    for causal, shape in ((False, (1, 2, 1, 4, 5, 3)), (True, (1, 2, 1, 5, 4, 3)), (True, (1, 1, 1, 4, 4, 2))):
        q, k, v, do = _inputs(11 + causal, *shape)
        scale = 0.7
        dq, dk, dv = mod.attention_bwd_ref(q, k, v, do, causal=causal, scale=scale)

        def loss(q_, k_, v_):
            o, _ = fwd_oracle.attention_ref(q_, k_, v_, causal=causal, scale=scale)
            return float(np.sum(o * do))

        h = 1e-5
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(g, num, tol=1e-7, what=f"finite differences d{name} causal={causal}")


# 2. torch float64 autograd through scaled_dot_product_attention (is_causal is top-left).
def pin_bwd_torch_autograd(mod):
    for causal, shape in ((False, (2, 4, 2, 13, 11, 8)), (True, (1, 6, 3, 17, 17, 16)), (True, (1, 2, 2, 9, 14, 4))):
        q, k, v, do = _inputs(21 + causal, *shape)
        scale = 1.0 / np.sqrt(shape[-1]) * 1.3
        dq, dk, dv = mod.attention_bwd_ref(q, k, v, do, causal=causal, scale=scale)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                                             enable_gqa=shape[1] != shape[2])
        o.backward(torch.tensor(do, dtype=torch.float64))
        _close(dq, tq.grad.numpy(), tol=1e-12, what="autograd dq")
        _close(dk, tk.grad.numpy(), tol=1e-12, what="autograd dk")
        _close(dv, tv.grad.numpy(), tol=1e-12, what="autograd dv")


# 3. Rows of dS sum to zero, so the dK rows of each key/value head sum to zero.
def pin_bwd_dk_rows_sum_to_zero(mod):
    for causal in (False, True):
        q, k, v, do = _inputs(31, 2, 4, 2, 19, 19, 8)
        _, dk, _ = mod.attention_bwd_ref(q, k, v, do, causal=causal, scale=0.4)
        s = dk.sum(axis=2)
        assert np.max(np.abs(s)) <= 1e-11 * (1 + np.max(np.abs(dk))), f"sum_j dK_j = {np.max(np.abs(s)):.3e}"


# 4. Softmax weights sum to one, so sum_j dV_j = sum over the group's rows of dO.
def pin_bwd_dv_rows_sum_to_do(mod):
    for causal in (False, True):
        q, k, v, do = _inputs(41, 1, 6, 2, 15, 15, 4)
        _, _, dv = mod.attention_bwd_ref(q, k, v, do, causal=causal, scale=0.5)
        for kvh in range(2):
            want = do[0, 3 * kvh:3 * kvh + 3].sum(axis=(0, 1))
            _close(dv[0, kvh].sum(axis=0), want, what=f"sum_j dV_j kvh={kvh}")


# 5. One key: every weight is 1, so dV_0 = sum of dO, and dQ = dK = 0.
def pin_bwd_single_key(mod):
    q, k, v, do = _inputs(51, 2, 2, 1, 7, 1, 5)
    dq, dk, dv = mod.attention_bwd_ref(q, k, v, do, causal=False, scale=0.9)
    assert np.max(np.abs(dq)) <= 1e-12 and np.max(np.abs(dk)) <= 1e-12
    _close(dv[:, 0, 0], do.sum(axis=(1, 2)), what="single-key dV")


# 6. Q = 0: uniform weights 1/Nkv, so dV_j = (1/Nkv) * sum of dO over the group's rows.
def pin_bwd_zero_query(mod):
    _, k, v, do = _inputs(61, 1, 2, 1, 6, 9, 3)
    q = np.zeros((1, 2, 6, 3))
    _, _, dv = mod.attention_bwd_ref(q, k, v, do, causal=False, scale=1.0)
    want = do[0].sum(axis=(0, 1)) / 9.0
    _close(dv[0, 0], np.broadcast_to(want, (9, 3)), what="Q=0 dV")


# 7. Grouped heads are repeated heads: GQA gradients equal MHA ones with K/V repeated,
#    dK and dV summed over each group.
def pin_bwd_gqa_is_repeated_mha(mod):
    q, k, v, do = _inputs(71, 1, 6, 2, 8, 10, 4)
    for causal in (False, True):
        dq, dk, dv = mod.attention_bwd_ref(q, k, v, do, causal=causal, scale=0.6)
        kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
        dq2, dk2, dv2 = mod.attention_bwd_ref(q, kr, vr, do, causal=causal, scale=0.6)
        _close(dq, dq2, what="gqa dq")
        _close(dk, dk2.reshape(1, 2, 3, 10, 4).sum(axis=2), what="gqa dk")
        _close(dv, dv2.reshape(1, 2, 3, 10, 4).sum(axis=2), what="gqa dv")


# 8. The scale can move onto Q: (scale a, Q) and (scale 1, aQ) give the same forward, so
#    dQ_a(Q) = a * dQ_1(aQ), while dK and dV agree.
def pin_bwd_scale_moves_to_q(mod):
    q, k, v, do = _inputs(81, 1, 2, 2, 7, 7, 4)
    a = 0.37
    for causal in (False, True):
        dq_a, dk_a, dv_a = mod.attention_bwd_ref(q, k, v, do, causal=causal, scale=a)
        dq_1, dk_1, dv_1 = mod.attention_bwd_ref(a * q, k, v, do, causal=causal, scale=1.0)
        _close(dq_a, a * dq_1, what="scale dq")
        _close(dk_a, dk_1, what="scale dk")
        _close(dv_a, dv_1, what="scale dv")


# 9. Causal: the last key is seen only by the last query row, with weight P[N-1, N-1].
def pin_bwd_causal_last_key(mod):
    q, k, v, do = _inputs(91, 1, 1, 1, 8, 8, 3)
    _, _, dv = mod.attention_bwd_ref(q, k, v, do, causal=True, scale=0.8)
    s = 0.8 * q[0, 0, 7] @ k[0, 0].T
    p_last = np.exp(s[7] - np.log(np.sum(np.exp(s))))
    _close(dv[0, 0, 7], p_last * do[0, 0, 7], what="causal last-key dV")


# 10. Sampled dQ rows agree with the full computation.
def pin_bwd_dq_rows_agree(mod):
    q, k, v, do = _inputs(101, 2, 4, 1, 12, 12, 6)
    for causal in (False, True):
        dq, _, _ = mod.attention_bwd_ref(q, k, v, do, causal=causal, scale=0.3)
        rows = [0, 5, 11]
        _close(mod.dq_rows(q, k, v, do, 1, 3, rows, causal=causal, scale=0.3), dq[1, 3, rows], what="dq rows")


# 11. Sliding windows: finite differences through the windowed forward oracle, and torch float64
#     autograd through SDPA with an explicit boolean band mask (windows that leave no row empty).
def pin_bwd_window(mod):
    q, k, v, do = _inputs(111, 1, 2, 1, 6, 7, 3)
    for left, right in ((1, 0), (0, 2), (2, None)):
        dq, dk, dv = mod.attention_bwd_ref(q, k, v, do, causal=False, scale=0.6, window=(left, right))

        def loss(q_, k_, v_):
            o, _ = fwd_oracle.attention_ref(q_, k_, v_, causal=False, scale=0.6, window=(left, right))
            return float(np.sum(o * do))

        h = 1e-5
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                ap = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                am = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num[idx] = (loss(*ap) - loss(*am)) / (2 * h)
            _close(g, num, tol=1e-7, what=f"window ({left},{right}) finite differences d{name}")
    q, k, v, do = _inputs(112, 1, 4, 2, 20, 20, 8)
    i = np.arange(20)[:, None]
    j = np.arange(20)[None, :]
    band = (j >= i - 5) & (j <= i + 2)
    dq, dk, dv = mod.attention_bwd_ref(q, k, v, do, causal=False, scale=0.35, window=(5, 2))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(band), scale=0.35,
                                                         enable_gqa=True)
    o.backward(torch.tensor(do, dtype=torch.float64))
    _close(dq, tq.grad.numpy(), tol=1e-12, what="window autograd dq")
    _close(dk, tk.grad.numpy(), tol=1e-12, what="window autograd dk")
    _close(dv, tv.grad.numpy(), tol=1e-12, what="window autograd dv")
    # a row whose window holds no key has zero gradients everywhere it could reach
    q, k, v, do = _inputs(113, 1, 1, 1, 8, 5, 3)
    dq, dk, dv = mod.attention_bwd_ref(q, k, v, do, causal=False, scale=0.5, window=(0, 0))
    assert np.all(dq[0, 0, 5:] == 0.0), "rows without keys have dQ = 0"


# 12. Packed variable-length sequences: finite differences through the (separately pinned) packed
#     forward oracle, torch float64 autograd through SDPA over all the packed tokens with a
#     block-diagonal (per-sequence, optionally causal) boolean mask, and zero gradients on the
#     tokens of sequences without queries or without keys.
def pin_bwd_varlen(mod):
    rng = _rng(121)
    cu_q, cu_k = [0, 2, 2, 5, 6], [0, 3, 4, 6, 6]   # sequence 1 has no queries, sequence 3 no keys
    q, k, v = rng.standard_normal((6, 2, 3)), rng.standard_normal((6, 1, 3)), rng.standard_normal((6, 1, 3))
    do = rng.standard_normal((6, 2, 3))
    for causal in (False, True):
        dq, dk, dv = mod.attention_varlen_bwd_ref(q, k, v, do, cu_q, cu_k, causal=causal, scale=0.8)

        def loss(q_, k_, v_):
            o, _ = fwd_oracle.attention_varlen_ref(q_, k_, v_, cu_q, cu_k, causal=causal, scale=0.8)
            return float(np.sum(o * do))

        h = 1e-5
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                ap = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                am = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num[idx] = (loss(*ap) - loss(*am)) / (2 * h)
            _close(g, num, tol=1e-7, what=f"varlen causal={causal} finite differences d{name}")
        assert np.all(dk[3] == 0.0) and np.all(dv[3] == 0.0), "keys of a sequence without queries"
        assert np.all(dq[5] == 0.0), "queries of a sequence without keys"
    # autograd: every sequence has queries and keys; group of 2
    lens_q, lens_k = [5, 1, 9, 4], [7, 3, 9, 1]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lens_q)]), np.concatenate([[0], np.cumsum(lens_k)])
    tq_, tk_ = int(cu_q[-1]), int(cu_k[-1])
    q, k, v = rng.standard_normal((tq_, 4, 8)), rng.standard_normal((tk_, 2, 8)), rng.standard_normal((tk_, 2, 8))
    do = rng.standard_normal((tq_, 4, 8))
    seq_q = np.repeat(np.arange(4), lens_q)
    seq_k = np.repeat(np.arange(4), lens_k)
    pos_q = np.arange(tq_) - cu_q[seq_q]
    pos_k = np.arange(tk_) - cu_k[seq_k]
    for causal in (False, True):
        mask = seq_q[:, None] == seq_k[None, :]
        if causal:
            mask &= pos_k[None, :] <= pos_q[:, None]
        dq, dk, dv = mod.attention_varlen_bwd_ref(q, k, v, do, cu_q, cu_k, causal=causal, scale=0.4)
        tq, tk, tv = (torch.tensor(x.transpose(1, 0, 2)[None], dtype=torch.float64, requires_grad=True)
                      for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=0.4,
                                                             enable_gqa=True)
        o.backward(torch.tensor(do.transpose(1, 0, 2)[None], dtype=torch.float64))
        for name, g, t in (("dq", dq, tq), ("dk", dk, tk), ("dv", dv, tv)):
            _close(g, t.grad.numpy()[0].transpose(1, 0, 2), tol=1e-12, what=f"varlen causal={causal} autograd {name}")


ALL_BWD_PINS = [
    pin_bwd_finite_differences,
    pin_bwd_torch_autograd,
    pin_bwd_dk_rows_sum_to_zero,
    pin_bwd_dv_rows_sum_to_do,
    pin_bwd_single_key,
    pin_bwd_zero_query,
    pin_bwd_gqa_is_repeated_mha,
    pin_bwd_scale_moves_to_q,
    pin_bwd_causal_last_key,
    pin_bwd_dq_rows_agree,
    pin_bwd_window,
    pin_bwd_varlen,
]
