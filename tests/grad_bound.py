"""Elementwise error bound of the HIP attention backward against the exact float64 gradients.

The tolerance of the backward parity tests is derived here from the roundings the kernel performs,
not chosen. For one (batch, query head) against its key/value head the kernel computes, with fp32
arithmetic and 16-bit operands in every matrix product:

    s~_ij   = fp32 sum over d of q_id k_jd (each product of two 16-bit values is exact in fp32)
    P~_ij   = exp2(scale log2(e) s~_ij - log2(e) lse16_i)     lse16 = the forward's stored LSE
    dP~_ij  = fp32 sum over d of dO_id v_jd,   Delta16_i = fp32 sum over d of O16_id dO_id
    dS~_ij  = P~_ij (dP~_ij - Delta16_i)                       O16 = the forward's stored 16-bit O
    dV_j    = rnd( sum_i rnd(P~_ij) dO_i )                      P rounded to the dtype
    dK_j    = rnd( scale sum_i rnd(dS~_ij) Q_i )                dS rounded to the dtype
    dQ_i    = rnd( scale sum_j (hi_ij + lo_ij) K_j )            dS as two dtype terms:
                                                               hi = rnd(dS~), lo = rnd(dS~ - hi)

(the P and dS roundings follow the Ascend notes, section 3: the vector unit forms P and dS, the
matrix unit takes them in the input dtype). Against the exact gradients -- exact P, exact O in
Delta -- each element's error is, to first order in the dtype's unit roundoff u (2^-8 bf16,
2^-11 fp16) and fp32's w = 2^-23 per operation (twice the unit roundoff, which also covers
rounding toward zero inside the matrix units), at most the sum of:

  (1) rounding the rounded factor of each term: u * sum|terms| (P for dV, dS for dK); the two-term
      dS of dQ leaves u^2 * sum|terms|. Near zero the errors are absolute instead: rounding to
      the dtype can land in its subnormal range (spacing 2^-24 in fp16, 2^-133 in bf16), an error
      of eta = half that spacing; and an fp32 intermediate below f = 2^-126 (a probability of a
      score far below the row maximum, the dS it forms) may be flushed to zero by the hardware.
      Per visible term: (eta + f) times the other factor's magnitude, plus f |dP_ij - Delta_i|
      times it for dK and dQ, where a flushed probability drops P (dP - Delta);
  (2) Delta formed from the stored O: d_i = Delta16_i - Delta_i moves dS_ij by -P_ij d_i, giving
      scale sum_i P_ij |d_i| |Q_id| for dK and scale |d_i| sum_j P_ij |K_jd| for dQ;
  (3) the recomputed probabilities: relative error at most e_ij = |lse16_i - lse_i| + scale D w
      sum_d |q_id k_jd| (the fp32 score sum) + 3 w (scale |s_ij| + |lse_i|) (the folded scale,
      the exponent's fused multiply-add, the lse product) + 4 w (exp2), which reaches every term
      of all three gradients through P (and dS = P (...)): e_ij * |term|;
  (4) dP~ and Delta16 in fp32: D w (sum_d |dO_id v_jd| + sum_d |O16_id dO_id|) on (dP - Delta),
      times P_ij and the other factor, for dK and dQ;
  (5) the fp32 accumulation of the n terms of each gradient sum: n w * sum|terms|;
  (6) the final rounding of the gradient to the dtype: u (|exact| + the above), plus eta + f of
      (1) (a tiny gradient can round into the subnormal range, be flushed or round to zero).

Terms of second order (products of two of these relative errors) are neglected; the comparison
uses no empirical factor. A kernel bug (a wrong term, mask, index or scale) makes errors of the
size of the terms themselves, far above this bound.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from oracle.attention_bwd import softmax_rows

W32 = 2.0 ** -23  # fp32 rounding per operation, doubled: covers rounding toward zero in the matrix units
UNIT = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}
SUBNORMAL_HALF = {torch.bfloat16: 2.0 ** -134, torch.float16: 2.0 ** -25}  # eta: half the dtype's subnormal spacing
FP32_FLUSH = 2.0 ** -126  # f: fp32's smallest normal, below which an intermediate may be flushed to zero


def _f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def head_bwd_bound(qh, kh, vh, doh, o16h, lse16h, *, causal: bool, scale: float, dtype,
                   window=None, rows: Optional[Sequence[int]] = None, dq_only: bool = False):
    """Bound of one query head's gradient errors: (bq, bk, bv), bq for the query rows `rows`
    (default all), bk and bv this head's part of its key/value head's bound (None if dq_only).

    qh, kh, vh: the 16-bit inputs (any float array); doh: dO; o16h, lse16h: the forward's stored
    O and LSE of this head (all rows)."""
    q, k, v, do, o16, lse16 = (_f64(t) for t in (qh, kh, vh, doh, o16h, lse16h))
    u, eta, f = UNIT[dtype], SUBNORMAL_HALF[dtype], FP32_FLUSH
    n_q, D = q.shape
    n_kv = k.shape[0]
    r = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    p = softmax_rows(q, k, r, causal, scale, window)                       # exact P of these rows
    vis = (p > 0).astype(np.float64)
    delta = np.sum((p @ v) * do[r], axis=1)                               # with the exact O
    delta16 = np.sum(o16[r] * do[r], axis=1)                              # with the stored O
    d = delta16 - delta                                                   # (2)
    lse = _row_lse(q, k, r, causal, scale, window)
    lse_err = np.where(np.isfinite(lse), np.abs(lse16[r] - lse), 0.0)
    lse_mag = np.where(np.isfinite(lse), np.abs(lse), 0.0)
    # (3) relative error of each recomputed probability
    e = (lse_err[:, None] + scale * D * W32 * (np.abs(q[r]) @ np.abs(k).T)
         + 3 * W32 * (scale * np.abs(q[r] @ k.T) + lse_mag[:, None]) + 4 * W32) * vis
    dp = do[r] @ v.T
    ds16_abs = np.abs(p * (dp - delta16[:, None]))                        # |dS| / scale as the kernel forms it
    g = D * W32 * (np.abs(do[r]) @ np.abs(v).T + np.sum(np.abs(o16[r] * do[r]), axis=1)[:, None])   # (4)
    k_abs, q_abs, do_abs = np.abs(k), np.abs(q[r]), np.abs(do[r])
    near0 = vis * ((eta + f) + f * np.abs(dp - delta16[:, None]))        # (1) near zero, dK and dQ
    # dQ_i = scale sum_j dS_ij K_j, two terms per key
    bq = scale * ((u * u + 2 * n_kv * W32) * (ds16_abs @ k_abs)          # (1), (5)
                  + near0 @ k_abs                                          # (1) near zero
                  + np.abs(d)[:, None] * (p @ k_abs)                       # (2)
                  + (ds16_abs * e) @ k_abs                                 # (3)
                  + (p * g) @ k_abs)                                       # (4)
    bq = _stored(bq, scale * ((p * (dp - delta[:, None])) @ k), u, eta + f)  # (6)
    if dq_only:
        return bq, None, None
    # dK_j = scale sum_i dS_ij Q_i; the group's heads and the rows of all tiles are n_q terms here
    bk = scale * ((u + n_q * W32) * (ds16_abs.T @ q_abs)
                  + near0.T @ q_abs
                  + (p * np.abs(d)[:, None]).T @ q_abs
                  + (ds16_abs * e).T @ q_abs
                  + (p * g).T @ q_abs)
    # dV_j = sum_i P_ij dO_i
    bv = (u + n_q * W32) * (p.T @ do_abs) + (eta + f) * (vis.T @ do_abs) + (p * e).T @ do_abs
    # (6) is applied once to the whole sum over query heads and rows: see finish_kv
    return bq, bk, bv


def _stored(b_rest, exact, u, floor):
    """(6): the stored value is the computed one rounded, which is within b_rest of the exact one:
    |rnd(x) - exact| <= b_rest + u (|exact| + b_rest) + floor (eta + f: the absolute error near zero)."""
    return b_rest * (1 + u) + u * np.abs(exact) + floor


def finish_kv(bk_rest, bv_rest, dk_exact, dv_exact, dtype):
    """Add (6) to the summed dK and dV bounds of a key/value head (its query heads' parts added)."""
    u, floor = UNIT[dtype], SUBNORMAL_HALF[dtype] + FP32_FLUSH
    return _stored(bk_rest, dk_exact, u, floor), _stored(bv_rest, dv_exact, u, floor)


def _row_lse(q, k, r, causal, scale, window):
    """Exact natural-log logsumexp of the visible scaled scores of rows r (-inf for an empty row)."""
    s = scale * (q[r] @ k.T)
    key_pos = np.arange(k.shape[0])
    if causal:
        s = np.where(key_pos[None, :] <= r[:, None], s, -np.inf)
    if window is not None:
        left, right = window
        if left is not None:
            s = np.where(key_pos[None, :] >= r[:, None] - left, s, -np.inf)
        if right is not None:
            s = np.where(key_pos[None, :] <= r[:, None] + right, s, -np.inf)
    m = np.max(s, axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        return np.where(np.isfinite(m), m_safe + np.log(np.sum(np.exp(s - m_safe[:, None]), axis=1)), -np.inf)


def attention_bwd_bound(q, k, v, do, o16, lse16, dk_exact, dv_exact, *, causal: bool, scale: float, dtype,
                        window=None):
    """Bounds (bq, bk, bv) shaped like q, k, v for BNSD tensors; grouped query heads add their
    terms into their key/value head's bound, as they add into its gradient. dk_exact, dv_exact:
    the oracle's gradients (for the final rounding of the summed dK, dV)."""
    q, k, v, do, o16, lse16 = (_f64(t) for t in (q, k, v, do, o16, lse16))
    B, Hq = q.shape[0], q.shape[1]
    group = Hq // k.shape[1]
    bq = np.empty_like(q)
    bk = np.zeros_like(k)
    bv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kvh = h // group
            gq, gk, gv = head_bwd_bound(q[b, h], k[b, kvh], v[b, kvh], do[b, h], o16[b, h], lse16[b, h],
                                        causal=causal, scale=scale, dtype=dtype, window=window)
            bq[b, h] = gq
            bk[b, kvh] += gk
            bv[b, kvh] += gv
    bk, bv = finish_kv(bk, bv, _f64(dk_exact), _f64(dv_exact), dtype)
    return bq, bk, bv


def varlen_bwd_bound(q, k, v, do, o16, lse16, cu_q, cu_k, dk_exact, dv_exact, *, causal: bool, scale: float,
                     dtype):
    """Bounds for packed sequences (token-major (total, H, D) tensors, lse16 (Hq, total_q)): each
    sequence is its own problem; tokens of a sequence without queries or keys get zero bounds
    (their gradients are exactly zero)."""
    q, k, v, do, o16, lse16, dk_exact, dv_exact = (_f64(t) for t in (q, k, v, do, o16, lse16, dk_exact, dv_exact))
    bq, bk, bv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    cq, ck = [int(x) for x in cu_q], [int(x) for x in cu_k]

    def bnsd(x, a, c):
        return x[a:c].transpose(1, 0, 2)[None]

    for s in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[s], cq[s + 1], ck[s], ck[s + 1]
        if q1 <= q0 or k1 <= k0:
            continue
        gq, gk, gv = attention_bwd_bound(bnsd(q, q0, q1), bnsd(k, k0, k1), bnsd(v, k0, k1), bnsd(do, q0, q1),
                                         bnsd(o16, q0, q1), lse16[:, q0:q1][None], bnsd(dk_exact, k0, k1),
                                         bnsd(dv_exact, k0, k1), causal=causal, scale=scale, dtype=dtype)
        bq[q0:q1], bk[k0:k1], bv[k0:k1] = gq[0].transpose(1, 0, 2), gk[0].transpose(1, 0, 2), gv[0].transpose(1, 0, 2)
    return bq, bk, bv


def bound_ratio(got, exact, bound) -> float:
    """Worst |got - exact| / bound over all elements (elements whose bound is 0 must match exactly)."""
    got, exact, bound = _f64(got), _f64(exact), _f64(bound)
    err = np.abs(got - exact)
    if np.any((bound <= 0) & (err > 0)):
        return float("inf")
    return float(np.max(np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), 0.0))) if err.size else 0.0
