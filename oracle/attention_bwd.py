"""Float64 CPU oracle for the scaled-dot-product attention backward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test suite and the benchmark's CPU-baseline leg
use it. It shares no code with the HIP library.

Given the upstream gradient dO of the forward output O, it returns the
gradients dQ, dK, dV of the loss sum(dO * O) with respect to Q, K and V,
written out in float64 exactly as the backward is stated in the Ascend notes
("FlashAttention on Ascend: Triton-Ascend CV pipeline", section 2):

* P is the forward's softmax of the scaled, masked scores, recomputed here
  from Q and K (the forward definition: scores scale * <q_i, k_j>, top-left
  causal key set j <= i, row-wise softmax);
* Delta_i = sum_d O_id * dO_id, with O = P V the exact forward output;
* dP = dO V^T;
* dS = scale * P * (dP - Delta), so hidden keys (P = 0) get no gradient;
* dQ = dS K, dK = dS^T Q, dV = P^T dO.

Readings where the pages leave a point open: the logsumexp the forward also
returns receives no gradient (only O does); with grouped-query heads the
query heads that read one key/value head all contribute to its dK and dV,
which are the sums of their per-head terms (the chain rule through the shared
tensor); Delta uses the exact O, not a rounded one. No tiling, recomputation
order or 16-bit rounding of the kernel is emulated.

With a sliding window (row i sees keys i - left .. i + right, as in the forward
oracle) P is the softmax over the window; a row whose window holds no key has
P = 0, so its dQ row is zero and it adds nothing to dK or dV.

Packed variable-length sequences (the CSR layout of the forward oracle's
attention_varlen_ref) are independent attention problems, so each sequence's
gradients are the dense backward of that sequence alone; a sequence with no
query rows or no keys has zero gradients on its tokens.

Query rows are processed in chunks purely to bound memory; the per-row terms
are independent and dK, dV are sums over rows.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = ["attention_bwd_ref", "head_bwd_ref", "dq_rows", "attention_varlen_bwd_ref", "softmax_rows"]


def _f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype != np.float64:
        a = a.astype(np.float64)
    return a


def softmax_rows(qh, kh, r, causal, scale, window=None):
    """P for query rows r of one head: softmax of the scaled scores over the visible keys (the
    forward definition: scores scale * <q_i, k_j>, top-left causal key set, optional window)."""
    s = scale * (qh[r] @ kh.T)
    key_pos = np.arange(kh.shape[0])
    if causal:
        s = np.where(key_pos[None, :] <= r[:, None], s, -np.inf)  # top-left causal key set
    if window is not None:
        left, right = window
        if left is not None:
            s = np.where(key_pos[None, :] >= r[:, None] - left, s, -np.inf)
        if right is not None:
            s = np.where(key_pos[None, :] <= r[:, None] + right, s, -np.inf)
    empty = np.all(s == -np.inf, axis=1)                # a window can leave a row without keys
    s[empty] = 0.0
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    e[empty] = 0.0
    z = np.sum(e, axis=1, keepdims=True)
    z[empty] = 1.0
    return e / z


def head_bwd_ref(qh, kh, vh, doh, *, causal: bool, scale: float,
                 row_chunk: int = 512, window=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of one query head against the key/value head it reads.

    qh: (Nq, D), kh: (Nkv, D), vh: (Nkv, Dv), doh: (Nq, Dv).
    Returns dq (Nq, D), dk (Nkv, D), dv (Nkv, Dv), float64; dk and dv hold this head's terms.
    """
    qh, kh, vh, doh = _f64(qh), _f64(kh), _f64(vh), _f64(doh)
    dq = np.empty_like(qh)
    dk = np.zeros_like(kh)
    dv = np.zeros_like(vh)
    rows = np.arange(qh.shape[0])
    for start in range(0, rows.shape[0], row_chunk):
        r = rows[start:start + row_chunk]
        p = softmax_rows(qh, kh, r, causal, scale, window)  # recomputed probabilities
        o = p @ vh                                       # exact forward output of these rows
        delta = np.sum(o * doh[r], axis=1)               # Delta = rowsum(O * dO)
        dp = doh[r] @ vh.T                               # dP = dO V^T
        ds = scale * p * (dp - delta[:, None])           # dS = scale * P * (dP - Delta)
        dq[r] = ds @ kh                                  # dQ = dS K
        dk += ds.T @ qh[r]                               # dK = dS^T Q
        dv += p.T @ doh[r]                               # dV = P^T dO
    return dq, dk, dv


def attention_bwd_ref(q, k, v, do, *, causal: bool, scale: Optional[float] = None,
                      row_chunk: int = 512, window=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Full attention backward in float64.

    q: (B, Hq, Nq, D); k: (B, Hkv, Nkv, D); v: (B, Hkv, Nkv, Dv); do: (B, Hq, Nq, Dv).
    ``scale`` defaults to 1/sqrt(D). Returns dq, dk, dv shaped like q, k, v (float64).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    if Nkv < 1:
        raise ValueError("softmax over an empty key set is undefined")
    if do.shape != (B, Hq, Nq, v.shape[3]):
        raise ValueError("do must be shaped like the forward output")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    group = Hq // Hkv
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kvh = h // group
            dq[b, h], dkh, dvh = head_bwd_ref(q[b, h], k[b, kvh], v[b, kvh], do[b, h], causal=causal,
                                              scale=scale, row_chunk=row_chunk, window=window)
            dk[b, kvh] += dkh   # every query head of the group adds its terms
            dv[b, kvh] += dvh
    return dq, dk, dv


def dq_rows(q, k, v, do, b: int, h: int, rows: Sequence[int], *, causal: bool,
            scale: Optional[float] = None) -> np.ndarray:
    """dQ of selected query rows of (batch b, query head h): each row needs only its own
    scores, so large shapes can be checked on a sample."""
    Hq, D = q.shape[1], q.shape[3]
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kvh = h // (Hq // Hkv)
    qh, kh, vh = _f64(q[b, h]), _f64(k[b, kvh]), _f64(v[b, kvh])
    r = np.asarray(rows, dtype=np.int64)
    p = softmax_rows(qh, kh, r, causal, scale)
    doh = _f64(do[b, h])[r]
    delta = np.sum((p @ vh) * doh, axis=1)
    ds = scale * p * (doh @ vh.T - delta[:, None])
    return ds @ kh


def attention_varlen_bwd_ref(q, k, v, do, cu_seqlens_q, cu_seqlens_k, *, causal: bool,
                             scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Backward over packed variable-length sequences, in float64.

    q: (total_q, Hq, D), k: (total_k, Hkv, D), v: (total_k, Hkv, Dv), do: (total_q, Hq, Dv), token-major;
    sequence b owns query tokens cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 and key tokens
    cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1, positions counted from its own start. Returns dq, dk, dv
    shaped like q, k, v.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    if len(cq) != len(ck) or cq[0] != 0 or ck[0] != 0 or cq[-1] != q.shape[0] or ck[-1] != k.shape[0]:
        raise ValueError("cu_seqlens must start at 0 and end at the token counts, one entry per sequence + 1")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[2])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 <= q0 or k1 <= k0:
            continue                      # nothing attends, nothing is attended: zero gradients
        gq, gk, gv = attention_bwd_ref(q[q0:q1].transpose(1, 0, 2)[None], k[k0:k1].transpose(1, 0, 2)[None],
                                       v[k0:k1].transpose(1, 0, 2)[None], do[q0:q1].transpose(1, 0, 2)[None],
                                       causal=causal, scale=scale)
        dq[q0:q1] = gq[0].transpose(1, 0, 2)
        dk[k0:k1] = gk[0].transpose(1, 0, 2)
        dv[k0:k1] = gv[0].transpose(1, 0, 2)
    return dq, dk, dv
