"""Float64 CPU oracle for the scaled-dot-product attention forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library.

What it computes is the plain definition of attention, written out in float64
with numpy; no tiling, online softmax or other reordering of the method is
emulated here:

* scores  s_ij = scale * <q_i, k_j>, for the keys j the row may see
  ("Write Triton Attention Kernel", Required reasoning process, step 5b;
  "FlashAttention on Ascend: Triton-Ascend CV pipeline" notes, section 1, the
  three-line forward definition);
* the causal key set is j <= i with zero-based positions, i.e. the mask is
  aligned at the top-left corner ("Write Triton Attention Kernel", step 5c);
  without the mask every key is visible;
* probabilities are the softmax of each score row, taken after subtracting the
  row maximum (safe softmax, two passes over the full row);
* o_i = sum_j p_ij v_j ("Build Triton-Ascend Fused Attention", Goal);
* lse_i = m_i + ln l_i = ln sum_j exp(s_ij), the natural-log logsumexp of the
  scaled, masked scores, indexed by (batch, query head, query position)
  ("Write Triton Attention Kernel", step 8 and Correctness requirements);
* grouped-query heads: query head h reads key/value head h // (Hq / Hkv)
  ("Write Triton Attention Kernel", step 1 and Kernel design rules).

A sliding window ("Write Triton Attention Kernel", Inputs item 3, which lists
sliding-window masks beside the causal one) restricts row i to keys
i - left <= j <= i + right (either side may be unbounded); the causal mask is
the window (unbounded, 0). A row whose visible key set is empty (possible only
with a window) has no softmax; the oracle returns o = 0 and lse = -inf for it.

Readings where the pages leave a point open: the causal mask is top-left even
when Nq != Nkv; a row whose key set is empty cannot occur under that reading
(key 0 is always visible), and empty key sets (Nkv = 0) are rejected; the
oracle does not round P to 16 bits before the P.V product, because it is the
exact definition and the stated tolerances absorb that rounding.

Query rows are processed in chunks purely to bound memory; every row is
computed independently, so chunking changes no arithmetic.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ProcessPoolExecutor
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = ["attention_ref", "attention_rows", "attention_ref_pool", "head_ref", "attention_varlen_ref"]


def _f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype != np.float64:
        a = a.astype(np.float64)
    return a


def _check_shapes(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> Tuple[int, int, int, int, int, int, int]:
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D (batch, heads, sequence, head_dim)")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nkv, Dk = k.shape
    if Bk != B or v.shape[0] != B:
        raise ValueError("batch sizes differ")
    if Dk != D:
        raise ValueError("q and k head_dim differ")
    if v.shape[1] != Hkv or v.shape[2] != Nkv:
        raise ValueError("k and v disagree on heads or sequence length")
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    if Nkv < 1:
        raise ValueError("softmax over an empty key set is undefined")
    return B, Hq, Hkv, Nq, Nkv, D, v.shape[3]


def head_ref(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, rows: np.ndarray, *, causal: bool,
             scale: float, row_chunk: int = 512,
             window: Optional[Tuple[Optional[int], Optional[int]]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of the selected query rows of one head against one key/value head.

    qh: (Nq, D), kh: (Nkv, D), vh: (Nkv, Dv), rows: integer query positions.
    window: optional (left, right); row i then sees keys i - left .. i + right (None = unbounded).
    Returns (o, lse) with shapes (len(rows), Dv) and (len(rows),), float64.
    """
    qh, kh, vh = _f64(qh), _f64(kh), _f64(vh)
    rows = np.asarray(rows, dtype=np.int64)
    n_kv = kh.shape[0]
    key_pos = np.arange(n_kv)
    o = np.empty((rows.shape[0], vh.shape[1]), dtype=np.float64)
    lse = np.empty((rows.shape[0],), dtype=np.float64)
    for start in range(0, rows.shape[0], row_chunk):
        r = rows[start:start + row_chunk]
        s = scale * (qh[r] @ kh.T)                      # scaled scores, (rows, Nkv)
        if causal:
            visible = key_pos[None, :] <= r[:, None]     # top-left causal: key j visible to row i iff j <= i
            s = np.where(visible, s, -np.inf)
        if window is not None:
            left, right = window
            if left is not None:
                s = np.where(key_pos[None, :] >= r[:, None] - left, s, -np.inf)   # j >= i - left
            if right is not None:
                s = np.where(key_pos[None, :] <= r[:, None] + right, s, -np.inf)  # j <= i + right
        empty = np.all(s == -np.inf, axis=1)             # only a window can leave a row without keys
        s[empty] = 0.0
        m = np.max(s, axis=1, keepdims=True)             # row maximum over the visible keys
        e = np.exp(s - m)                                # masked entries give exp(-inf) = 0
        e[empty] = 0.0
        l = np.sum(e, axis=1, keepdims=True)             # softmax denominator
        l[empty] = 1.0
        o[start:start + r.shape[0]] = (e / l) @ vh       # softmax-weighted sum of value rows
        lse[start:start + r.shape[0]] = np.where(empty, -np.inf, m[:, 0] + np.log(l[:, 0]))
    return o, lse


def attention_ref(q, k, v, *, causal: bool, scale: Optional[float] = None,
                  row_chunk: int = 512, window=None) -> Tuple[np.ndarray, np.ndarray]:
    """Full attention forward in float64.

    q: (B, Hq, Nq, D); k: (B, Hkv, Nkv, D); v: (B, Hkv, Nkv, Dv); any float dtype,
    any strides. ``scale`` defaults to 1/sqrt(D); ``window`` is an optional (left, right)
    sliding window (None on a side = unbounded). Returns o (B, Hq, Nq, Dv) and
    lse (B, Hq, Nq), both float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, Nq, Nkv, D, Dv = _check_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    group = Hq // Hkv
    o = np.empty((B, Hq, Nq, Dv), dtype=np.float64)
    lse = np.empty((B, Hq, Nq), dtype=np.float64)
    rows = np.arange(Nq)
    for b in range(B):
        for h in range(Hq):
            kvh = h // group
            o[b, h], lse[b, h] = head_ref(q[b, h], k[b, kvh], v[b, kvh], rows, causal=causal,
                                          scale=scale, row_chunk=row_chunk, window=window)
    return o, lse


def attention_rows(q, k, v, b: int, h: int, rows: Sequence[int], *, causal: bool,
                   scale: Optional[float] = None, window=None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention for selected query rows of (batch b, query head h) only.

    Used to check sampled outputs of shapes too large to compute in full.
    Only the one key/value head that h reads is converted to float64.
    """
    Hq, D = q.shape[1], q.shape[3]
    Hkv = k.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kvh = h // (Hq // Hkv)
    return head_ref(_f64(q[b, h]), _f64(k[b, kvh]), _f64(v[b, kvh]), np.asarray(rows), causal=causal,
                    scale=scale, window=window)


# ---------------------------------------------------------------------------------------------
# Process-pool driver: the same per-head computation, one (batch, head) unit per task.
# Each worker pins its BLAS library to one thread so the pool uses one core per worker.

_POOL_ARGS = None


def _pool_init(q, k, v, causal, scale):
    global _POOL_ARGS
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass
    _POOL_ARGS = (q, k, v, causal, scale)


def _pool_unit(unit):
    q, k, v, causal, scale = _POOL_ARGS
    b, h = unit
    group = q.shape[1] // k.shape[1]
    kvh = h // group
    return unit, head_ref(q[b, h], k[b, kvh], v[b, kvh], np.arange(q.shape[2]), causal=causal, scale=scale)


def attention_ref_pool(q, k, v, *, causal: bool, scale: Optional[float] = None,
                       units: Optional[Iterable[Tuple[int, int]]] = None,
                       workers: Optional[int] = None):
    """Run ``head_ref`` for each (b, h) unit in a process pool.

    Returns ({(b, h): (o, lse)}, workers_used). ``units`` defaults to every
    (b, h) pair. Inputs are float arrays as for ``attention_ref``.
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    _check_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[3])
    if units is None:
        units = [(b, h) for b in range(q.shape[0]) for h in range(q.shape[1])]
    units = list(units)
    if workers is None:
        workers = len(os.sched_getaffinity(0))
    workers = max(1, min(workers, len(units)))
    out = {}
    with ProcessPoolExecutor(max_workers=workers, initializer=_pool_init,
                             initargs=(q, k, v, causal, scale)) as ex:
        for unit, res in ex.map(_pool_unit, units):
            out[unit] = res
    return out, workers


def attention_varlen_ref(q, k, v, cu_seqlens_q, cu_seqlens_k, *, causal: bool,
                         scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention over packed variable-length sequences, in float64.

    The CSR layout named in "Write Triton Attention Kernel" (Inputs, item 6; Correctness
    requirements: the key loop of a batch element ends at that element's own length):
    q: (total_q, Hq, D), k: (total_k, Hkv, D), v: (total_k, Hkv, Dv); sequence b owns query tokens
    cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 and key tokens cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1,
    positions counted from the start of its own sequence (so the causal mask is top-left per
    sequence). Returns o (total_q, Hq, Dv) and lse (Hq, total_q). A sequence with no keys gives its
    rows o = 0 and lse = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    if len(cq) != len(ck) or cq[0] != 0 or ck[0] != 0 or cq[-1] != q.shape[0] or ck[-1] != k.shape[0]:
        raise ValueError("cu_seqlens must start at 0 and end at the token counts, one entry per sequence + 1")
    Hq, Dv = q.shape[1], v.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[2])
    o = np.zeros((q.shape[0], Hq, Dv), dtype=np.float64)
    lse = np.full((Hq, q.shape[0]), -np.inf, dtype=np.float64)
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 <= q0 or k1 <= k0:
            continue                      # no rows, or rows without keys (o = 0, lse = -inf)
        ob, lb = attention_ref(q[q0:q1].transpose(1, 0, 2)[None], k[k0:k1].transpose(1, 0, 2)[None],
                               v[k0:k1].transpose(1, 0, 2)[None], causal=causal, scale=scale)
        o[q0:q1] = ob[0].transpose(1, 0, 2)
        lse[:, q0:q1] = lb[0]
    return o, lse
