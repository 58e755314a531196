"""Long sequences: 128K and 64K tokens per head through the forward and the backward.

At these lengths every index, offset and item count is far past the named workloads (a head's K
and V take 32 MiB, a causal head has 1024 query tiles and the longest sees 2048 key tiles), so the
test looks for overflow and accumulation trouble: O and LSE on sampled rows against the float64
oracle, dQ on sampled rows against the derived error bound, dK and dV through the sum identities
(every row of dS sums to zero; the softmax weights of a row sum to one).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import grad_bound as gb
from tests.parity_util import f32_scale, sampled_check, to_f64
from tests.test_bwd_parity import _sum_identities

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [(1, 4, 1, 131072, 128, torch.bfloat16, True), (1, 2, 2, 65536, 64, torch.float16, False)]


@pytest.mark.parametrize("B,Hq,Hkv,N,D,dtype,causal", CASES,
                         ids=[f"b{c[0]}h{c[1]}kv{c[2]}n{c[3]}d{c[4]}-{'c' if c[6] else 'n'}" for c in CASES])
def test_long_sequence_forward_and_backward(B, Hq, Hkv, N, D, dtype, causal):
    import scaled_dot_product_fa2_amd as fa
    print(f"[case] long sequence B={B} Hq={Hq} Hkv={Hkv} N={N} D={D} {dtype} causal={causal}", flush=True)
    q, k, v = workloads.make_random(B, Hq, Hkv, N, N, D, dtype, seed=N // 1024 + D)
    do = torch.randn(B, Hq, N, D, generator=torch.Generator().manual_seed(N + D)).to(dtype)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, lse, dod, causal=causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng(N + 7)
    rows = sorted({0, 1, 127, 128, N // 2, N - 129, N - 128, N - 1, *map(int, rng.integers(0, N, 6))})
    heads = [(0, h) for h in range(Hq)]
    r, e = sampled_check(q, k, v, o, lse, causal, 1.0 / np.sqrt(D), heads, rows, what=f"n{N}")
    print(f"[result] n{N} forward: sampled rows, worst O error ratio {r:.3f}, worst LSE error {e:.2e}", flush=True)
    sc = f32_scale(1.0 / np.sqrt(D))
    G = Hq // Hkv
    q64, k64, v64, do64, o64, lse64 = (to_f64(t) for t in (q, k, v, do, o, lse))
    for h in range(Hq):
        ref = oracle.dq_rows(q64, k64, v64, do64, 0, h, rows, causal=causal, scale=sc)
        bq, _, _ = gb.head_bwd_bound(q64[0, h], k64[0, h // G], v64[0, h // G], do64[0, h], o64[0, h], lse64[0, h],
                                     causal=causal, scale=sc, dtype=dtype, rows=rows, dq_only=True)
        ratio = gb.bound_ratio(to_f64(dq[0, h])[rows], ref, bq)
        print(f"[result] n{N} h={h}: sampled dq rows, error / bound {ratio:.4f}", flush=True)
        assert ratio <= 1.0, f"h={h}: dq ratio {ratio:.3f}"
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()
    _sum_identities(dk, dv, dod, G, dtype)
