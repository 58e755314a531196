"""GPU parity of the packed variable-length forward (fa_fwd_varlen) against the float64 oracle:
every output element, same tolerances as the dense forward. Sequences of zero queries or zero keys,
lengths off every tile boundary, GQA and both masks; one packed sequence must reproduce the dense
entry point bitwise."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.parity_util import O_TOL, LSE_ATOL, f32_scale, o_ratio, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import scaled_dot_product_fa2_amd as fa
    return fa


def _packed(lens_q, lens_k, Hq, Hkv, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    tq, tk = sum(lens_q), sum(lens_k)
    q = torch.randn(tq, Hq, D, generator=g).to(dtype)
    k = torch.randn(tk, Hkv, D, generator=g).to(dtype)
    v = torch.randn(tk, Hkv, D, generator=g).to(dtype)
    cq = torch.tensor(np.concatenate([[0], np.cumsum(lens_q)]), dtype=torch.int32)
    ck = torch.tensor(np.concatenate([[0], np.cumsum(lens_k)]), dtype=torch.int32)
    return q, k, v, cq, ck


def _check(lens_q, lens_k, Hq, Hkv, D, dtype, causal, seed):
    print(f"[case] varlen q{lens_q} k{lens_k} Hq{Hq} Hkv{Hkv} D{D} {dtype} causal={causal}", flush=True)
    fa = _fa()
    q, k, v, cq, ck = _packed(lens_q, lens_k, Hq, Hkv, D, dtype, seed)
    o, lse = fa.fa_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV), ck.to(DEV), max(lens_q), max(lens_k),
                              causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen_ref(to_f64(q), to_f64(k), to_f64(v), cq.numpy(), ck.numpy(),
                                               causal=causal, scale=f32_scale(1.0 / np.sqrt(D)))
    og, lg = to_f64(o), to_f64(lse)
    assert np.all(np.isfinite(og)), "non-finite O"
    r = o_ratio(og, o_ref, dtype)
    assert r <= 1.0, f"O error ratio {r:.3f} ({O_TOL[dtype]})"
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lg), empty), "LSE = -inf exactly on the rows of key-less sequences"
    if (~empty).any():
        assert np.max(np.abs(lg[~empty] - l_ref[~empty])) <= LSE_ATOL
    return r


CASES = [
    ([128, 1, 300, 77, 0, 64], [128, 1, 300, 77, 5, 64]),
    ([33, 200, 129], [500, 17, 129]),
    ([5, 0, 70], [0, 9, 200]),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_varlen_mixed_lengths(case, causal):
    lens_q, lens_k = CASES[case]
    _check(lens_q, lens_k, 4, 2, 128, torch.bfloat16, causal, 1000 + case)


@pytest.mark.parametrize("D", [16, 32, 64, 256])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_varlen_head_dims(D, dtype):
    _check([90, 257, 3], [90, 257, 40], 2, 1, D, dtype, True, 1100 + D)


def test_varlen_one_sequence_matches_dense():
    """A single packed sequence reproduces fa_fwd on the same data bitwise."""
    fa = _fa()
    q, k, v, cq, ck = _packed([777], [777], 8, 2, 128, torch.bfloat16, 1200)
    for causal in (False, True):
        o, lse = fa.fa_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV), ck.to(DEV), 777, 777, causal=causal)
        qd, kd, vd = (t.to(DEV).permute(1, 0, 2)[None] for t in (q, k, v))
        od, ld = fa.fa_fwd(qd, kd, vd, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o, od[0].permute(1, 0, 2)), f"O causal={causal}"
        assert torch.equal(lse, ld[0]), f"LSE causal={causal}"


def test_varlen_many_sequences():
    """64 sequences of 1..400 tokens, GQA 4, causal."""
    rng = np.random.default_rng(1300)
    lens = [int(x) for x in rng.integers(1, 400, size=64)]
    _check(lens, lens, 8, 2, 64, torch.float16, True, 1301)
