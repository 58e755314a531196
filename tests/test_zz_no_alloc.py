"""fa_bwd_noalloc (Delta in the library's fixed device array, nothing allocated) against fa_bwd (Delta
in a caller workspace), both called through the C ABI on the same inputs: the gradients must agree to
the bit, since the same kernels run on the same data. Two calls in a row, the second smaller, so the
second runs on an array that still holds the first call's Delta."""
import ctypes

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
_DT = {torch.float16: 0, torch.bfloat16: 1}


def _st(t):
    return (ctypes.c_int64 * 4)(*t.stride())


def _call(lib, name, q, k, v, o, lse, do, dq, dk, dv, delta, causal, stream):
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    ptrs = [t.data_ptr() for t in (q, k, v, o, lse, do, dq, dk, dv)]
    if delta is not None:
        ptrs.append(delta.data_ptr())
    st = [_st(t) for t in (q, k, v, o, do, dq, dk, dv)]
    return getattr(lib, name)(*ptrs, B, Hq, Hkv, Nq, Nkv, D, *st, ctypes.c_float(D ** -0.5), int(causal),
                              _DT[q.dtype], ctypes.c_void_p(stream.cuda_stream))


CASES = [  # the second is smaller than the first
    (1, 32, 8, 4096, 4096, 128, torch.bfloat16, True),
    (2, 4, 2, 150, 333, 64, torch.float16, False),
]


def test_noalloc_backward_matches_fa_bwd():
    import scaled_dot_product_fa2_amd as fa
    from scaled_dot_product_fa2_amd import _binding
    lib = _binding.load_library()
    stream = torch.cuda.current_stream(DEV)
    for i, (B, Hq, Hkv, Nq, Nkv, D, dtype, causal) in enumerate(CASES):
        print(f"[case] no-alloc backward call {i}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} D={D} {dtype} "
              f"causal={causal}", flush=True)
        assert B * Hq * Nq <= _binding.FA_NOALLOC_MAX_ROWS
        q, k, v = (t.to(DEV) for t in workloads.make_random(B, Hq, Hkv, Nq, Nkv, D, dtype, seed=900 + i))
        g = torch.Generator().manual_seed(950 + i)
        do = torch.randn(B, Hq, Nq, D, generator=g).to(dtype).to(DEV)
        o, lse = fa.fa_fwd(q, k, v, causal=causal)
        ref = [torch.full_like(t, float("nan")) for t in (q, k, v)]
        delta = torch.empty(B, Hq, Nq, dtype=torch.float32, device=DEV)
        assert _call(lib, "fa_bwd", q, k, v, o, lse, do, *ref, delta, causal, stream) == 0
        got = [torch.full_like(t, float("nan")) for t in (q, k, v)]
        assert _call(lib, "fa_bwd_noalloc", q, k, v, o, lse, do, *got, None, causal, stream) == 0
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.isfinite(b).all(), f"{name}: fa_bwd left non-finite values"
            assert torch.equal(a, b), f"{name}: fa_bwd_noalloc differs from fa_bwd (max |diff| " \
                                      f"{(a.float() - b.float()).abs().max().item():.3e})"
        print(f"[result] no-alloc backward call {i}: dq, dk, dv bitwise equal to fa_bwd", flush=True)


def test_noalloc_rejects_delta_past_its_array():
    """A shape whose Delta exceeds the fixed array is refused with FA_ERR_SCRATCH, nothing written."""
    from scaled_dot_product_fa2_amd import _binding
    lib = _binding.load_library()
    B, Hq, Hkv, D = 1, 2, 1, 16
    Nq = _binding.FA_NOALLOC_MAX_ROWS // 2 + 1
    q = torch.zeros(B, Hq, Nq, D, dtype=torch.float16, device=DEV)
    k = torch.zeros(B, Hkv, 64, D, dtype=torch.float16, device=DEV)
    lse = torch.zeros(B, Hq, Nq, dtype=torch.float32, device=DEV)
    dq = torch.full_like(q, float("nan"))
    dk, dv = torch.full_like(k, float("nan")), torch.full_like(k, float("nan"))
    rc = _call(lib, "fa_bwd_noalloc", q, k, k, q, lse, q, dq, dk, dv, None, False, torch.cuda.current_stream(DEV))
    assert rc == -9, rc
    torch.cuda.synchronize()
    assert torch.isnan(dq).all() and torch.isnan(dk).all()
