"""The binding rejects tensors that are not on q's GPU before anything is enqueued.

The C ABI takes raw pointers and cannot tell a host pointer from a device one, so a host-side
output or workspace (lse, delta, out, dq, dk, dv, cu_seqlens) must be caught in the binding.
Each case pre-fills the GPU outputs that are passed with NaN and checks they are untouched.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import scaled_dot_product_fa2_amd as fa
    return fa


def _inputs(dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(3)
    q = torch.randn(1, 2, 64, 64, generator=g).to(dtype).to(DEV)
    k = torch.randn(1, 2, 64, 64, generator=g).to(dtype).to(DEV)
    v = torch.randn(1, 2, 64, 64, generator=g).to(dtype).to(DEV)
    return q, k, v


def test_fwd_host_lse_or_out_rejected():
    fa = _fa()
    q, k, v = _inputs()
    out = torch.full_like(q, float("nan"))
    with pytest.raises(ValueError, match="lse"):
        fa.fa_fwd(q, k, v, out=out, lse=torch.empty(1, 2, 64, dtype=torch.float32))
    lse = torch.full((1, 2, 64), float("nan"), device=DEV)
    with pytest.raises(ValueError, match="out"):
        fa.fa_fwd(q, k, v, out=torch.empty(q.shape, dtype=q.dtype), lse=lse)
    with pytest.raises(ValueError, match="lse"):
        fa.fa_fwd_window(q, k, v, window_left=8, window_right=0, out=out,
                         lse=torch.empty(1, 2, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="k"):
        fa.fa_fwd(q, k.cpu(), v, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(lse).all(), "a rejected call wrote its outputs"


def test_bwd_host_delta_or_grads_rejected():
    fa = _fa()
    q, k, v = _inputs()
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    do = torch.randn_like(o)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    with pytest.raises(ValueError, match="delta"):
        fa.fa_bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv,
                  delta=torch.empty(1, 2, 64, dtype=torch.float32))
    delta = torch.full((1, 2, 64), float("nan"), device=DEV)
    for name in ("dq", "dk", "dv"):
        grads = {"dq": dq, "dk": dk, "dv": dv}
        grads[name] = torch.empty(grads[name].shape, dtype=q.dtype)
        with pytest.raises(ValueError, match=name):
            fa.fa_bwd(q, k, v, o, lse, do, causal=True, delta=delta, **grads)
    with pytest.raises(ValueError, match="lse"):
        fa.fa_bwd(q, k, v, o, lse.cpu(), do, causal=True, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, delta):
        assert torch.isnan(t).all(), "a rejected call wrote its outputs"


def test_varlen_host_offsets_rejected():
    fa = _fa()
    g = torch.Generator().manual_seed(4)
    q = torch.randn(100, 2, 64, generator=g).to(torch.float16).to(DEV)
    k = torch.randn(100, 2, 64, generator=g).to(torch.float16).to(DEV)
    v = torch.randn(100, 2, 64, generator=g).to(torch.float16).to(DEV)
    cu = torch.tensor([0, 40, 100], dtype=torch.int32)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((2, 100), float("nan"), device=DEV)
    with pytest.raises(ValueError, match="cu_seqlens"):
        fa.fa_fwd_varlen(q, k, v, cu, cu.to(DEV), 60, 60, out=out, lse=lse)
    with pytest.raises(ValueError, match="lse"):
        fa.fa_fwd_varlen(q, k, v, cu.to(DEV), cu.to(DEV), 60, 60, out=out,
                         lse=torch.empty(2, 100, dtype=torch.float32))
    o, l = fa.fa_fwd_varlen(q, k, v, cu.to(DEV), cu.to(DEV), 60, 60)
    with pytest.raises(ValueError, match="delta"):
        fa.fa_bwd_varlen(q, k, v, o, l, torch.randn_like(o), cu.to(DEV), cu.to(DEV), 60, 60,
                         delta=torch.empty(2, 100, dtype=torch.float32))
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(lse).all(), "a rejected call wrote its outputs"
