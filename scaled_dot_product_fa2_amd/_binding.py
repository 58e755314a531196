"""ctypes binding of libfa.so. Argument marshalling only; every step of the
attention forward and backward runs in the library's kernels."""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional, Tuple

import torch

FA_DTYPE_F16 = 0
FA_DTYPE_BF16 = 1
FA_NOALLOC_MAX_ROWS = 4194304  # fa_bwd_noalloc: largest B * Hq * Nq (its fixed Delta array)
_DTYPES = {torch.float16: FA_DTYPE_F16, torch.bfloat16: FA_DTYPE_BF16}

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG_DIR, "libfa.so")


class FaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"fa error {code}: {msg}")
        self.code = code


class _Plan(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int64), ("block_threads", ctypes.c_int32), ("block_q", ctypes.c_int32),
                ("block_kv", ctypes.c_int32), ("lds_bytes", ctypes.c_int32), ("tile_pairs", ctypes.c_int64)]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libfa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or lib_path
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m scaled_dot_product_fa2_amd.build`")
    lib = ctypes.CDLL(p)
    i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64p, i64p, i64p, i64p, f32, i32,
                           i32, vp]
    lib.fa_fwd.restype = i32
    lib.fa_fwd_balanced.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64p, i64p, i64p, i64p, f32,
                                    i32, i32, vp, vp]
    lib.fa_fwd_balanced.restype = i32
    lib.fa_fwd_balance_applies.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32]
    lib.fa_fwd_balance_applies.restype = i32
    lib.fa_fwd_window.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64p, i64p, i64p, i64p, f32,
                                  i64, i64, i32, vp]
    lib.fa_fwd_window.restype = i32
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, i64p, i64p,
                                  i64p, i64p, f32, i32, i32, vp]
    lib.fa_fwd_varlen.restype = i32
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                           i64p, i64p, i64p, i64p, i64p, i64p, i64p, i64p, f32, i32, i32, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                   i64p, i64p, i64p, i64p, i64p, i64p, i64p, i64p, f32, i32, i32, vp]
    lib.fa_bwd_noalloc.restype = i32
    lib.fa_bwd_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                  i64p, i64p, i64p, i64p, i64p, i64p, i64p, i64p, f32, i64, i64, i32, vp]
    lib.fa_bwd_window.restype = i32
    i64_3 = ctypes.POINTER(ctypes.c_int64)
    lib.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                  i64, i64_3, i64_3, i64_3, i64_3, i64_3, i64_3, i64_3, i64_3, f32, i32, i32, vp]
    lib.fa_bwd_varlen.restype = i32
    lib.fa_fwd_plan.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32, ctypes.POINTER(_Plan)]
    lib.fa_fwd_plan.restype = i32
    lib.fa_tile_pairs.argtypes = [i64, i64, i64, i64, i32]
    lib.fa_tile_pairs.restype = i64
    lib.fa_strerror.argtypes = [i32]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i32
    if path is None:
        _lib = lib
    return lib


def fa_strerror(code: int) -> str:
    return load_library().fa_strerror(code).decode()


def fa_version() -> int:
    return load_library().fa_version()


def fa_tile_pairs(Nq: int, Nkv: int, bq: int, bkv: int, causal: bool) -> int:
    return load_library().fa_tile_pairs(Nq, Nkv, bq, bkv, int(bool(causal)))


def _check(code: int):
    if code != 0:
        raise FaError(code, fa_strerror(code))


def fa_fwd_plan(B: int, Hq: int, Hkv: int, Nq: int, Nkv: int, D: int, causal: bool, dtype) -> dict:
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    plan = _Plan()
    _check(load_library().fa_fwd_plan(B, Hq, Hkv, Nq, Nkv, D, int(bool(causal)), dt, ctypes.byref(plan)))
    return {f: getattr(plan, f) for f, _ in _Plan._fields_}


def fa_fwd_balance_applies(B: int, Hq: int, Hkv: int, Nq: int, Nkv: int, D: int, causal: bool, dtype) -> bool:
    """Whether the forward of this shape claims the tail of its schedule (see fa_fwd_balanced)."""
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    rc = load_library().fa_fwd_balance_applies(B, Hq, Hkv, Nq, Nkv, D, int(bool(causal)), dt)
    if rc < 0:
        raise FaError(rc, fa_strerror(rc))
    return rc == 1


def _strides(t: torch.Tensor):
    return (ctypes.c_int64 * 4)(*t.stride())


def _on_device(dev: torch.device, **tensors) -> None:
    """Every tensor must be a GPU tensor on `dev`: the C ABI takes raw pointers and cannot tell a host
    pointer, or one on another GPU, from a valid device pointer."""
    for name, t in tensors.items():
        if not t.is_cuda or t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev} (all tensors on one GPU)")


def _stream_for(dev: torch.device, stream):
    """The stream to launch on (default: the current stream of `dev`); it must belong to `dev`."""
    if stream is None:
        return torch.cuda.current_stream(dev)
    if stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, expected {dev}")
    return stream


# fa_fwd_balanced's counter words (FA_BALANCE_COUNTERS in fa.h), one zeroed buffer per (device,
# stream): calls in order on one stream may share a buffer, calls on different streams may not.
BALANCE_COUNTERS = 16
_balance_buffers = {}
_balance_lock = threading.Lock()


def _balance_counters(dev: torch.device, stream) -> torch.Tensor:
    """The counter buffer of `stream`, zero-filled on that stream on first use (so the fill is ordered
    before the stream's first forward) and kept for the life of the process; every forward leaves it
    zero again."""
    key = (dev.index, stream.cuda_stream)
    with _balance_lock:
        buf = _balance_buffers.get(key)
        if buf is None:
            with torch.cuda.device(dev), torch.cuda.stream(stream):
                buf = torch.zeros(BALANCE_COUNTERS, dtype=torch.int32, device=dev)
            _balance_buffers[key] = buf
    return buf


def _call_on(dev: torch.device, fn, *args) -> int:
    """Call a library entry point with `dev` as the current device. A launch on a null stream handle
    (the default stream) goes to the current device, and fa_bwd_noalloc looks up its array there, so
    it must be the device the tensors live on."""
    if torch.cuda.current_device() == dev.index:
        return fn(*args)
    with torch.cuda.device(dev):
        return fn(*args)


class FaCall:
    """A validated, pre-marshalled forward call on fixed tensors: calling it enqueues one forward
    (through fa_fwd_balanced, like ``fa_fwd``).

    Built by ``fa_fwd_call``; the ctypes argument tuple is prepared once, so repeated launches cost
    only the foreign call. The tensors must stay alive and keep their storage while it is used.
    """

    def __init__(self, dev, args, keepalive):
        self._fn = load_library().fa_fwd_balanced
        self._dev = dev
        self._args = args
        self._keepalive = keepalive

    def __call__(self) -> None:
        code = _call_on(self._dev, self._fn, *self._args)
        if code != 0:
            raise FaError(code, fa_strerror(code))


def fa_fwd_call(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor, *,
                causal: bool = False, scale: Optional[float] = None,
                stream: Optional[torch.cuda.Stream] = None) -> FaCall:
    """Prepare repeated forwards of the same tensors (see FaCall); checks arguments once."""
    fa_fwd(q, k, v, causal=causal, scale=scale, out=out, lse=lse, stream=stream)  # validates and runs once
    B, Hq, Nq, D = q.shape
    _, Hkv, Nkv, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    stream = _stream_for(q.device, stream)
    strides = [_strides(t) for t in (q, k, v, out)]
    counters = _balance_counters(q.device, stream)
    args = (ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
            ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
            B, Hq, Hkv, Nq, Nkv, D, *strides, ctypes.c_float(scale), int(bool(causal)), _DTYPES[q.dtype],
            ctypes.c_void_p(counters.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
    return FaCall(q.device, args, (q, k, v, out, lse, strides, counters))


class FaBwdCall:
    """A validated, pre-marshalled fa_bwd call on fixed tensors: calling it enqueues one backward
    (its three kernels). Built by ``fa_bwd_call``; the tensors must stay alive while it is used."""

    def __init__(self, dev, args, keepalive):
        self._fn = load_library().fa_bwd
        self._dev = dev
        self._args = args
        self._keepalive = keepalive

    def __call__(self) -> None:
        code = _call_on(self._dev, self._fn, *self._args)
        if code != 0:
            raise FaError(code, fa_strerror(code))


def fa_bwd_call(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                dout: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor, delta: torch.Tensor, *,
                causal: bool = False, scale: Optional[float] = None,
                stream: Optional[torch.cuda.Stream] = None) -> FaBwdCall:
    """Prepare repeated backwards of the same tensors (see FaBwdCall); checks arguments once."""
    fa_bwd(q, k, v, o, lse, dout, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv, delta=delta,
           stream=stream)  # validates and runs once
    B, Hq, Nq, D = q.shape
    _, Hkv, Nkv, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    stream = _stream_for(q.device, stream)
    strides = [_strides(t) for t in (q, k, v, o, dout, dq, dk, dv)]
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, o, lse, dout, dq, dk, dv, delta)]
    args = (*ptrs, B, Hq, Hkv, Nq, Nkv, D, *strides, ctypes.c_float(scale), int(bool(causal)), _DTYPES[q.dtype],
            ctypes.c_void_p(stream.cuda_stream))
    return FaBwdCall(q.device, args, (q, k, v, o, lse, dout, dq, dk, dv, delta, strides))


def fa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
           scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None
           ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention forward on BNSD tensors: returns (o, lse).

    q: (B, Hq, Nq, D); k, v: (B, Hkv, Nkv, D); fp16 or bf16 on one GPU; any strides with a unit
    head-dim stride and 16-byte aligned rows. ``scale`` defaults to 1/sqrt(D). ``out`` (same shape
    and dtype as q) and ``lse`` (contiguous float32 (B, Hq, Nq)) may be passed in; otherwise they are
    allocated. The kernel is enqueued on ``stream`` (default: the current stream), through
    fa_fwd_balanced with the stream's counter buffer: long causal launches then even out the XCDs'
    uneven clocks, with outputs bitwise those of fa_fwd.
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D (B, H, N, D)")
    if not q.is_cuda:
        raise ValueError("q, k, v must be GPU tensors")
    _on_device(q.device, k=k, v=v)
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPES:
        raise ValueError("q, k, v must share one dtype, float16 or bfloat16")
    B, Hq, Nq, D = q.shape
    _, Hkv, Nkv, _ = k.shape
    if k.shape != (B, Hkv, Nkv, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, Nq, D), dtype=q.dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, Hq, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (B, Hq, Nq) tensor")
    _on_device(q.device, out=out, lse=lse)
    stream = _stream_for(q.device, stream)
    counters = _balance_counters(q.device, stream)
    code = _call_on(
        q.device, load_library().fa_fwd_balanced, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr(), B, Hq, Hkv, Nq, Nkv, D, _strides(q), _strides(k), _strides(v), _strides(out),
        float(scale), int(bool(causal)), _DTYPES[q.dtype], ctypes.c_void_p(counters.data_ptr()),
        ctypes.c_void_p(stream.cuda_stream))
    _check(code)
    return out, lse


def fa_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
           dout: torch.Tensor, *, causal: bool = False, scale: Optional[float] = None,
           dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
           delta: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None,
           window: Optional[Tuple[int, int]] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Attention backward: returns (dq, dk, dv) for the forward (o, lse) = fa_fwd(q, k, v).

    dout is the gradient of the loss with respect to o (same shape and dtype). dq, dk, dv (shaped
    like q, k, v) and the float32 workspace ``delta`` (contiguous (B, Hq, Nq)) are allocated when
    not passed. Same dtype, stride and alignment rules as ``fa_fwd``. ``window=(left, right)``
    runs the backward of ``fa_fwd_window`` (then ``causal`` must be False).
    """
    if not q.is_cuda:
        raise ValueError("all tensors must be on the GPU")
    _on_device(q.device, k=k, v=v, o=o, lse=lse, dout=dout)
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype) or q.dtype not in _DTYPES:
        raise ValueError("q, k, v, o, dout must share one dtype, float16 or bfloat16")
    B, Hq, Nq, D = q.shape
    _, Hkv, Nkv, _ = k.shape
    if k.shape != (B, Hkv, Nkv, D) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v, o and dout")
    if lse.shape != (B, Hq, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (B, Hq, Nq) tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{name} must match the shape and dtype of its input")
    if delta is None:
        delta = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    elif delta.shape != (B, Hq, Nq) or delta.dtype != torch.float32 or not delta.is_contiguous():
        raise ValueError("delta must be a contiguous float32 (B, Hq, Nq) tensor")
    _on_device(q.device, dq=dq, dk=dk, dv=dv, delta=delta)
    stream = _stream_for(q.device, stream)
    common = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
              dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
              B, Hq, Hkv, Nq, Nkv, D, _strides(q), _strides(k), _strides(v), _strides(o), _strides(dout),
              _strides(dq), _strides(dk), _strides(dv), float(scale))
    if window is None:
        code = _call_on(q.device, load_library().fa_bwd, *common, int(bool(causal)), _DTYPES[q.dtype],
                        ctypes.c_void_p(stream.cuda_stream))
    else:
        if causal:
            raise ValueError("pass either causal or window, not both (the causal mask is window (-1, 0))")
        code = _call_on(q.device, load_library().fa_bwd_window, *common, int(window[0]), int(window[1]),
                        _DTYPES[q.dtype], ctypes.c_void_p(stream.cuda_stream))
    _check(code)
    return dq, dk, dv


def fa_bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                   dout: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor, *, causal: bool = False,
                   scale: Optional[float] = None, stream: Optional[torch.cuda.Stream] = None) -> None:
    """``fa_bwd`` through the entry point that allocates nothing: Delta lives in the library's fixed
    per-GPU array (B * Hq * Nq <= FA_NOALLOC_MAX_ROWS), so no workspace is passed, and dq, dk, dv must
    be given. Calls that overlap in time on one GPU share that array and must not be issued."""
    if not q.is_cuda:
        raise ValueError("all tensors must be on the GPU")
    _on_device(q.device, k=k, v=v, o=o, lse=lse, dout=dout, dq=dq, dk=dk, dv=dv)
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype) or q.dtype not in _DTYPES:
        raise ValueError("q, k, v, o, dout must share one dtype, float16 or bfloat16")
    B, Hq, Nq, D = q.shape
    _, Hkv, Nkv, _ = k.shape
    if k.shape != (B, Hkv, Nkv, D) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v, o and dout")
    if lse.shape != (B, Hq, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (B, Hq, Nq) tensor")
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{name} must match the shape and dtype of its input")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    stream = _stream_for(q.device, stream)
    _check(_call_on(
        q.device, load_library().fa_bwd_noalloc, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nkv, D, _strides(q), _strides(k), _strides(v),
        _strides(o), _strides(dout), _strides(dq), _strides(dk), _strides(dv), float(scale), int(bool(causal)),
        _DTYPES[q.dtype], ctypes.c_void_p(stream.cuda_stream)))


def fa_fwd_window(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, window_left: int = -1,
                  window_right: int = -1, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None
                  ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention forward with a sliding window: query row i sees keys i - window_left .. i + window_right
    (-1 = unbounded on that side). Same tensors, rules and return values as ``fa_fwd``; a row whose
    window holds no key gets O = 0 and LSE = -inf."""
    if not q.is_cuda:
        raise ValueError("q, k, v must be GPU tensors")
    _on_device(q.device, k=k, v=v)
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPES:
        raise ValueError("q, k, v must share one dtype, float16 or bfloat16")
    B, Hq, Nq, D = q.shape
    _, Hkv, Nkv, _ = k.shape
    if k.shape != (B, Hkv, Nkv, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, Nq, D), dtype=q.dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, Hq, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (B, Hq, Nq) tensor")
    _on_device(q.device, out=out, lse=lse)
    stream = _stream_for(q.device, stream)
    code = _call_on(
        q.device, load_library().fa_fwd_window, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
        B, Hq, Hkv, Nq, Nkv, D, _strides(q), _strides(k), _strides(v), _strides(out),
        float(scale), int(window_left), int(window_right), _DTYPES[q.dtype], ctypes.c_void_p(stream.cuda_stream))
    _check(code)
    return out, lse


def fa_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                  cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, *, causal: bool = False,
                  scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None
                  ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward over packed variable-length sequences.

    q: (total_q, Hq, D), k, v: (total_k, Hkv, D) token-major GPU tensors; cu_seqlens_q/k: int32 GPU
    tensors of B + 1 offsets. Returns o (total_q, Hq, D) and lse (Hq, total_q) float32.
    max_seqlen_q/k must be at least every sequence's length (the offsets stay on the GPU and are not
    checked here): rows of a longer sequence past it are left unwritten.
    """
    if not q.is_cuda:
        raise ValueError("all tensors must be on the GPU")
    _on_device(q.device, k=k, v=v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k)
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPES:
        raise ValueError("q, k, v must share one dtype, float16 or bfloat16")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if (cu_seqlens_q.dim() != 1 or not (cu_seqlens_q.is_contiguous() and cu_seqlens_k.is_contiguous())
            or cu_seqlens_q.shape != cu_seqlens_k.shape):
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be contiguous with B + 1 entries each")
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D token-major (total, H, D) tensors")
    total_q, Hq, D = q.shape
    total_k, Hkv, _ = k.shape
    if k.shape != (total_k, Hkv, D) or v.shape != k.shape:
        raise ValueError("k and v must be (total_k, Hkv, D) with q's head dim")
    B = cu_seqlens_q.shape[0] - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    elif lse.shape != (Hq, total_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (Hq, total_q) tensor")
    _on_device(q.device, out=out, lse=lse)
    stream = _stream_for(q.device, stream)

    def st3(t):
        return (ctypes.c_int64 * 3)(*t.stride())

    code = _call_on(
        q.device, load_library().fa_fwd_varlen, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), cu_seqlens_q.data_ptr(),
        cu_seqlens_k.data_ptr(), B, Hq, Hkv, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), D,
        st3(q), st3(k), st3(v), st3(out), float(scale), int(bool(causal)), _DTYPES[q.dtype],
        ctypes.c_void_p(stream.cuda_stream))
    _check(code)
    return out, lse


def fa_bwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                  dout: torch.Tensor, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int,
                  max_seqlen_k: int, *, causal: bool = False, scale: Optional[float] = None,
                  dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                  dv: Optional[torch.Tensor] = None, delta: Optional[torch.Tensor] = None,
                  stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward of ``fa_fwd_varlen``: returns (dq, dk, dv) shaped like q, k, v (token-major).

    o and lse are that call's outputs ((total_q, Hq, D) and (Hq, total_q) float32), dout the gradient
    of the loss with respect to o. The float32 workspace ``delta`` is (Hq, total_q).
    """
    if not q.is_cuda:
        raise ValueError("all tensors must be on the GPU")
    _on_device(q.device, k=k, v=v, o=o, lse=lse, dout=dout, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k)
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype) or q.dtype not in _DTYPES:
        raise ValueError("q, k, v, o, dout must share one dtype, float16 or bfloat16")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if (cu_seqlens_q.dim() != 1 or not (cu_seqlens_q.is_contiguous() and cu_seqlens_k.is_contiguous())
            or cu_seqlens_q.shape != cu_seqlens_k.shape):
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be contiguous with B + 1 entries each")
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D token-major (total, H, D) tensors")
    total_q, Hq, D = q.shape
    total_k, Hkv, _ = k.shape
    if k.shape != (total_k, Hkv, D) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v, o and dout")
    if lse.shape != (Hq, total_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (Hq, total_q) tensor")
    B = cu_seqlens_q.shape[0] - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{name} must match the shape and dtype of its input")
    if delta is None:
        delta = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    elif delta.shape != (Hq, total_q) or delta.dtype != torch.float32 or not delta.is_contiguous():
        raise ValueError("delta must be a contiguous float32 (Hq, total_q) tensor")
    _on_device(q.device, dq=dq, dk=dk, dv=dv, delta=delta)
    stream = _stream_for(q.device, stream)

    def st3(t):
        return (ctypes.c_int64 * 3)(*t.stride())

    code = _call_on(
        q.device, load_library().fa_bwd_varlen, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
        dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, Hq, Hkv,
        total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), D, st3(q), st3(k), st3(v), st3(o), st3(dout),
        st3(dq), st3(dk), st3(dv), float(scale), int(bool(causal)), _DTYPES[q.dtype],
        ctypes.c_void_p(stream.cuda_stream))
    _check(code)
    return dq, dk, dv
