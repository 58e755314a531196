"""fa_fwd_balanced against fa_fwd, through the C ABI.

The balanced entry point changes only which workgroup runs an item, never how an item is computed,
so its outputs must be bitwise those of fa_fwd on every launch, the ones that take the claimed tail
(dense causal, long key range, many rounds of items) and the ones that do not. Its counter buffer
must be left zero after every call, so that a buffer can serve call after call on one stream;
buffers of two streams must not interfere. Parity of the values themselves with the float64
oracle is covered by the forward parity tests, which run through the same entry point (the long
GQA workload among them takes the claimed tail). FA_RANDOM_SWEEP=<n> in the environment adds n/10
seeded random long launches of 8 192-20 000 tokens, compared the same way.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import pytest
import torch

import workloads
from scaled_dot_product_fa2_amd import _binding

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _args(q, k, v, o, lse, causal):
    B, Hq, Nq, D = q.shape
    _, Hkv, Nkv, _ = k.shape
    st = [(ctypes.c_int64 * 4)(*t.stride()) for t in (q, k, v, o)]
    dt = 1 if q.dtype == torch.bfloat16 else 0
    return (ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
            ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()), B, Hq, Hkv, Nq, Nkv, D, *st,
            ctypes.c_float(1.0 / math.sqrt(D)), int(causal), dt)


def _static(q, k, v, causal, stream):
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    rc = _binding.load_library().fa_fwd(*_args(q, k, v, o, lse, causal), ctypes.c_void_p(stream.cuda_stream))
    assert rc == 0, _binding.fa_strerror(rc)
    return o, lse


def _balanced(q, k, v, causal, counters, stream):
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    rc = _binding.load_library().fa_fwd_balanced(*_args(q, k, v, o, lse, causal),
                                                 ctypes.c_void_p(counters.data_ptr()),
                                                 ctypes.c_void_p(stream.cuda_stream))
    assert rc == 0, _binding.fa_strerror(rc)
    return o, lse


def _inputs(B, Hq, Hkv, N, D, dtype, seed):
    return tuple(t.to(DEV) for t in workloads.make_random(B, Hq, Hkv, N, N, D, dtype, seed=seed))


# (B, Hq, Hkv, N, D, dtype): launches that take the claimed tail (D <= 128, >= 128 key tiles, >= 8
# rounds; either mask)
TAKES_TAIL = [(4, 16, 16, 8192, 128, torch.bfloat16), (1, 32, 8, 16384, 128, torch.bfloat16),
              (4, 16, 16, 16384, 64, torch.float16), (5, 16, 2, 8192, 128, torch.float16),
              (8, 16, 16, 8192, 32, torch.bfloat16)]


CASES = [(s, True) for s in TAKES_TAIL] + [(TAKES_TAIL[1], False), (TAKES_TAIL[2], False)]


@pytest.mark.parametrize("shape,causal", CASES,
                         ids=[f"b{s[0]}h{s[1]}kv{s[2]}n{s[3]}d{s[4]}-{'c' if c else 'n'}" for s, c in CASES])
def test_balanced_is_bitwise_fa_fwd_and_leaves_counters_zero(shape, causal):
    B, Hq, Hkv, N, D, dtype = shape
    print(f"[case] balanced {shape} causal={causal}", flush=True)
    assert _binding.fa_fwd_balance_applies(B, Hq, Hkv, N, N, D, causal, dtype)
    q, k, v = _inputs(B, Hq, Hkv, N, D, dtype, seed=4000 + N // 64 + D)
    stream = torch.cuda.current_stream(DEV)
    counters = torch.zeros(_binding.BALANCE_COUNTERS, dtype=torch.int32, device=DEV)
    o_ref, l_ref = _static(q, k, v, causal, stream)
    for rep in range(3):  # call after call on one buffer
        o, lse = _balanced(q, k, v, causal, counters, stream)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"call {rep}: outputs differ from fa_fwd"
        assert not counters.any(), f"call {rep}: counters left {counters.tolist()}"


@pytest.mark.parametrize("shape,causal", [((4, 16, 16, 1024, 128), True), ((4, 16, 16, 1024, 128), False),
                                          ((4, 16, 16, 4096, 128), True), ((16, 16, 16, 4096, 128), False),
                                          ((2, 16, 16, 16384, 256), True)],
                         ids=["bench-causal", "bench-full", "n4096-causal", "n4096-full", "d256-causal"])
def test_static_launches_leave_counters_untouched(shape, causal):
    B, Hq, Hkv, N, D = shape
    assert not _binding.fa_fwd_balance_applies(B, Hq, Hkv, N, N, D, causal, torch.bfloat16)
    q, k, v = _inputs(B, Hq, Hkv, N, D, torch.bfloat16, seed=4100 + N // 64)
    stream = torch.cuda.current_stream(DEV)
    # a sentinel pattern the kernel would have zeroed had it taken the claimed tail
    counters = torch.full((_binding.BALANCE_COUNTERS,), 7, dtype=torch.int32, device=DEV)
    o_ref, l_ref = _static(q, k, v, causal, stream)
    o, lse = _balanced(q, k, v, causal, counters, stream)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    assert (counters == 7).all(), "a launch on the static schedule touched the counters"


def test_balanced_ragged_unequal_lengths():
    """A launch that takes the claimed tail with Nq != Nkv, neither a tile multiple."""
    B, Hq, Hkv, Nq, Nkv, D = 4, 16, 16, 8100, 12345, 128
    assert _binding.fa_fwd_balance_applies(B, Hq, Hkv, Nq, Nkv, D, True, torch.bfloat16)
    q, k, v = (t.to(DEV) for t in workloads.make_random(B, Hq, Hkv, Nq, Nkv, D, torch.bfloat16, seed=4400))
    stream = torch.cuda.current_stream(DEV)
    counters = torch.zeros(_binding.BALANCE_COUNTERS, dtype=torch.int32, device=DEV)
    o_ref, l_ref = _static(q, k, v, True, stream)
    for _ in range(2):
        o, lse = _balanced(q, k, v, True, counters, stream)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        assert not counters.any()


def test_two_streams_with_their_own_buffers():
    """Two streams run balanced launches at the same time, each with its own counters."""
    q, k, v = _inputs(4, 16, 16, 8192, 128, torch.bfloat16, seed=4200)
    q2, k2, v2 = _inputs(1, 32, 8, 16384, 128, torch.bfloat16, seed=4201)
    main = torch.cuda.current_stream(DEV)
    o_ref, l_ref = _static(q, k, v, True, main)
    o2_ref, l2_ref = _static(q2, k2, v2, True, main)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    c1 = torch.zeros(_binding.BALANCE_COUNTERS, dtype=torch.int32, device=DEV)
    c2 = torch.zeros(_binding.BALANCE_COUNTERS, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        outs.append((_balanced(q, k, v, True, c1, s1), _balanced(q2, k2, v2, True, c2, s2)))
    torch.cuda.synchronize()
    for (o, lse), (o2, lse2) in outs:
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        assert torch.equal(o2, o2_ref) and torch.equal(lse2, l2_ref)
    assert not c1.any() and not c2.any()


# Opt-in (FA_RANDOM_SWEEP=<n>): n/10 seeded random long launches, most of which take the claimed tail,
# each bitwise against fa_fwd with the counters left zero.
def _draw_long(n: int, seed: int):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([32, 64, 128]))
        hkv = int(rng.choice([3, 4, 5, 8]))
        Hq, B = hkv * int(rng.choice([2, 4])), int(rng.integers(2, 5))
        N = int(rng.integers(8192, 20000))
        Nk = N if rng.random() < 0.6 else int(rng.integers(8192, 20000))
        out.append((B, Hq, hkv, N, Nk, D, bool(rng.integers(2)), [torch.bfloat16, torch.float16][int(rng.integers(2))],
                    seed * 100 + i))
    return out


LONG = _draw_long(int(os.environ.get("FA_RANDOM_SWEEP", "0")) // 10, 71)
if LONG:  # defined only when asked for
    @pytest.mark.parametrize("case", LONG, ids=[f"b{c[0]}h{c[1]}kv{c[2]}-{c[3]}x{c[4]}-d{c[5]}-{'c' if c[6] else 'n'}"
                                                for c in LONG])
    def test_random_long_launch_is_bitwise_fa_fwd(case):
        B, Hq, Hkv, N, Nk, D, causal, dtype, seed = case
        print(f"[case] balanced random {case}", flush=True)
        q, k, v = (t.to(DEV) for t in workloads.make_random(B, Hq, Hkv, N, Nk, D, dtype, seed=seed))
        stream = torch.cuda.current_stream(DEV)
        counters = torch.zeros(_binding.BALANCE_COUNTERS, dtype=torch.int32, device=DEV)
        o_ref, l_ref = _static(q, k, v, causal, stream)
        for _ in range(2):
            o, lse = _balanced(q, k, v, causal, counters, stream)
            torch.cuda.synchronize()
            assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
            assert not counters.any()


def test_binding_forward_uses_the_stream_buffer():
    """fa_fwd (the binding) goes through fa_fwd_balanced with a zeroed buffer per stream."""
    import scaled_dot_product_fa2_amd as fa
    q, k, v = _inputs(4, 16, 16, 8192, 128, torch.bfloat16, seed=4300)
    o_ref, l_ref = _static(q, k, v, True, torch.cuda.current_stream(DEV))
    s = torch.cuda.Stream(DEV)
    with torch.cuda.stream(s):
        o, lse = fa.fa_fwd(q, k, v, causal=True)
        call = fa.fa_fwd_call(q, k, v, o, lse, causal=True)
        call()
        call()
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    buf = _binding._balance_counters(q.device, s)
    assert not buf.any()
