"""The C-ABI library without a GPU: it loads, exports every function include/fa.h declares, and
rejects every invalid call before touching HIP. Only invalid calls are made here (validation
returns before any HIP call), so nothing is ever launched."""
import ctypes
import json
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
LIB = os.path.join(ROOT, "scaled_dot_product_fa2_amd", "libfa.so")


def _lib():
    if not os.path.exists(LIB):
        pytest.fail("libfa.so is not built (python -m scaled_dot_product_fa2_amd.build)")
    from scaled_dot_product_fa2_amd import _binding
    return _binding.load_library()


def _header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\**\s+\**(fa_[a-z0-9_]+)\s*\(", src, re.M)))


def _header_defines():
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(FA_[A-Z0-9_]+)\s+(-?\d+)", open(HEADER).read())}


def test_exports_every_declared_function():
    names = _header_functions()
    assert set(names) >= {"fa_fwd", "fa_fwd_plan", "fa_tile_pairs", "fa_strerror", "fa_version"}
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(\w+)$", out, re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    lib = _lib()
    for n in names:
        assert hasattr(lib, n)


def test_version_and_strerror():
    lib = _lib()
    d = _header_defines()
    assert lib.fa_version() == d["FA_ABI_VERSION"]
    codes = [v for k, v in d.items() if k.startswith("FA_ERR_") or k == "FA_OK"]
    msgs = {lib.fa_strerror(c).decode() for c in codes}
    assert len(msgs) == len(codes), "every code has its own message"
    assert lib.fa_strerror(12345).decode() == "unknown error code"


def _st(*s):
    return (ctypes.c_int64 * 4)(*s)


VALID = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, lse=0x50000, B=1, Hq=2, Hkv=1, Nq=128, Nkv=128,
             D=64, qs=(16384, 8192, 64, 1), ks=(8192, 8192, 64, 1), vs=(8192, 8192, 64, 1),
             os=(16384, 8192, 64, 1), scale=0.125, causal=0, dtype=1)


def _call(**over):
    a = dict(VALID)
    a.update(over)
    lib = _lib()
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nkv"],
                      a["D"], _st(*a["qs"]) if a["qs"] else None, _st(*a["ks"]) if a["ks"] else None,
                      _st(*a["vs"]) if a["vs"] else None, _st(*a["os"]) if a["os"] else None, a["scale"],
                      a["causal"], a["dtype"], None)


D_ = _header_defines()
BAD = [
    ("null_q", dict(q=0), "FA_ERR_NULL"), ("null_lse", dict(lse=0), "FA_ERR_NULL"),
    ("null_stride", dict(ks=None), "FA_ERR_NULL"),
    ("dtype", dict(dtype=7), "FA_ERR_DTYPE"),
    ("head_dim_48", dict(D=48), "FA_ERR_HEAD_DIM"), ("head_dim_512", dict(D=512), "FA_ERR_HEAD_DIM"),
    ("gqa_3_2", dict(Hq=3, Hkv=2), "FA_ERR_GQA"), ("gqa_hkv0", dict(Hkv=0), "FA_ERR_GQA"),
    ("zero_nq", dict(Nq=0), "FA_ERR_SHAPE"), ("zero_nkv", dict(Nkv=0), "FA_ERR_SHAPE"),
    ("neg_b", dict(B=-1), "FA_ERR_SHAPE"), ("huge_n", dict(Nq=1 << 31), "FA_ERR_SHAPE"),
    ("huge_extent", dict(qs=(1 << 61, 8192, 64, 1), B=8), "FA_ERR_SHAPE"),
    ("d_stride", dict(qs=(16384, 8192, 64, 2)), "FA_ERR_LAYOUT"),
    ("odd_row_stride", dict(ks=(8192, 8192, 60, 1)), "FA_ERR_LAYOUT"),
    ("neg_stride", dict(vs=(8192, -8192, 64, 1)), "FA_ERR_LAYOUT"),
    ("zero_out_stride", dict(os=(16384, 0, 64, 1)), "FA_ERR_LAYOUT"),
    ("huge_row_stride", dict(ks=(1 << 30, 1 << 30, (1 << 22) + 8, 1)), "FA_ERR_LAYOUT"),
    ("misaligned_ptr", dict(k=0x20008), "FA_ERR_LAYOUT"), ("misaligned_lse", dict(lse=0x50002), "FA_ERR_LAYOUT"),
    ("scale_zero", dict(scale=0.0), "FA_ERR_SCALE"), ("scale_neg", dict(scale=-0.1), "FA_ERR_SCALE"),
    ("scale_nan", dict(scale=float("nan")), "FA_ERR_SCALE"), ("scale_inf", dict(scale=float("inf")), "FA_ERR_SCALE"),
]


@pytest.mark.parametrize("name,over,code", BAD, ids=[b[0] for b in BAD])
def test_validation_rejects(name, over, code):
    assert _call(**over) == D_[code]


def _call_balanced(counters=0x60000, **over):
    a = dict(VALID)
    a.update(over)
    return _lib().fa_fwd_balanced(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                                  a["Nkv"], a["D"], _st(*a["qs"]) if a["qs"] else None,
                                  _st(*a["ks"]) if a["ks"] else None, _st(*a["vs"]) if a["vs"] else None,
                                  _st(*a["os"]) if a["os"] else None, a["scale"], a["causal"], a["dtype"],
                                  counters, None)


@pytest.mark.parametrize("name,over,code", BAD, ids=[b[0] for b in BAD])
def test_balanced_validation_rejects(name, over, code):
    # fa_fwd_balanced validates exactly as fa_fwd, before any HIP call
    assert _call_balanced(**over) == D_[code]


# (B, Hq, Hkv, N, D, causal, expected): the balanced entry point claims the tail only of dense
# launches at D <= 128 with >= 128 key tiles and >= 8 rounds of items on an XCD
BALANCE_POLICY = [
    ((4, 16, 16, 1024, 128), True, 0),     # the benchmark shape: one round, 16 key tiles
    ((4, 16, 16, 1024, 128), False, 0),
    ((1, 32, 8, 16384, 128), True, 1),     # the long GQA workload: 8 rounds, 256 key tiles
    ((1, 32, 8, 16384, 128), False, 1),    # no mask: 8 rounds as well
    ((2, 16, 16, 4096, 256), True, 0),     # the D = 256 workload: 2 rounds
    ((128, 8, 8, 1024, 64), True, 0),      # many rounds, 16 key tiles
    ((4, 16, 16, 8192, 128), True, 1),     # exactly 8 rounds and 128 key tiles
    ((4, 16, 16, 4096, 128), True, 0),     # 4 rounds
    ((16, 16, 16, 4096, 128), False, 0),   # 16 rounds, but 64 key tiles
    ((2, 16, 16, 16384, 256), False, 0),   # D = 256
    ((2, 16, 16, 16384, 256), True, 0),    # 8 rounds, but D = 256: a stolen item's K/V stream costs more
    ((4, 16, 16, 16384, 64), True, 1),     # D = 64: 11 rounds, 256 key tiles
]


@pytest.mark.parametrize("shape,causal,want", BALANCE_POLICY,
                         ids=[f"b{s[0]}h{s[1]}kv{s[2]}n{s[3]}d{s[4]}-{'c' if c else 'n'}" for s, c, _ in BALANCE_POLICY])
def test_balance_policy(shape, causal, want):
    B, Hq, Hkv, N, D = shape
    assert _lib().fa_fwd_balance_applies(B, Hq, Hkv, N, N, D, int(causal), 1) == want
    assert _lib().fa_fwd_balance_applies(B, Hq, Hkv, N, N, D, int(causal), 0) == want


def test_balance_policy_rejects_what_fa_fwd_rejects():
    assert _lib().fa_fwd_balance_applies(1, 2, 1, 128, 128, 48, 1, 1) == D_["FA_ERR_HEAD_DIM"]
    assert _lib().fa_fwd_balance_applies(1, 3, 2, 128, 128, 64, 1, 1) == D_["FA_ERR_GQA"]
    assert _lib().fa_fwd_balance_applies(1, 2, 1, 128, 128, 64, 1, 9) == D_["FA_ERR_DTYPE"]


def test_balanced_counter_buffer_is_checked():
    from scaled_dot_product_fa2_amd import _binding
    assert D_["FA_BALANCE_COUNTERS"] == _binding.BALANCE_COUNTERS
    assert _call_balanced(counters=0) == D_["FA_ERR_NULL"]
    assert _call_balanced(counters=0x60004) == D_["FA_ERR_LAYOUT"]  # 64-byte alignment
    # and the counter checks come first: a bad buffer is reported even with a bad shape
    assert _call_balanced(counters=0, D=48) == D_["FA_ERR_NULL"]


def test_plan_and_tile_pairs():
    from scaled_dot_product_fa2_amd import fa_fwd_plan, fa_tile_pairs
    p = fa_fwd_plan(4, 16, 16, 1024, 1024, 128, False, 1)
    n_items = 4 * 16 * ((1024 + p["block_q"] - 1) // p["block_q"])
    # persistent grid: at most the items, at most what fits on the 256 CUs at once
    assert 8 <= p["grid"] <= n_items and p["grid"] <= 256 * 4
    assert fa_fwd_plan(1, 1, 1, 16, 16, 64, False, 0)["grid"] >= 1
    big = fa_fwd_plan(1, 32, 8, 16384, 16384, 128, True, 1)
    assert big["grid"] < 32 * 16384 // big["block_q"]
    assert p["block_threads"] % 64 == 0 and p["lds_bytes"] <= 160 * 1024
    nq_t = 1024 // p["block_q"]
    nkv_t = 1024 // p["block_kv"]
    assert p["tile_pairs"] == 4 * 16 * nq_t * nkv_t
    pc = fa_fwd_plan(4, 16, 16, 1024, 1024, 128, True, 1)
    assert pc["tile_pairs"] < p["tile_pairs"]
    assert fa_tile_pairs(0, 5, 4, 4, True) == -1


def test_causal_tile_count_golden():
    """The lower-triangle tile count printed for an 8 x 8 tile grid (tests/golden/causal_tiles.json)."""
    from scaled_dot_product_fa2_amd import fa_tile_pairs
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "causal_tiles.json")))
    for case in g["cases"]:
        n = case["tiles_per_side"] * case["tile"]
        assert fa_tile_pairs(n, n, case["tile"], case["tile"], False) == case["full_tiles"]
        assert fa_tile_pairs(n, n, case["tile"], case["tile"], True) == case["causal_tiles"]
        saved = 1 - case["causal_tiles"] / case["full_tiles"]
        assert abs(saved - case["saved_fraction"]) < 1e-12


def test_layout_selftest_cpp(tmp_path):
    """The kernel's index arithmetic, simulated lane by lane on the CPU (tests/layout_selftest.cpp)."""
    exe = tmp_path / "layout_selftest"
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "scaled_dot_product_fa2_amd", "csrc"),
                    os.path.join(ROOT, "tests", "layout_selftest.cpp"), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], stdout=subprocess.PIPE, text=True)
    assert res.returncode == 0, res.stdout


def test_product_path_has_no_cpu_fallback():
    """The binding never imports the oracle and raises when the library is missing."""
    src = open(os.path.join(ROOT, "scaled_dot_product_fa2_amd", "_binding.py")).read()
    assert "oracle" not in src
    from scaled_dot_product_fa2_amd import _binding
    with pytest.raises(RuntimeError):
        _binding.load_library("/nonexistent/libfa.so")


BWD_VALID = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, lse=0x50000, do=0x60000, dq=0x70000, dk=0x80000,
                 dv=0x90000, delta=0xA0000, B=1, Hq=2, Hkv=1, Nq=128, Nkv=128, D=64,
                 qs=(16384, 8192, 64, 1), ks=(8192, 8192, 64, 1), vs=(8192, 8192, 64, 1), os=(16384, 8192, 64, 1),
                 dos=(16384, 8192, 64, 1), dqs=(16384, 8192, 64, 1), dks=(8192, 8192, 64, 1),
                 dvs=(8192, 8192, 64, 1), scale=0.125, causal=1, dtype=1)


def _bwd_call(**over):
    a = dict(BWD_VALID)
    a.update(over)
    lib = _lib()
    st = [(_st(*a[n]) if a[n] else None) for n in ("qs", "ks", "vs", "os", "dos", "dqs", "dks", "dvs")]
    return lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["delta"],
                      a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nkv"], a["D"], *st, a["scale"], a["causal"],
                      a["dtype"], None)


BWD_BAD = [
    ("null_do", dict(do=0), "FA_ERR_NULL"), ("null_delta", dict(delta=0), "FA_ERR_NULL"),
    ("null_dk", dict(dk=0), "FA_ERR_NULL"), ("null_do_stride", dict(dos=None), "FA_ERR_NULL"),
    ("dtype", dict(dtype=3), "FA_ERR_DTYPE"), ("head_dim", dict(D=96), "FA_ERR_HEAD_DIM"),
    ("gqa", dict(Hq=3, Hkv=2), "FA_ERR_GQA"), ("zero_nkv", dict(Nkv=0), "FA_ERR_SHAPE"),
    ("grid_over_2p31", dict(B=300, Nq=1 << 30, Nkv=1 << 30, qs=(0, 0, 64, 1), ks=(0, 0, 64, 1), vs=(0, 0, 64, 1),
                            os=(0, 0, 64, 1), dos=(0, 0, 64, 1)), "FA_ERR_SHAPE"),
    ("dq_d_stride", dict(dqs=(16384, 8192, 64, 2)), "FA_ERR_LAYOUT"),
    ("dk_zero_stride", dict(dks=(8192, 8192, 0, 1)), "FA_ERR_LAYOUT"),
    ("misaligned_dv", dict(dv=0x90008), "FA_ERR_LAYOUT"), ("misaligned_delta", dict(delta=0xA0002), "FA_ERR_LAYOUT"),
    ("do_odd_stride", dict(dos=(16384, 8192, 60, 1)), "FA_ERR_LAYOUT"),
    ("scale_nan", dict(scale=float("nan")), "FA_ERR_SCALE"),
]


@pytest.mark.parametrize("name,over,code", BWD_BAD, ids=[b[0] for b in BWD_BAD])
def test_bwd_validation_rejects(name, over, code):
    assert _bwd_call(**over) == D_[code]


def _bwd_noalloc_call(**over):
    a = dict(BWD_VALID)
    a.update(over)
    lib = _lib()
    st = [(_st(*a[n]) if a[n] else None) for n in ("qs", "ks", "vs", "os", "dos", "dqs", "dks", "dvs")]
    return lib.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                              a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nkv"], a["D"], *st, a["scale"], a["causal"],
                              a["dtype"], None)


def _noalloc_over_limit():
    """A shape one query row per head past the fixed Delta array (B * Hq * Nq = max + 2)."""
    nq = D_["FA_NOALLOC_MAX_ROWS"] // 2 + 1
    qs = (2 * nq * 64, nq * 64, 64, 1)
    return dict(B=1, Hq=2, Hkv=1, Nq=nq, Nkv=128, qs=qs, os=qs, dos=qs, dqs=qs)


@pytest.mark.parametrize("name,over,code", [b for b in BWD_BAD if "delta" not in b[0]] +
                         [("over_scratch", _noalloc_over_limit(), "FA_ERR_SCRATCH")],
                         ids=[b[0] for b in BWD_BAD if "delta" not in b[0]] + ["over_scratch"])
def test_bwd_noalloc_validation_rejects(name, over, code):
    """The no-allocation backward validates like fa_bwd, then rejects a Delta larger than its fixed array,
    all before any HIP call."""
    assert _bwd_noalloc_call(**over) == D_[code]


def test_noalloc_limit_matches_binding():
    from scaled_dot_product_fa2_amd import _binding
    assert _binding.FA_NOALLOC_MAX_ROWS == D_["FA_NOALLOC_MAX_ROWS"]


def _bwd_win_call(left, right, **over):
    a = dict(BWD_VALID)
    a.update(over)
    lib = _lib()
    st = [(_st(*a[n]) if a[n] else None) for n in ("qs", "ks", "vs", "os", "dos", "dqs", "dks", "dvs")]
    return lib.fa_bwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                             a["delta"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nkv"], a["D"], *st, a["scale"], left,
                             right, a["dtype"], None)


@pytest.mark.parametrize("left,right,over,code", [
    (-2, 0, {}, "FA_ERR_SHAPE"), (3, -7, {}, "FA_ERR_SHAPE"),
    (4, 4, dict(Nkv=(1 << 30) + 1, ks=(0, 64 * ((1 << 30) + 1), 64, 1), vs=(0, 64 * ((1 << 30) + 1), 64, 1),
                dks=(0, 64 * ((1 << 30) + 1), 64, 1), dvs=(0, 64 * ((1 << 30) + 1), 64, 1)), "FA_ERR_SHAPE"),
    (4, 4, dict(D=80), "FA_ERR_HEAD_DIM"), (4, 4, dict(dq=0), "FA_ERR_NULL"), (4, 4, dict(lse=0x50001), "FA_ERR_LAYOUT"),
    (4, 4, dict(scale=-1.0), "FA_ERR_SCALE"), (4, 4, dict(dtype=7), "FA_ERR_DTYPE"),
], ids=["left_below_minus1", "right_below_minus1", "nkv_over_2p30", "head_dim", "null_dq", "misaligned_lse",
        "scale", "dtype"])
def test_bwd_window_validation_rejects(left, right, over, code):
    assert _bwd_win_call(left, right, **over) == D_[code]


def _win_call(left, right, **over):
    a = dict(VALID)
    a.update(over)
    lib = _lib()
    return lib.fa_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nkv"],
                             a["D"], _st(*a["qs"]), _st(*a["ks"]), _st(*a["vs"]), _st(*a["os"]), a["scale"], left, right,
                             a["dtype"], None)


@pytest.mark.parametrize("left,right,over,code", [
    (-2, 0, {}, "FA_ERR_SHAPE"), (0, -5, {}, "FA_ERR_SHAPE"),
    (4, 4, dict(Nq=(1 << 30) + 1, qs=(0, 64 * ((1 << 30) + 1), 64, 1), os=(0, 64 * ((1 << 30) + 1), 64, 1)),
     "FA_ERR_SHAPE"),
    (4, 4, dict(D=48), "FA_ERR_HEAD_DIM"), (4, 4, dict(q=0), "FA_ERR_NULL"), (4, 4, dict(scale=0.0), "FA_ERR_SCALE"),
], ids=["left_below_minus1", "right_below_minus1", "nq_over_2p30", "head_dim", "null_q", "scale"])
def test_window_validation_rejects(left, right, over, code):
    assert _win_call(left, right, **over) == D_[code]


VL = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, lse=0x50000, cq=0x60000, ck=0x61000, B=3, Hq=4, Hkv=2,
          tq=300, tk=400, mq=150, mk=200, D=64, qs=(256, 64, 1), ks=(128, 64, 1), vs=(128, 64, 1), os=(256, 64, 1),
          scale=0.125, causal=1, dtype=0)


def _vl_call(**over):
    a = dict(VL)
    a.update(over)
    st3 = lambda s: (ctypes.c_int64 * 3)(*s) if s else None
    return _lib().fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"], a["B"], a["Hq"], a["Hkv"],
                                a["tq"], a["tk"], a["mq"], a["mk"], a["D"], st3(a["qs"]), st3(a["ks"]), st3(a["vs"]),
                                st3(a["os"]), a["scale"], a["causal"], a["dtype"], None)


VL_BAD = [
    ("null_cu", dict(cq=0), "FA_ERR_NULL"), ("null_stride", dict(ks=None), "FA_ERR_NULL"),
    ("zero_total", dict(tq=0), "FA_ERR_SHAPE"), ("max_over_total", dict(mk=401), "FA_ERR_SHAPE"),
    ("zero_max", dict(mq=0), "FA_ERR_SHAPE"), ("misaligned_cu", dict(ck=0x61002), "FA_ERR_LAYOUT"),
    ("head_dim", dict(D=40), "FA_ERR_HEAD_DIM"), ("gqa", dict(Hq=3), "FA_ERR_GQA"),
    ("dim_stride", dict(qs=(256, 64, 2)), "FA_ERR_LAYOUT"), ("dtype", dict(dtype=9), "FA_ERR_DTYPE"),
    ("extent_overflow", dict(qs=(1 << 55, 64, 1)), "FA_ERR_SHAPE"),
    ("o_zero_token_stride", dict(os=(0, 64, 1)), "FA_ERR_LAYOUT"),
    # one-token sequences: the zero token stride would make every sequence write the same O row
    ("o_zero_token_stride_one_token_seqs", dict(mq=1, os=(0, 64, 1)), "FA_ERR_LAYOUT"),
]


@pytest.mark.parametrize("name,over,code", VL_BAD, ids=[b[0] for b in VL_BAD])
def test_varlen_validation_rejects(name, over, code):
    assert _vl_call(**over) == D_[code]


VLB = dict(VL, do=0x70000, dq=0x80000, dk=0x90000, dv=0xA0000, delta=0xB0000, dos=(256, 64, 1), dqs=(256, 64, 1),
           dks=(128, 64, 1), dvs=(128, 64, 1))


def _vlb_call(**over):
    a = dict(VLB)
    a.update(over)
    st3 = lambda s: (ctypes.c_int64 * 3)(*s) if s else None
    return _lib().fa_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                                a["delta"], a["cq"], a["ck"], a["B"], a["Hq"], a["Hkv"], a["tq"], a["tk"], a["mq"],
                                a["mk"], a["D"], st3(a["qs"]), st3(a["ks"]), st3(a["vs"]), st3(a["os"]), st3(a["dos"]),
                                st3(a["dqs"]), st3(a["dks"]), st3(a["dvs"]), a["scale"], a["causal"], a["dtype"], None)


VLB_BAD = [
    ("null_cu", dict(ck=0), "FA_ERR_NULL"), ("null_do", dict(do=0), "FA_ERR_NULL"),
    ("null_delta", dict(delta=0), "FA_ERR_NULL"), ("null_dq_stride", dict(dqs=None), "FA_ERR_NULL"),
    ("zero_total", dict(tk=0), "FA_ERR_SHAPE"), ("max_over_total", dict(mq=301), "FA_ERR_SHAPE"),
    ("zero_batch", dict(B=0), "FA_ERR_SHAPE"), ("misaligned_cu", dict(cq=0x60001), "FA_ERR_LAYOUT"),
    ("misaligned_dk", dict(dk=0x90004), "FA_ERR_LAYOUT"), ("misaligned_delta", dict(delta=0xB0002), "FA_ERR_LAYOUT"),
    ("dv_dim_stride", dict(dvs=(128, 64, 2)), "FA_ERR_LAYOUT"), ("dq_zero_token_stride", dict(dqs=(0, 64, 1)),
                                                                 "FA_ERR_LAYOUT"),
    ("head_dim", dict(D=24), "FA_ERR_HEAD_DIM"), ("gqa", dict(Hkv=3), "FA_ERR_GQA"),
    ("dtype", dict(dtype=5), "FA_ERR_DTYPE"), ("scale", dict(scale=float("inf")), "FA_ERR_SCALE"),
    ("extent_overflow", dict(dos=(256, 1 << 62, 1)), "FA_ERR_SHAPE"),
    ("row_stride_over_limit", dict(dos=(1 << 55, 64, 1)), "FA_ERR_LAYOUT"),
]


@pytest.mark.parametrize("name,over,code", VLB_BAD, ids=[b[0] for b in VLB_BAD])
def test_varlen_bwd_validation_rejects(name, over, code):
    assert _vlb_call(**over) == D_[code]


def test_launch_runs_with_the_tensors_device_current(monkeypatch):
    """A launch on a null stream handle goes to the current device, so the binding makes the tensors'
    device current around each library call, and only when another device is current (host logic,
    with the device calls replaced by stand-ins)."""
    import torch
    from scaled_dot_product_fa2_amd import _binding
    state = {"current": 0, "entered": []}

    class _Guard:
        def __init__(self, dev):
            self.dev = dev

        def __enter__(self):
            state["entered"].append(self.dev.index)
            self.prev, state["current"] = state["current"], self.dev.index

        def __exit__(self, *exc):
            state["current"] = self.prev
            return False

    monkeypatch.setattr(torch.cuda, "current_device", lambda: state["current"])
    monkeypatch.setattr(torch.cuda, "device", _Guard)
    seen = []
    fn = lambda *args: seen.append((state["current"], args)) or 0
    assert _binding._call_on(torch.device("cuda", 0), fn, 1, 2) == 0
    assert seen[-1] == (0, (1, 2)) and state["entered"] == []      # already current: no switch
    assert _binding._call_on(torch.device("cuda", 3), fn, 7) == 0
    assert seen[-1] == (3, (7,)) and state["entered"] == [3]       # switched for the call
    assert state["current"] == 0                                   # and back afterwards
