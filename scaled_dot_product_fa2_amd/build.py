"""Build libfa.so (the gfx950 attention forward and backward) in-tree with hipcc.

The kernel instances are compiled per (element type, head dim) as separate objects, in parallel
(fa_fwd_inst.hip and fa_bwd_inst.hip with -DFA_INST_T / -DFA_INST_D), next to the C ABI in
fa_api.hip; the objects are then linked into one shared library.

Usage: python -m scaled_dot_product_fa2_amd.build [-j JOBS] [--timeline]

--timeline builds libfa_timeline.so instead: the same sources compiled with -DFA_TIMELINE, whose
forward kernels also record per-workgroup clock stamps (bench.py --timeline reads them). libfa.so,
which the binding loads, never contains them.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
TIMELINE_LIB_PATH = os.path.join(PKG_DIR, "libfa_timeline.so")
HEAD_DIMS = (16, 32, 64, 128, 256)
DTYPES = ((0, "f16"), (1, "bf16"))

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are switched off for every device pass.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", *DEVICE_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}"]


def compile_jobs(obj_dir: str = OBJ_DIR, extra=()):
    """(object path, hipcc command) for every translation unit."""
    flags = [*COMMON, *extra]
    api = os.path.join(obj_dir, "fa_api.o")
    jobs = [(api, [HIPCC, *flags, "-c", os.path.join(CSRC, "fa_api.hip"), "-o", api])]
    for part in ("bwd", "fwd"):  # the backward instances are the slower ones: start them first
        for d in sorted(HEAD_DIMS, reverse=True):
            for t, tn in DTYPES:
                obj = os.path.join(obj_dir, f"fa_{part}_{tn}_d{d}.o")
                jobs.append((obj, [HIPCC, *flags, f"-DFA_INST_T={t}", f"-DFA_INST_D={d}", "-c",
                                   os.path.join(CSRC, f"fa_{part}_inst.hip"), "-o", obj]))
    return jobs


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = ("not a recognized feature", "loop not unrolled")
    lines = [l for l in res.stdout.splitlines() if not any(n in l for n in noise)]
    return res.returncode, "\n".join(lines)


def build(verbose: bool = True, jobs: int | None = None, timeline: bool = False) -> str:
    """Compile every instance and the C ABI, link libfa.so in place (atomically replaced); with
    timeline=True the clock-stamping variant libfa_timeline.so instead."""
    obj_dir = os.path.join(OBJ_DIR, "timeline") if timeline else OBJ_DIR
    lib_path = TIMELINE_LIB_PATH if timeline else LIB_PATH
    os.makedirs(obj_dir, exist_ok=True)
    todo = compile_jobs(obj_dir, ("-DFA_TIMELINE",) if timeline else ())
    if jobs is None:
        jobs = min(16, len(os.sched_getaffinity(0)))
    if verbose:
        print(f"[build] {len(todo)} translation units with {jobs} parallel hipcc jobs", flush=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda j: _run(j[1]), todo))
    failed = [(j, out) for j, (rc, out) in zip(todo, results) if rc != 0]
    if failed:
        for (obj, cmd), out in failed:
            sys.stderr.write(f"[build] FAILED: {' '.join(cmd)}\n{out}\n")
        raise RuntimeError(f"hipcc failed on {len(failed)} translation unit(s)")
    tmp = lib_path + ".tmp"
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for o, _ in todo], "-o", tmp]
    if verbose:
        print("[build]", " ".join(link), flush=True)
    rc, out = _run(link)
    if rc != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"link failed with exit code {rc}")
    os.replace(tmp, lib_path)
    return lib_path


def clean() -> None:
    shutil.rmtree(OBJ_DIR, ignore_errors=True)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", "--jobs", type=int, default=None)
    ap.add_argument("--timeline", action="store_true", help="build libfa_timeline.so (clock stamps)")
    args = ap.parse_args()
    build(jobs=args.jobs, timeline=args.timeline)
