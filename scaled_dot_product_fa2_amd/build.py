"""Build libfa.so (the gfx950 attention forward and backward) in-tree with hipcc.

Usage: python -m scaled_dot_product_fa2_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
SOURCES = [os.path.join(CSRC, "fa_api.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("fa_fwd_kernel.h", "fa_bwd_kernel.h", "fa_layout.h")] + [os.path.join(INCLUDE, "fa.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are switched off for every device pass.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_cmd(out: str = LIB_PATH):
    return [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
            *DEVICE_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *SOURCES, "-o", out]


def build(verbose: bool = True) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = build_cmd(tmp)
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = ("not a recognized feature", "loop not unrolled")
    lines = [l for l in res.stdout.splitlines() if not any(n in l for n in noise)]
    if res.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build()
