"""Properties of the generated gfx950 code that the numerics rely on (CPU: compiles to assembly).

The dQ kernel feeds dS to the matrix cores as two fp16 terms, hi = round(dS) and lo = round(dS - hi),
both taken from the one fp32 dS. The backend can fold the conversion of a product to fp16 into a
mixed-precision multiply-add (one rounding of the exact product) for one use of hi and keep the
plain conversion of the fp32 product for another; where the product lies next to an fp16 rounding
midpoint the two hi values then differ by one unit in the last place and hi + lo misses dS by that
much (seen as a dQ element 5 % outside its derived error bound on a seeded fp16 window case). The
kernel makes dS opaque before converting it; this test checks that no dQ instance of the fp16
build contains such a fused conversion.
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from scaled_dot_product_fa2_amd import build as b


def _dq_bodies(T: int, D: int, tmp_path) -> dict:
    out = os.path.join(str(tmp_path), f"bwd_{T}_{D}.s")
    cmd = [b.HIPCC, f"--offload-arch={b.ARCH}", "-O3", "-std=c++17", *b.DEVICE_FLAGS, f"-I{b.INCLUDE}",
           f"-I{b.CSRC}", f"-DFA_INST_T={T}", f"-DFA_INST_D={D}", "-S", "--offload-device-only",
           os.path.join(b.CSRC, "fa_bwd_inst.hip"), "-o", out]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout[-2000:]
    text = open(out).read()
    bodies = {}
    for m in re.finditer(r"^(_ZN2fa16fa_bwd_dq_kernel\S+):", text, re.M):
        end = text.find(".Lfunc_end", m.start())
        bodies[m.group(1)] = text[m.start():end]
    return bodies


@pytest.mark.skipif(not os.path.exists(b.HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("D", [32, 128])
def test_fp16_dq_terms_come_from_one_fp32_value(D, tmp_path):
    bodies = _dq_bodies(0, D, tmp_path)
    # dense (both masks), window and packed-sequence (both masks) instances
    assert len(bodies) == 5, sorted(bodies)
    for name, body in bodies.items():
        assert "v_mfma" in body, f"{name}: no matrix instructions found (wrong function boundaries?)"
        assert not re.search(r"\bv_fma_mix", body), f"{name}: a conversion to fp16 is fused into a multiply"
