"""Mutation check of the oracle's pins.

Each case plants one plausible mistake in a private copy of the oracle's source
(a dropped term, an off-by-one mask, a wrong head index, a transposed or
reversed operand, a wrong logarithm base) and asserts that at least one pin
rejects the broken copy. The real oracle module is never modified.
"""
import os
import types

import pytest

from tests import oracle_pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTANTS = [
    ("causal_strict", "key_pos[None, :] <= r[:, None]", "key_pos[None, :] < r[:, None]"),
    ("causal_reversed", "key_pos[None, :] <= r[:, None]", "key_pos[None, :] >= r[:, None]"),
    ("causal_ignored", "if causal:\n            visible", "if False:\n            visible"),
    ("scale_dropped", "s = scale * (qh[r] @ kh.T)", "s = (qh[r] @ kh.T)"),
    ("scale_squared", "s = scale * (qh[r] @ kh.T)", "s = scale * scale * (qh[r] @ kh.T)"),
    ("default_scale_1_over_d", "scale = 1.0 / math.sqrt(D)\n    group", "scale = 1.0 / D\n    group"),
    ("gqa_modulo", "kvh = h // group\n", "kvh = h % Hkv\n"),
    ("gqa_rows_modulo", "kvh = h // (Hq // Hkv)", "kvh = h % Hkv"),
    ("lse_drops_max", "m[:, 0] + np.log(l[:, 0])", "np.log(l[:, 0])"),
    ("lse_log2", "m[:, 0] + np.log(l[:, 0])", "m[:, 0] + np.log2(l[:, 0])"),
    ("no_normalisation", "(e / l) @ vh", "e @ vh"),
    ("no_max_shift", "e = np.exp(s - m)", "e = np.exp(s)"),
    ("values_reversed", "(e / l) @ vh", "(e / l) @ vh[::-1]"),
    ("keys_reversed", "(qh[r] @ kh.T)", "(qh[r] @ kh[::-1].T)"),
    ("q_rows_shifted", "(qh[r] @ kh.T)", "(qh[(r + 1) % qh.shape[0]] @ kh.T)"),
    ("max_over_all_rows", "m = np.max(s, axis=1, keepdims=True)", "m = np.max(s, keepdims=True)"),
    ("denominator_offset", "l = np.sum(e, axis=1, keepdims=True)", "l = np.sum(e, axis=1, keepdims=True) + 1e-3"),
    ("window_left_off_by_one", "r[:, None] - left, s", "r[:, None] - left + 1, s"),
    ("window_right_ignored", "if right is not None:\n                s", "if False:\n                s"),
    ("window_right_as_left", "r[:, None] + right, s", "r[:, None] + left, s"),
    ("empty_row_lse_zero", "np.where(empty, -np.inf,", "np.where(empty, 0.0,"),
    ("varlen_keys_shifted", "k[k0:k1].transpose(1, 0, 2)[None],", "k[k0 + 1:k1 + 1].transpose(1, 0, 2)[None],"),
    ("varlen_q_offsets_for_keys", "v[k0:k1].transpose(1, 0, 2)[None]", "v[q0:q0 + k1 - k0].transpose(1, 0, 2)[None]"),
]


def _load_mutant(find, replace):
    with open(SRC_PATH) as f:
        src = f.read()
    assert src.count(find) >= 1, f"mutation anchor not found in oracle source: {find!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = SRC_PATH
    exec(compile(src.replace(find, replace), SRC_PATH + "[mutant]", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,find,replace", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, find, replace):
    mod = _load_mutant(find, replace)
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as exc:  # AssertionError or a crash both count as caught
            failures.append(f"{pin.__name__}: {type(exc).__name__}")
    assert failures, f"mutant {name} passed every pin"


def test_unmutated_copy_passes():
    mod = _load_mutant("s = scale * (qh[r] @ kh.T)", "s = scale * (qh[r] @ kh.T)")
    for pin in oracle_pins.ALL_PINS:
        pin(mod)
