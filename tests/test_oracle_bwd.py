"""The float64 backward oracle against its pins, and a mutation check of those pins: each
plausible mistake planted in a private copy of the oracle's source must fail at least one pin."""
import os
import types

import pytest

import oracle
from oracle import attention_bwd
from tests import oracle_bwd_pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention_bwd.py")


@pytest.mark.parametrize("pin", oracle_bwd_pins.ALL_BWD_PINS, ids=[p.__name__ for p in oracle_bwd_pins.ALL_BWD_PINS])
def test_backward_oracle_pin(pin):
    pin(attention_bwd)


MUTANTS = [
    ("delta_dropped", "ds = scale * p * (dp - delta[:, None])", "ds = scale * p * dp"),
    ("delta_sign", "ds = scale * p * (dp - delta[:, None])", "ds = scale * p * (dp + delta[:, None])"),
    ("ds_scale_dropped", "ds = scale * p * (dp - delta[:, None])", "ds = p * (dp - delta[:, None])"),
    ("delta_without_o", "delta = np.sum(o * doh[r], axis=1)", "delta = np.sum(doh[r], axis=1)"),
    ("dk_from_p", "dk += ds.T @ qh[r]", "dk += p.T @ qh[r]"),
    ("dv_from_ds", "dv += p.T @ doh[r]", "dv += ds.T @ doh[r]"),
    ("dv_from_o", "dv += p.T @ doh[r]", "dv += p.T @ o"),
    ("dq_keys_reversed", "dq[r] = ds @ kh", "dq[r] = ds @ kh[::-1]"),
    ("dp_values_reversed", "dp = doh[r] @ vh.T", "dp = doh[r] @ vh[::-1].T"),
    ("causal_strict", "key_pos[None, :] <= r[:, None]", "key_pos[None, :] < r[:, None]"),
    ("causal_ignored", "if causal:\n        s = np.where", "if False:\n        s = np.where"),
    ("group_not_summed", "dk[b, kvh] += dkh", "dk[b, kvh] = dkh"),
    ("gqa_modulo", "kvh = h // group", "kvh = h % Hkv"),
    ("no_normalisation", "return e / z", "return e"),
    ("window_left_off_by_one", "r[:, None] - left, s", "r[:, None] - left - 1, s"),
    ("window_right_ignored", "if right is not None:\n            s", "if False:\n            s"),
    ("rows_dq_scale_dropped", "ds = scale * p * (doh @ vh.T - delta[:, None])", "ds = p * (doh @ vh.T - delta[:, None])"),
    ("varlen_keys_at_query_offsets", "k[k0:k1].transpose(1, 0, 2)[None],\n", "k[q0:q0 + k1 - k0].transpose(1, 0, 2)[None],\n"),
    ("varlen_dk_not_written", "dk[k0:k1] = gk[0].transpose(1, 0, 2)", "pass"),
    ("varlen_causal_dropped", "v[k0:k1].transpose(1, 0, 2)[None], do[q0:q1].transpose(1, 0, 2)[None],\n                                       causal=causal",
     "v[k0:k1].transpose(1, 0, 2)[None], do[q0:q1].transpose(1, 0, 2)[None],\n                                       causal=False"),
]


def _load_mutant(find, replace):
    src = open(SRC_PATH).read()
    assert src.count(find) >= 1, f"mutation anchor not found: {find!r}"
    mod = types.ModuleType("oracle_bwd_mutant")
    mod.__file__ = SRC_PATH
    exec(compile(src.replace(find, replace), SRC_PATH + "[mutant]", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,find,replace", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_backward_pins_catch_mutant(name, find, replace):
    mod = _load_mutant(find, replace)
    failures = []
    for pin in oracle_bwd_pins.ALL_BWD_PINS:
        try:
            pin(mod)
        except Exception as exc:
            failures.append(f"{pin.__name__}: {type(exc).__name__}")
    assert failures, f"mutant {name} passed every pin"


def test_exported():
    assert oracle.attention_bwd_ref is attention_bwd.attention_bwd_ref
    assert oracle.attention_varlen_bwd_ref is attention_bwd.attention_varlen_bwd_ref
