"""The float64 oracle against its pins (closed forms, invariants, brute force, library routines)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_pool_matches_serial():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 4, 33, 16))
    k = rng.standard_normal((2, 2, 33, 16))
    v = rng.standard_normal((2, 2, 33, 16))
    o, lse = oracle.attention_ref(q, k, v, causal=True, scale=0.4)
    res, workers = oracle.attention_ref_pool(q, k, v, causal=True, scale=0.4, workers=2)
    assert workers == 2 and len(res) == 8
    for (b, h), (ob, lb) in res.items():
        assert np.array_equal(ob, o[b, h]) and np.array_equal(lb, lse[b, h])


def test_rejects_bad_shapes():
    z = np.zeros
    with pytest.raises(ValueError):
        oracle.attention_ref(z((1, 3, 4, 8)), z((1, 2, 4, 8)), z((1, 2, 4, 8)), causal=False)
    with pytest.raises(ValueError):
        oracle.attention_ref(z((1, 2, 4, 8)), z((1, 2, 0, 8)), z((1, 2, 0, 8)), causal=False)
    with pytest.raises(ValueError):
        oracle.attention_ref(z((1, 2, 4, 8)), z((1, 2, 4, 4)), z((1, 2, 4, 8)), causal=False)
