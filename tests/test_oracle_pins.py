"""The fp64 oracle against its pins (CPU only)."""
import math

import numpy as np
import pytest

from oracle import lse_combine_ref, mla_decode_ref
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(mla_decode_ref)


def test_lse_combine_closed_forms():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((4, 512))
    l = rng.standard_normal(4)
    # an empty range (lse = -inf) is neutral
    out, lse = lse_combine_ref([o, rng.standard_normal((4, 512))], [l, np.full(4, -np.inf)])
    np.testing.assert_array_equal(lse, l)
    np.testing.assert_allclose(out, o, rtol=0, atol=0)
    # all empty -> lse = -inf, out = 0
    out, lse = lse_combine_ref([o, o], [np.full(4, -np.inf)] * 2)
    assert np.all(np.isneginf(lse)) and np.all(out == 0)
    # two identical halves: lse + ln 2, same out
    out, lse = lse_combine_ref([o, o], [l, l])
    np.testing.assert_allclose(lse, l + math.log(2.0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(out, o, rtol=0, atol=1e-15)
    # weights: exp(l_a) : exp(l_b) = 1 : 3
    oa, ob = np.ones((1, 512)), 5 * np.ones((1, 512))
    out, lse = lse_combine_ref([oa, ob], [np.array([0.0]), np.array([math.log(3.0)])])
    np.testing.assert_allclose(out, 4.0 * np.ones((1, 512)), rtol=0, atol=1e-14)
    assert abs(lse[0] - math.log(4.0)) < 1e-15
