"""The fp16 storage of split partials (CPU): a row of a piece's normalized
output o is stored as fp16(o * 2^(15 - e)), e the binary exponent of the row's
largest |o| (so every stored magnitude is below 2^15), and read back times
2^(e - 15).  The merged output out = sum_s w_s o_s (w_s = exp(lse_s - lse))
then differs from the exact merge by at most 2^-11 max_s |o_s| + 2^-40 max|o|
per element.  This checks that bound on random partials, including rows with
very different magnitudes and values that fall into fp16's subnormal range."""
import numpy as np
import pytest


def store_load(o):
    """fp16 round trip of each row with its power-of-two scale."""
    amax = np.max(np.abs(o), axis=-1, keepdims=True)
    e = np.maximum(np.frexp(amax)[1], -110)  # amax = m 2^e, 0.5 <= m < 1
    c = np.ldexp(1.0, 15 - e)
    h = (o * c).astype(np.float16)
    assert np.all(np.isfinite(h))
    return h.astype(np.float64) / c


@pytest.mark.parametrize("seed", range(6))
def test_fp16_partials_error_bound(seed):
    rng = np.random.default_rng(seed)
    S, rows, cols = int(rng.integers(2, 40)), 64, 512
    # partial outputs: weighted means of V rows, magnitudes from tiny to large
    o = rng.standard_normal((S, rows, cols)) * np.exp2(rng.integers(-30, 8, (S, rows, 1)))
    o[0, 0, :5] = 1e-12  # elements far below the row maximum: fp16 subnormals after scaling
    lse = rng.standard_normal((S, rows)) * 5
    w = np.exp(lse - np.logaddexp.reduce(lse, axis=0))
    exact = np.einsum("sr,src->rc", w, o)
    merged = np.einsum("sr,src->rc", w, store_load(o))
    bound = 2.0**-11 * np.max(np.abs(o), axis=0) + 2.0**-40 * np.max(np.abs(o))
    assert np.all(np.abs(merged - exact) <= bound + 1e-300)
    # and the bound is not loose by orders of magnitude: rounding uses most of it somewhere
    assert np.max(np.abs(merged - exact) / bound) > 0.05


def test_scale_keeps_fp16_in_range():
    # the row maximum maps into [2^14, 2^15): no overflow, full precision
    for amax in [1e-30, 3e-8, 0.7, 1.0, 65504.0, 1e20]:
        o = np.array([[amax, -amax / 3, amax / 1e6]])
        e = np.frexp(amax)[1]
        scaled = amax * 2.0 ** (15 - e)
        assert 2**14 <= scaled < 2**15
        assert np.all(np.isfinite(store_load(o)))
