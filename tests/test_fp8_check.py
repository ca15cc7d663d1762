"""The FP8 code check of the GPU tests (tests/gpu_util.py check_fp8), on the CPU,
against planted cases: it must accept a code that differs from the oracle's only
where the oracle's scaled value sits within the pooling error of the midpoint
between the two codes, and refuse every other difference."""

import numpy as np
import pytest

from oracle import e4m3_decode, quantize_e4m3_rows
from tests.gpu_util import EPS_POOL, check_fp8, pool_magnitude

GRID = e4m3_decode(np.arange(0x7F))


def row_with_value(y_at_3, amax=448.0):
    """A four-head entry whose scales are 1 (amax 448) and whose element 3 of head 0
    scales to y_at_3; the others are plain grid values (one planted difference is
    then 1/512 of the codes, under the check's 0.5% limit)."""
    x = np.zeros((4, 128))
    x[:, 0] = amax
    x[:, 1:] = GRID[40]
    x[0, 3] = y_at_3
    return x


def flip(codes, i):
    """The code one grid step above element i's (same sign)."""
    c = codes.copy()
    c[0, i] += 1
    return c


def test_accepts_identical_codes():
    x = row_with_value(GRID[50])
    codes, s, _ = quantize_e4m3_rows(x)
    check_fp8(codes, s, codes, s, x, "same")


@pytest.mark.parametrize("mag", [None, 1.0])
def test_accepts_a_flip_at_the_midpoint(mag):
    mid = (GRID[50] + GRID[51]) / 2
    x = row_with_value(mid * (1 - 0.2 * EPS_POOL))        # just below the midpoint
    codes, s, _ = quantize_e4m3_rows(x)
    assert e4m3_decode(codes[0, 3]) == GRID[50]
    m = None if mag is None else np.full(x.shape, mid)
    check_fp8(flip(codes, 3), s, codes, s, x, "flip at the midpoint", m)


def test_refuses_a_flip_away_from_the_midpoint():
    x = row_with_value(GRID[50] * (1 + 0.01))
    codes, s, _ = quantize_e4m3_rows(x)
    with pytest.raises(AssertionError):
        check_fp8(flip(codes, 3), s, codes, s, x, "far flip", np.full(x.shape, GRID[50]))


def test_refuses_two_steps_and_sign_flips():
    mid = (GRID[50] + GRID[51]) / 2
    x = row_with_value(mid)
    codes, s, _ = quantize_e4m3_rows(x)
    two = codes.copy()
    two[0, 3] += 2
    with pytest.raises(AssertionError):
        check_fp8(two, s, codes, s, x, "two steps", np.full(x.shape, mid))
    neg = codes.copy()
    neg[0, 3] ^= 0x80
    with pytest.raises(AssertionError):
        check_fp8(neg, s, codes, s, x, "sign", np.full(x.shape, mid))


def test_zero_and_its_neighbours():
    """Around 0: +0 against -0 where y is within the error of 0; the smallest
    subnormal against a zero of the other sign near their midpoint. A zero against a
    code two steps away is refused."""
    x = row_with_value(1e-9)                               # rounds to +0
    codes, s, _ = quantize_e4m3_rows(x)
    assert codes[0, 3] == 0x00
    negz = codes.copy()
    negz[0, 3] = 0x80
    check_fp8(negz, s, codes, s, x, "-0", np.full(x.shape, 1e-4))
    half = 2.0 ** -10                                      # midpoint of 0 and 2**-9
    x = row_with_value(half * (1 - 0.2 * EPS_POOL))
    codes, s, _ = quantize_e4m3_rows(x)
    assert codes[0, 3] == 0x00
    up = codes.copy()
    up[0, 3] = 0x01
    check_fp8(up, s, codes, s, x, "zero up", np.full(x.shape, half))
    up2 = codes.copy()
    up2[0, 3] = 0x02
    with pytest.raises(AssertionError):
        check_fp8(up2, s, codes, s, x, "two steps from zero", np.full(x.shape, half))
    crossed = codes.copy()
    crossed[0, 3] = 0x81                                   # -2**-9: across zero
    with pytest.raises(AssertionError):
        check_fp8(crossed, s, codes, s, x, "across zero", np.full(x.shape, half))


def test_small_values_take_the_error_of_their_terms():
    """A value near the subnormal codes pooled from large terms: its float32 error
    follows the terms (mag), not its own size, so a flip 2e-4 of its size from the
    midpoint is accepted with mag and refused without."""
    mid = (GRID[9] + GRID[10]) / 2                       # 9 and 10 x 2**-9
    x = row_with_value(mid * (1 + 2 * EPS_POOL))
    codes, s, _ = quantize_e4m3_rows(x)
    assert e4m3_decode(codes[0, 3]) == GRID[10]
    low = codes.copy()
    low[0, 3] -= 1
    with pytest.raises(AssertionError):
        check_fp8(low, s, codes, s, x, "no mag")
    check_fp8(low, s, codes, s, x, "with mag", np.full(x.shape, 1.0))


def test_scales_must_agree():
    x = row_with_value(GRID[50])
    codes, s, _ = quantize_e4m3_rows(x)
    with pytest.raises(AssertionError):
        check_fp8(codes, s * (1 + 1e-5), codes, s, x, "scale")


def test_pool_magnitude_bounds_the_pooled_value():
    """|pooled x| <= sum_t alpha_t |x_t|, with equality when every token agrees in sign."""
    from oracle import gated_pool
    rng = np.random.default_rng(3)
    K = rng.standard_normal((128, 16, 128))
    V = rng.standard_normal((128, 16, 128))
    W = rng.standard_normal((16, 128)) * 0.02
    hk, hv = gated_pool(K, V, W, rounded=False)
    mk, mv = pool_magnitude(K, V, W)
    assert np.all(np.abs(hk) <= mk * (1 + 1e-12)) and np.all(np.abs(hv) <= mv * (1 + 1e-12))
    hk2, _ = gated_pool(np.abs(K), V, W, rounded=False)
    mk2, _ = pool_magnitude(np.abs(K), V, W)
    np.testing.assert_allclose(hk2, mk2, rtol=1e-12)
