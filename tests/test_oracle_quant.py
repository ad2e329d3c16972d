"""Pins for code assignment and the least-squares scale (ResidualQuant,
newx.sg page, Abstract: INT2 residual codes with least-square scaling)."""
import itertools

import numpy as np
import pytest
import scipy.optimize

import oracle


def _levels(bits):
    off = oracle.level_offset(bits)
    return np.arange(2 ** bits) - off


def test_level_grids():
    np.testing.assert_array_equal(_levels(2), [-1.5, -0.5, 0.5, 1.5])
    np.testing.assert_array_equal(_levels(4), np.arange(-7.5, 8.0, 1.0))
    np.testing.assert_array_equal(_levels(3), [-3.5, -2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 3.5])
    np.testing.assert_array_equal(_levels(8), np.arange(-127.5, 128.0, 1.0))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_codes_are_nearest_level_per_element(bits):
    rng = np.random.default_rng(7)
    y = rng.standard_normal((400, 32)) * rng.uniform(0.01, 10, size=(400, 1))
    codes, s0 = oracle.assign_codes(y, bits)
    lev = _levels(bits)
    # exhaustive search over all levels at step s0
    dist = np.abs(y[..., None] - s0[:, None, None] * lev)
    best = dist.min(axis=-1)
    chosen = np.take_along_axis(dist, codes[..., None], axis=-1)[..., 0]
    np.testing.assert_allclose(chosen, best, rtol=0, atol=1e-12 * np.abs(y).max())


@pytest.mark.parametrize("bits,n", [(2, 1), (2, 3), (2, 6), (3, 2), (3, 4), (4, 2), (4, 3), (8, 1), (8, 2)])
def test_joint_search_equals_separable_choice(bits, n):
    """Over all code vectors of a tiny group, the one closest to y at step s0
    is the per-element choice (the grid is separable)."""
    rng = np.random.default_rng(100 + n)
    lev = _levels(bits)
    for _ in range(20):
        y = rng.standard_normal(n)
        codes, s0 = oracle.assign_codes(y[None], bits)
        best, best_err = None, np.inf
        for combo in itertools.product(range(2 ** bits), repeat=n):
            err = np.sum((y - s0[0] * lev[list(combo)]) ** 2)
            if err < best_err - 1e-15:
                best, best_err = combo, err
        np.testing.assert_array_equal(codes[0], best)


def test_threshold_ties_and_extremes():
    # m = 1.5 -> s0 = 1, so the INT2 thresholds sit at -1, 0, 1 exactly
    y = np.array([[1.5, 1.0, 0.0, -1.0, -1.5, 0.99, -0.01]])
    codes, s0 = oracle.assign_codes(y, 2)
    assert s0[0] == 1.0
    np.testing.assert_array_equal(codes[0], [3, 3, 2, 1, 0, 2, 1])
    # INT4: m = 7.5 -> s0 = 1, thresholds at the integers -7..7
    y4 = np.array([[7.5, -7.5, 0.0, 3.0, -3.0, 2.5]])
    c4, _ = oracle.assign_codes(y4, 4)
    np.testing.assert_array_equal(c4[0], [15, 0, 8, 11, 5, 10])
    # INT3: m = 3.5 -> s0 = 1, thresholds at -3..3
    y3 = np.array([[3.5, -3.5, 0.0, 1.0, -1.0, -0.5, 2.99]])
    c3, _ = oracle.assign_codes(y3, 3)
    np.testing.assert_array_equal(c3[0], [7, 0, 4, 5, 3, 3, 6])
    # INT8: m = 127.5 -> s0 = 1, thresholds at -127..127
    y8 = np.array([[127.5, -127.5, 0.0, -0.25, 126.9, -127.0]])
    c8, _ = oracle.assign_codes(y8, 8)
    np.testing.assert_array_equal(c8[0], [255, 0, 128, 127, 254, 1])


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_ls_scale_is_the_least_squares_minimum(bits):
    rng = np.random.default_rng(3)
    for _ in range(30):
        y = rng.standard_normal(6) * rng.uniform(0.1, 5)
        codes, s0 = oracle.assign_codes(y[None], bits)
        q = codes[0] - oracle.level_offset(bits)
        s = oracle.ls_scale(y, q)
        f = lambda t: np.sum((y - t * q) ** 2)  # noqa: E731
        res = scipy.optimize.minimize_scalar(f, bracket=(0.0, 2 * s0[0] + 1.0))
        assert abs(res.x - s) <= 1e-6 * max(1.0, abs(s))
        grid = np.linspace(0, 3 * s0[0], 20001)
        errs = ((y[None, :] - grid[:, None] * q[None, :]) ** 2).sum(axis=1)
        assert f(s) <= errs.min() + 1e-12
        # the LS fit is never worse than the absmax step it started from
        assert f(s) <= f(s0[0]) + 1e-15
        assert s > 0


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_zero_group(bits):
    codes, s = oracle.quantize_groups(np.zeros((3, 32)), bits)
    assert np.all(codes == 2 ** (bits - 1))
    assert np.all(s == 0.0)


def test_scale_storage_rounds_and_saturates():
    assert oracle.f64_to_f16(np.array([0.15]))[0] == 0x30CD
    assert oracle.f64_to_f16(np.array([1e6]))[0] == 0x7BFF  # 65504, not inf
    assert oracle.f16_to_f64(np.array([0x7BFF], dtype=np.uint16))[0] == 65504.0


def test_bf16_decoding_and_rounding():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.bf16_to_f64(bits), [1.0, -1.0, 3.140625, 0.0])
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even mantissa (1.0)
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6 -> even (1 + 2^-6)
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -30, -2.5])
    np.testing.assert_array_equal(oracle.f64_to_bf16(x), [0x3F80, 0x3F82, 0x3F81, 0xC020])


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_refits_never_raise_the_error_and_reach_a_fixed_point(bits):
    """Alternating the two least-squares half-steps (codes for a fixed scale,
    scale for fixed codes) cannot raise |y - s q|; after enough rounds the
    codes are the nearest levels at their own LS scale."""
    rng = np.random.default_rng(11 + bits)
    y = rng.standard_normal((500, 32)) * rng.uniform(0.1, 3.0, size=(500, 1))
    off = oracle.level_offset(bits)
    prev = None
    for k in range(6):
        c, s = oracle.quantize_groups(y, bits, refits=k)
        err = np.linalg.norm(y - s[:, None] * (c - off), axis=1)
        if prev is not None:
            assert np.all(err <= prev * (1 + 1e-12))
        prev = err
    c, s = oracle.quantize_groups(y, bits, refits=50)
    c2 = oracle.refit_codes(y, s, bits)
    np.testing.assert_array_equal(c2, c)
    # refits = 0 is the plain encoder
    c0, s0 = oracle.quantize_groups(y, bits)
    ca, sa = oracle.quantize_groups(y, bits, refits=0)
    np.testing.assert_array_equal(c0, ca)
    np.testing.assert_array_equal(s0, sa)


def test_refit_assignment_is_nearest_level_at_the_step():
    """refit_codes picks, per element, the grid level closest to y at step s
    (brute force over all levels; ties at a threshold go up)."""
    rng = np.random.default_rng(5)
    for bits in (2, 3, 4, 8):
        y = rng.standard_normal((200, 32))
        s = rng.uniform(0.2, 1.5, size=200) / 2 ** (bits - 2)
        c = oracle.refit_codes(y, s, bits)
        lev = (np.arange(2 ** bits) - oracle.level_offset(bits))[None, None, :] * s[:, None, None]
        best = np.argmin(np.abs(y[..., None] - lev), axis=-1)
        np.testing.assert_array_equal(c, best)


def test_refit_gain_on_gaussian_groups():
    """Quality sanity: on Gaussian groups one refit lowers the INT2 error by
    about a tenth, and the fixed point sits near 0.33 (Lloyd-style uniform-grid
    quantizer)."""
    rng = np.random.default_rng(0)
    y = rng.standard_normal((4000, 32))
    off = oracle.level_offset(2)
    e = []
    for k in (0, 1, 8):
        c, s = oracle.quantize_groups(y, 2, refits=k)
        e.append(np.linalg.norm(y - s[:, None] * (c - off)) / np.linalg.norm(y))
    assert 0.39 < e[0] < 0.42 and e[1] < 0.92 * e[0] and 0.32 < e[2] < 0.345
