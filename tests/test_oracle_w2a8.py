"""Pins of the W2A8 oracle (oracle/w2a8.py) against closed forms, rounding
bounds, special cases and brute force on tiny inputs.  CPU only."""

import numpy as np
import pytest

from oracle import w2a8


# ---------------------------------------------------------------------------
# activation codes
# ---------------------------------------------------------------------------


def test_activation_codes_round_half_to_even():
    # max |x| = 127 gives s = 1 exactly, so the codes are x rounded half to even
    x = np.array([0.5, 1.5, 2.5, -0.5, -2.5, 127.0, 3.49, -126.5], dtype=np.float32)
    q, s = w2a8.quantize_activations_absmax(x)
    assert s == np.float32(1.0)
    assert q.tolist() == [0, 2, 2, 0, -2, 127, 3, -126]
    assert q.dtype == np.int8


def test_activation_codes_unit_range():
    # max |x| = 1: s = 127; -0.5 * 127 = -63.5 rounds to the even -64
    x = np.array([1.0, -0.5, 0.25, 0.0, -1.0], dtype=np.float32)
    q, s = w2a8.quantize_activations_absmax(x)
    assert s == np.float32(127.0)
    assert q.tolist() == [127, -64, 32, 0, -127]


def test_activation_zero_vector():
    q, s = w2a8.quantize_activations_absmax(np.zeros(64, dtype=np.float32))
    assert np.all(q == 0)
    assert s == np.float32(127.0) / np.float32(1e-5)


def test_activation_codes_rounding_bound_and_range():
    rng = np.random.default_rng(5)
    for _ in range(20):
        x = (rng.standard_normal(1000) * rng.uniform(0.01, 100)).astype(np.float32)
        q, s = w2a8.quantize_activations_absmax(x)
        # each code is within half a step of x * s, the largest |x| maps to +-127
        err = np.abs(x.astype(np.float64) * np.float64(s) - q.astype(np.float64))
        assert err.max() <= 0.5 + 1e-4
        assert np.abs(q).max() == 127
        assert q[np.argmax(np.abs(x))] == np.sign(x[np.argmax(np.abs(x))]) * 127


def test_activation_codes_scale_invariant_under_powers_of_two():
    rng = np.random.default_rng(6)
    x = rng.standard_normal(300).astype(np.float32)
    q0, s0 = w2a8.quantize_activations_absmax(x)
    for c in (0.25, 2.0, 1024.0):
        q, s = w2a8.quantize_activations_absmax(x * np.float32(c))
        assert np.array_equal(q, q0)
        assert s == s0 / np.float32(c)


# ---------------------------------------------------------------------------
# ternary weights
# ---------------------------------------------------------------------------


def test_weight_codes_closed_forms():
    w = np.array([[0.5, -0.5, 0.1, 0.0],      # gamma 0.275: 1.82, -1.82, 0.36, 0 -> 1, -1, 0, 0
                  [3.0, -3.0, 3.0, -3.0],     # gamma 3: the signs
                  [0.0, 0.0, 0.0, 0.0],       # gamma 0: zeros (eps avoids 0/0)
                  [2.0, 1.0, 0.4, 0.6]])      # gamma 1: 2 -> clip 1, 1, 0.4 -> 0, 0.6 -> 1
    q, g = w2a8.quantize_weights_absmean(w, eps=0.0 + 1e-12)
    assert q.tolist() == [[1, -1, 0, 0], [1, -1, 1, -1], [0, 0, 0, 0], [1, 1, 0, 1]]
    assert np.allclose(g, [0.275, 3.0, 0.0, 1.0])


def test_weight_codes_are_ternary_and_rowwise():
    rng = np.random.default_rng(7)
    w = rng.standard_normal((12, 40)) * np.arange(1, 13)[:, None]   # rows of very different scale
    q, g = w2a8.quantize_weights_absmean(w)
    assert set(np.unique(q).tolist()) <= {-1, 0, 1}
    # scaling one row scales its gamma and leaves every code unchanged
    w2 = w.copy()
    w2[3] *= 8.0
    q2, g2 = w2a8.quantize_weights_absmean(w2)
    assert np.array_equal(q2, q)
    assert np.isclose(g2[3], 8 * g[3]) and np.allclose(np.delete(g2, 3), np.delete(g, 3))


# ---------------------------------------------------------------------------
# the product
# ---------------------------------------------------------------------------


def test_gemv_integer_sum_brute_force():
    rng = np.random.default_rng(8)
    rows, cols = 5, 23                      # rectangular: a transposed operand cannot pass
    codes = rng.integers(-1, 2, size=(rows, cols)).astype(np.int8)
    xq = rng.integers(-128, 128, size=cols).astype(np.int8)
    y = w2a8.w2a8_gemv(codes, np.ones(rows, np.float32), xq, np.float32(1.0))
    for r in range(rows):
        acc = 0
        for k in range(cols):
            acc += int(codes[r, k]) * int(xq[k])
        assert y[r] == np.float32(acc)


def test_gemv_extremes_and_signs():
    cols = 4096
    xq = np.full(cols, -128, dtype=np.int8)
    codes = np.stack([np.full(cols, 1), np.full(cols, -1), np.zeros(cols)]).astype(np.int8)
    y = w2a8.w2a8_gemv(codes, np.ones(3, np.float32), xq, np.float32(1.0))
    assert y.tolist() == [-128.0 * cols, 128.0 * cols, 0.0]


def test_linear_exact_on_representable_inputs():
    # x already on the code grid with s = 1 (max |x| = 127) and gamma a power
    # of two: the W2A8 result equals the float64 product gamma * Q @ x exactly
    rng = np.random.default_rng(9)
    rows, cols = 7, 96
    codes = rng.integers(-1, 2, size=(rows, cols)).astype(np.int8)
    x = rng.integers(-127, 128, size=cols).astype(np.float32)
    x[0] = 127.0
    gamma = np.float32(2.0) ** rng.integers(-6, 3, size=rows).astype(np.float32)
    y = w2a8.w2a8_linear(codes, gamma, x)
    ref = gamma.astype(np.float64) * (codes.astype(np.float64) @ x.astype(np.float64))
    assert np.array_equal(y.astype(np.float64), ref)


def test_linear_approximates_the_dequantised_product():
    # with the codes fixed, y differs from gamma * Q @ x only by the activation
    # rounding: |y - gamma Q x| <= gamma * sum|Q| * 0.5 / s (plus float32 slack)
    rng = np.random.default_rng(10)
    rows, cols = 16, 512
    w = rng.standard_normal((rows, cols))
    codes, gamma = w2a8.quantize_weights_absmean(w)
    x = rng.standard_normal(cols).astype(np.float32)
    _, s = w2a8.quantize_activations_absmax(x)
    y = w2a8.w2a8_linear(codes, gamma, x).astype(np.float64)
    exact = gamma.astype(np.float64) * (codes.astype(np.float64) @ x.astype(np.float64))
    bound = gamma.astype(np.float64) * np.abs(codes).sum(axis=1) * 0.5 / float(s)
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-5) + 1e-6 * np.abs(exact))
    # and the error is not trivially zero: the bound is what is being checked
    assert np.any(np.abs(y - exact) > 0)


def test_empty_vector():
    q, s = w2a8.quantize_activations_absmax(np.zeros(0, dtype=np.float32))
    assert q.size == 0
    y = w2a8.w2a8_gemv(np.zeros((3, 0), np.int8), np.ones(3, np.float32), q, s)
    assert y.tolist() == [0.0, 0.0, 0.0]


@pytest.mark.parametrize("bad", [np.nan, np.inf])
def test_nonfinite_input_is_not_silently_coded(bad):
    # a non-finite activation makes the scale 0 or NaN; the codes are then
    # meaningless, and the oracle must not report a finite, plausible result
    x = np.array([1.0, bad, 0.5], dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        q, s = w2a8.quantize_activations_absmax(x)
    assert not (np.isfinite(s) and s > 0 and np.all(np.abs(q) <= 127) and q[0] != 0)
