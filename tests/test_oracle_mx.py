"""Pins for the MXFP4 oracle (CPU only): E8M0 closed form, the pages' 4.25 bits per element,
the shared-exponent rule against brute force, nearest-grid rounding against an exhaustive
search, power-of-two equivariance, error bounds and stochastic rounding."""
import numpy as np
import pytest

import oracle
import workloads


def test_e8m0_closed_form():
    c = np.arange(255)
    assert np.array_equal(oracle.e8m0_decode(c), 2.0 ** (c.astype(np.float64) - 127))
    assert np.isnan(oracle.e8m0_decode([255])[0])


def test_bits_per_element_is_four_and_a_quarter():
    # the explainer's storage comparison: MXFP4 costs 4.25 bits per element
    x = workloads.bf16_bits_to_f32(workloads.normal_bf16((64, 256), 71))
    codes, scales = oracle.quantize_mxfp4(x)
    assert (codes.nbytes + scales.nbytes) * 8 == 4.25 * x.size


def test_shared_exponent_brute_force():
    # smallest e with amax / 2^e < 8, i.e. the largest element lands in [4, 8)
    rng = np.random.default_rng(3)
    a = np.concatenate([np.ldexp(rng.uniform(1, 2, 4000), rng.integers(-140, 127, 4000)),
                        [2.0 ** -149, 4.0, 7.999, 8.0, 6.0, 3.4e38]]).astype(np.float32)
    got = oracle.mx_shared_exponent(a)
    for v, e in zip(a.astype(np.float64), got):
        want = next(k for k in range(-300, 300) if v / 2.0 ** k < 8.0)
        assert e == max(-127, min(127, want)), (v, e, want)
    assert oracle.mx_shared_exponent([0.0])[0] == -127


def test_rounding_is_nearest_grid_point_exhaustive():
    # every element code against an argmin over the 15 E2M1 values in the scaled domain
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((32, 64)) * np.ldexp(1.0, rng.integers(-8, 8, (32, 1)))).astype(np.float32)
    codes, scales = oracle.quantize_mxfp4(x)
    c = oracle.unpack_nibbles(codes)
    e = scales.astype(np.int64) - 127
    for r in range(32):
        for k in range(64):
            y = float(x[r, k]) / 2.0 ** e[r, k // 32]
            d = np.abs(grid - min(abs(y), 6.0))
            best = np.flatnonzero(d == d.min())
            idx = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
            assert (c[r, k] & 7) == idx and (c[r, k] >> 3) == (1 if np.signbit(x[r, k]) else 0)


def test_block_max_encodes_as_four_or_six_and_error_bound():
    x = workloads.bf16_bits_to_f32(workloads.with_outliers_bf16((128, 512), 72))
    codes, scales = oracle.quantize_mxfp4(x)
    xh = oracle.dequantize_mxfp4(codes, scales)
    c = oracle.unpack_nibbles(codes).reshape(128, 16, 32)
    xb = np.abs(x).reshape(128, 16, 32)
    top = np.take_along_axis(c & 7, xb.argmax(axis=2)[:, :, None], axis=2)
    assert np.all((top == 6) | (top == 7))                      # magnitudes 4 or 6
    X = np.repeat(oracle.e8m0_decode(scales), 32, axis=1)
    # within half a grid gap (<= 1 in the scaled domain) unless saturated (|x|/X in (6, 8))
    err = np.abs(x - xh) / X
    sat = np.abs(x) / X > 6
    assert np.all(err[~sat] <= 1.0) and np.all(err[sat] < 2.0)


def test_power_of_two_equivariance():
    x = workloads.bf16_bits_to_f32(workloads.normal_bf16((16, 128), 73))
    c0, s0 = oracle.quantize_mxfp4(x)
    for k in (-20, -1, 3, 40):
        c1, s1 = oracle.quantize_mxfp4(np.ldexp(x, k).astype(np.float32))
        assert np.array_equal(c0, c1) and np.array_equal(s1.astype(int), s0.astype(int) + k)


def test_zero_and_tiny_blocks():
    x = np.zeros((2, 64), np.float32)
    x[1, 32:] = 2.0 ** -140
    x[1, 33] = -0.0
    codes, scales = oracle.quantize_mxfp4(x)
    assert list(scales[0]) == [0, 0] and scales[1, 1] == 0        # clamped to 2^-127
    c = oracle.unpack_nibbles(codes)
    assert np.all(c[0] == 0) and c[1, 33] == 8 and np.all(c[1, 32:] & 7 == 0)


def test_stochastic_rounding_unbiased_and_on_grid():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((1, 64)) * 3).astype(np.float32)
    c, s = oracle.quantize_mxfp4(x)
    on = oracle.dequantize_mxfp4(c, s).astype(np.float32)
    c2, s2 = oracle.quantize_mxfp4(on, "sr", seed=9, offset=1)
    assert np.array_equal(c2, c)                                   # grid values are kept
    acc = np.zeros(64)
    n = 2048
    for off in range(n):
        cs, ss = oracle.quantize_mxfp4(x, "sr", seed=11, offset=off)
        acc += oracle.dequantize_mxfp4(cs, ss)[0]
    X = oracle.e8m0_decode(s)[0].repeat(32)
    gap = np.where(np.abs(x[0]) / X < 2, 0.5, np.where(np.abs(x[0]) / X < 4, 1.0, 2.0)) * X
    sat = np.abs(x[0]) / X > 6                                      # clipped to 6 (R10), no bias claim
    assert sat.any() and np.all(np.abs(acc / n)[sat] == 6 * X[sat])
    assert np.all((np.abs(acc / n - x[0]) <= gap / 256 + 4 * gap / np.sqrt(n))[~sat])


def test_rejects_ragged_columns():
    with pytest.raises(ValueError):
        oracle.quantize_mxfp4(np.zeros((2, 48), np.float32))
