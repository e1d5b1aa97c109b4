"""Pins for the oracle's E2M1 / E4M3 codecs and rounding rules (CPU only).

Each check compares the oracle with something other than itself: IEEE half precision from
numpy (E2M1 embeds exactly into float16 subnormals), torch's float8_e4m3fn cast, closed-form
rounding thresholds, and counting arguments for stochastic rounding."""
import numpy as np
import pytest
import torch

import oracle
from oracle.formats import E2M1_GRID


def _f32(v):
    return np.asarray(v, dtype=np.float32)


def test_e2m1_decode_matches_float16_embedding():
    # Bits (e1 e0 m) placed at float16 bits 11..9 give exactly e2m1 * 2^-14 (bias 1 vs 15,
    # with both subnormal ranges aligned), so numpy's float16 decodes E2M1 independently.
    for code in range(16):
        mag_bits = np.array([(code & 7) << 9], dtype=np.uint16)
        ref = float(mag_bits.view(np.float16)[0]) * 2.0 ** 14
        ref = -ref if code & 8 else ref
        got = float(oracle.e2m1_decode(code))
        assert got == ref and np.signbit(got) == bool(code & 8)
    assert list(E2M1_GRID) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _rn_closed_form(a):
    # Thresholds at the midpoints; ties go to the code with mantissa bit 0.
    a = np.asarray(a, dtype=np.float64)
    return ((a > 0.25).astype(int) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5)
            + (a >= 3.5) + (a > 5.0))


def test_e2m1_rn_thresholds_all_bf16_patterns():
    bits = np.arange(65536, dtype=np.uint32) << 16
    y = bits.view(np.float32)
    y = y[np.isfinite(y)]
    codes = oracle.e2m1_encode_rn(y)
    assert np.array_equal(codes & 7, _rn_closed_form(np.abs(y)))
    assert np.array_equal((codes >> 3) & 1, np.signbit(y).astype(np.uint8))


def test_e2m1_rn_midpoint_neighbours():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    vals = []
    for m in mids:
        m = np.float32(m)
        vals += [np.nextafter(m, np.float32(0)), m, np.nextafter(m, np.float32(10))]
    vals = _f32(vals + [0.0, 1e-30, 7.0, 1e30, np.inf])
    for s in (1.0, -1.0):
        y = vals * np.float32(s)
        codes = oracle.e2m1_encode_rn(y)
        assert np.array_equal(codes & 7, _rn_closed_form(np.abs(y)))


def test_e2m1_rn_roundtrip_and_negative_zero():
    for code in range(16):
        assert int(oracle.e2m1_encode_rn(_f32([oracle.e2m1_decode(code)]))[0]) == code
    assert int(oracle.e2m1_encode_rn(_f32([-0.1]))[0]) == 0x8


def test_e2m1_sr_counts_match_floor_rule():
    # For each value, count how many of the 256 bytes round up; the rule says floor(256*frac).
    rng = np.random.default_rng(7)
    y = _f32(np.concatenate([rng.uniform(0, 6.5, 3000), E2M1_GRID, [0.2, 5.999, 6.0, 9.0]]))
    a = np.minimum(y.astype(np.float64), 6.0)
    lo_v = np.array([E2M1_GRID[E2M1_GRID <= v].max() for v in a])
    hi_v = np.array([E2M1_GRID[E2M1_GRID >= v].min() for v in a])
    up_counts = np.zeros(y.size, dtype=np.int64)
    for rb in range(256):
        codes = oracle.e2m1_encode_sr(y, np.full(y.shape, rb, np.uint8))
        mag = E2M1_GRID[codes & 7]
        assert np.all((mag == lo_v) | (mag == hi_v))
        up_counts += (mag > a)
    gap = np.where(hi_v > lo_v, hi_v - lo_v, 1.0)
    expect = np.where(hi_v > lo_v, np.floor(256.0 * (a - lo_v) / gap), 0)
    assert np.array_equal(up_counts, expect.astype(np.int64))


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    got = oracle.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_e4m3_encode_matches_torch_cast_below_448():
    vals = oracle.e4m3_decode(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(3)
    t = np.concatenate([vals, mids, rng.uniform(0, 448, 20000),
                        2.0 ** rng.uniform(-14, 8.8, 20000)]).astype(np.float32)
    t = np.concatenate([t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(448))])
    t = t[(t >= 0) & (t <= 448)]
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(t), ref)


def test_e4m3_saturation_and_flush():
    t = _f32([448.0, 449.0, 464.0, 480.0, 1e10, np.inf])
    assert np.all(oracle.e4m3_encode(t) == 0x7E)
    assert int(oracle.e4m3_encode(_f32([2.0 ** -10]))[0]) == 0        # tie -> even (zero)
    assert int(oracle.e4m3_encode(_f32([np.nextafter(np.float32(2.0 ** -10), 1)]))[0]) == 1
    assert int(oracle.e4m3_encode(_f32([1e-30]))[0]) == 0
    for c in range(0x7F):
        assert int(oracle.e4m3_encode(_f32([oracle.e4m3_decode(c)]))[0]) == c


@pytest.mark.parametrize("value", [0.1, 0.3, 0.7, 1.1, 2.2, 3.3, 4.4, 5.5])
def test_sr_mean_converges(value):
    # Unbiased in expectation up to the 8-bit resolution: |E[q] - a| < gap/256.
    n = 1 << 16
    r = np.random.default_rng(11).integers(0, 256, n).astype(np.uint8)
    codes = oracle.e2m1_encode_sr(_f32(np.full(n, value)), r)
    q = oracle.e2m1_decode(codes)
    a = np.float64(np.float32(value))
    lo = E2M1_GRID[E2M1_GRID <= a].max()
    hi = E2M1_GRID[E2M1_GRID >= a].min()
    gap = hi - lo
    sigma = gap * 0.5 / np.sqrt(n)
    assert abs(q.mean() - a) <= gap / 256 + 4 * sigma
