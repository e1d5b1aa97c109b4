"""Pins for the oracle's random Hadamard transform (CPU only).

The pages say the transform multiplies the wgrad inputs by a random Hadamard matrix and is
undone analytically. Pins: the butterfly's matrix equals the Kronecker power of H2 (numpy),
H H^T = 16 I, the rounded output against exact rational arithmetic (narrow blocks) and
against math.fsum's exact summation for blocks of any exponent spread (BF16 and FP32 inputs,
hand-made corner blocks), a worked wide-spread block whose correct rounding differs from a
binary64 evaluation, signed zeros, overflow, exact undo, Parseval, and invariance of the
wgrad GEMM when both operands are transformed."""
import math
from fractions import Fraction

import numpy as np

import oracle
import workloads


def _bf16(shape, seed, std=1.0):
    return workloads.bf16_bits_to_f32(workloads.normal_bf16(shape, seed, std))


def _fraction_to_f32(q: Fraction) -> np.float32:
    """Correctly rounded (nearest-even) binary32 of an exact rational, by integer arithmetic."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    m = q / ulp
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return np.float32(sign * float(lo * ulp))


def test_butterfly_is_sylvester_kronecker_power():
    h2 = np.array([[1.0, 1.0], [1.0, -1.0]])
    h16 = np.kron(h2, np.kron(h2, np.kron(h2, h2)))
    assert np.array_equal(oracle.hadamard_matrix_from_butterfly(), h16)


def test_hadamard_orthogonality():
    h = oracle.hadamard_matrix_from_butterfly()
    assert np.array_equal(h @ h.T, 16 * np.eye(16))


def test_rounded_output_equals_exact_rational():
    x = _bf16((64, 8), 3)
    x[5, 2] *= 50.0
    for mask in (0, 0xFFFF, 0x6E04, 0x8001):
        y = oracle.rht_columnwise(x, mask)
        h = oracle.hadamard_matrix_from_butterfly().astype(int)
        sig = [(-1 if (mask >> j) & 1 else 1) for j in range(16)]
        for c in range(x.shape[1]):
            for t in range(x.shape[0] // 16):
                v = [Fraction(float(x[16 * t + j, c])) for j in range(16)]
                for i in range(16):
                    s = sum(Fraction(int(h[i, j]) * sig[j]) * v[j] for j in range(16)) / 4
                    assert y[c, 16 * t + i] == _fraction_to_f32(s)


def test_undo_restores_input_exactly():
    x = _bf16((128, 16), 5)
    mask = workloads.wgrad_sign_mask()
    y64 = oracle.rht_columnwise_f64(x, mask)                 # [cols, tokens]
    h = oracle.hadamard_matrix_from_butterfly()
    sig = np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(16)])
    blocks = y64.reshape(16, -1, 16)                          # [col, tblock, 16]
    back = 0.25 * np.einsum("j,ji,cti->ctj", sig, h, blocks)  # Q^T = 1/4 D H^T, H^T = H
    assert np.array_equal(back.reshape(16, -1).T, x.astype(np.float64))
    assert np.allclose((y64 ** 2).sum(axis=1), (x.astype(np.float64) ** 2).sum(axis=0), rtol=1e-14)


def test_unit_vector_spreads_evenly():
    x = np.zeros((16, 1), np.float32)
    x[0, 0] = 1.0
    for mask in (0, 1):
        y = oracle.rht_columnwise(x, mask)
        s0 = -1.0 if mask & 1 else 1.0
        assert np.all(y == np.float32(0.25 * s0))


def test_wgrad_gemm_invariant_under_shared_transform():
    dy = _bf16((64, 24), 7, std=1e-3)
    x = _bf16((64, 40), 8)
    mask = 0x6E04
    ref = dy.astype(np.float64).T @ x.astype(np.float64)
    got = oracle.rht_columnwise_f64(dy, mask) @ oracle.rht_columnwise_f64(x, mask).T
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_transform_spreads_a_spike_over_its_block():
    # The pages' point of the rotation: an outlier no longer dominates its block. With one
    # spike of 50 sigma among Gaussian entries, the block's max/RMS ratio drops from ~4 (a
    # lone spike in 16 entries) to near 1 after the transform; energy is preserved.
    rng = np.random.default_rng(4)
    x = rng.standard_normal((16 * 64, 1)).astype(np.float32)
    x[np.arange(64) * 16 + rng.integers(0, 16, 64), 0] = 50.0
    y = oracle.rht_columnwise_f64(x, workloads.wgrad_sign_mask()).reshape(64, 16)
    v = x.astype(np.float64).reshape(64, 16)

    def crest(b):
        return np.abs(b).max(axis=1) / np.sqrt((b ** 2).mean(axis=1))

    assert np.all(crest(y) < 0.5 * crest(v))
    assert np.allclose((y ** 2).sum(axis=1), (v ** 2).sum(axis=1), rtol=1e-13)


def test_rht_quantize_column_subset():
    x = _bf16((64, 48), 9)
    mask = 0x1234
    full = oracle.rht_quantize(x, mask, "sr", seed=3, offset=2)
    A = oracle.amax(oracle.rht_columnwise(x, mask))
    cols = np.array([0, 7, 47])
    sub = oracle.rht_quantize(x[:, cols], mask, "sr", seed=3, offset=2, amax_vals=A, col_ids=cols)
    assert np.array_equal(sub[0], full[0][cols]) and np.array_equal(sub[1], full[1][cols])


def test_rht_quantize_segments_rn_equal_separate_token_ranges():
    # each token range is transformed block by block (blocks never cross a range boundary)
    # and quantized with its own tensor scale: with nearest rounding it is the plain
    # transform-and-quantize of its own tokens
    x = _bf16((96, 40), 10)
    mask = workloads.wgrad_sign_mask()
    seg = [0, 32, 32, 96]
    codes, scales, s_dec = oracle.rht_quantize_segments(x, mask, seg)
    for g in range(3):
        lo, hi = seg[g], seg[g + 1]
        if hi == lo:
            assert s_dec[g] == 1.0
            continue
        c, s, sd = oracle.rht_quantize(x[lo:hi], mask)
        assert np.array_equal(codes[:, lo // 2:hi // 2], c)
        assert np.array_equal(scales[:, lo // 16:hi // 16], s) and s_dec[g] == sd[0]


def test_rowwise_transform_is_the_block_matrix_on_each_row():
    # each row's 16-blocks times (1/4 H16 D)^T, against the explicit matrix product in
    # binary64 (exact for these values) rounded once to float32
    x = _bf16((8, 48), 21)
    mask = 0x6E04
    H = oracle.hadamard_matrix_from_butterfly()
    T = 0.25 * H @ np.diag(oracle.hadamard.sign_vector(mask))
    want = (x.astype(np.float64).reshape(8, 3, 16) @ T.T).reshape(8, 48).astype(np.float32)
    assert np.array_equal(oracle.rht_rowwise(x, mask), want)


def test_dgrad_gemm_invariant_under_rowwise_and_columnwise_transforms():
    # R23: (dY Q^T) against (W^T Q^T) contracts to dY W: the rowwise transform of dY and the
    # columnwise (along N) transform of W cancel, with the same mask
    dy = _bf16((32, 64), 22, std=1e-3)
    w = _bf16((64, 48), 23, std=0.02)          # [N, K]
    mask = 0x1234
    ref = dy.astype(np.float64) @ w.astype(np.float64)
    a = oracle.rht_columnwise_f64(np.ascontiguousarray(dy.T), mask)                # [M, N] rowwise, exact
    b = oracle.rht_columnwise_f64(w, mask)                                         # [K, N]
    assert np.allclose(a @ b.T, ref, rtol=1e-12, atol=1e-18)


def test_rowwise_quantize_is_quantize_of_the_transformed_rows():
    x = _bf16((16, 64), 24)
    q = oracle.rht_rowwise_quantize(x, 0x00FF, "sr", seed=3, offset=9)
    y = oracle.rht_rowwise(x, 0x00FF)
    r = oracle.quantize_1x16(y, "sr", seed=3, offset=9)
    for u, v in zip(q, r):
        assert np.array_equal(u, v)
    # the transformed block's largest element maps near the grid's top, as any 1x16 block
    assert oracle.amax(y)[0] > 0


def _rn32_of_exact_sum(terms) -> np.float32:
    """binary32 nearest-even of the exact sum of binary64 terms, built on math.fsum (exact
    summation, correctly rounded to binary64) instead of rational arithmetic: s = fsum(terms)
    is the sum rounded to binary64 and r = fsum(terms + [-s]) carries the sign of what that
    rounding dropped. Rounding s once more to binary32 is correct unless s is exactly halfway
    between two binary32 values; then r decides (r = 0: a true tie, nearest-even)."""
    s = math.fsum(terms)
    if s == 0.0:
        return np.float32(0.0)              # the terms are multiples of 2^-151: exact zero
    r = math.fsum(list(terms) + [-s])
    a = np.float32(s)
    if not np.isfinite(a) or float(a) == s:
        return a
    b = np.nextafter(a, np.float32(np.inf) if s > float(a) else np.float32(-np.inf))
    if (float(a) + float(b)) / 2 != s or r == 0.0:
        return a
    hi, lo = (a, b) if a > b else (b, a)
    return hi if r > 0 else lo


def _reference(x, mask):
    """y[c, 16t+i] from _rn32_of_exact_sum over the 16 terms H[i][j] sigma_j x[16t+j, c] / 4."""
    x = np.asarray(x, np.float32)
    h = oracle.hadamard_matrix_from_butterfly()
    sig = [(-1.0 if (mask >> j) & 1 else 1.0) for j in range(16)]
    out = np.empty((x.shape[1], x.shape[0]), np.float32)
    for c in range(x.shape[1]):
        for t in range(x.shape[0] // 16):
            v = [float(x[16 * t + j, c]) for j in range(16)]
            for i in range(16):
                out[c, 16 * t + i] = _rn32_of_exact_sum([h[i, j] * sig[j] * v[j] / 4 for j in range(16)])
    return out


def _same_bits(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


def test_tie_broken_by_a_far_term_rounds_up():
    # the column (1, 2^-24, 2^-70, 0, ...) with no sign flips: y_0 = (1 + 2^-24 + 2^-70) / 4 =
    # 2^-2 + 2^-26 + 2^-72. binary32's spacing above 2^-2 is 2^-25, so 2^-2 + 2^-26 is a tie
    # that the 2^-72 term breaks upwards: 2^-2 + 2^-25. A binary64 sum drops 2^-72 and then
    # rounds the tie to even (2^-2). Outputs with H[i][2] = -1 sit just below the tie (2^-2);
    # odd outputs are 2^-2 - 2^-26 (exact below 2^-2) minus or plus 2^-72, which rounds away.
    x = np.zeros((16, 1), np.float32)
    x[0:3, 0] = [1.0, 2.0 ** -24, 2.0 ** -70]
    y = oracle.rht_columnwise(x, 0)[0]
    want = np.array([0.25 + 2.0 ** -25 if i % 4 == 0 else 0.25 if i % 2 == 0 else 0.25 - 2.0 ** -26
                     for i in range(16)], np.float32)
    assert _same_bits(y, want)
    assert float(np.float32(np.float64(0.25) + 2.0 ** -26)) == 0.25       # the binary64 route


def test_any_exponent_spread_equals_exact_sum_bf16():
    x = workloads.bf16_bits_to_f32(workloads.exponent_spread_bf16(64, 24, 31))
    for mask in (0, 0x6E04, 0xFFFF):
        assert _same_bits(oracle.rht_columnwise(x, mask), _reference(x, mask))


def test_any_exponent_spread_equals_exact_sum_fp32():
    x = workloads.exponent_spread_f32(64, 24, 32)
    for mask in (0, 0x8001, 0x6E04):
        assert _same_bits(oracle.rht_columnwise(x, mask), _reference(x, mask))


def test_corner_blocks_equal_exact_sum():
    x = workloads.bf16_bits_to_f32(workloads.hadamard_edge_blocks_bf16())
    for mask in (0, 0x6E04, 0xFFFF):
        with np.errstate(over="ignore"):
            ref = _reference(x, mask)
        assert _same_bits(oracle.rht_columnwise(x, mask), ref)


def test_zero_sums_are_positive_zero():
    # all-zero blocks (with -0 inputs) and blocks whose terms cancel give +0 for every mask
    x = np.zeros((48, 1), np.float32)
    x[0:16:3, 0] = -0.0
    x[16, 0], x[17, 0] = 1.0, 1.0                       # outputs with H[i][1] = -1 cancel
    x[32:48, 0] = -0.0
    for mask in (0, 1, 0x8000, 0xFFFF, 0x6E04):
        y = oracle.rht_columnwise(x, mask)[0]
        zero = y == 0
        assert zero[:16].all() and zero[32:].all() and zero[16:32].sum() == 8
        assert not np.signbit(y[zero]).any()


def test_underflow_keeps_the_sign():
    # one FP32 subnormal 2^-149: every output is +-2^-151, which rounds to a zero carrying the
    # sign of H[i][0] * sigma_0 * v = sigma_0 * v
    for v in (2.0 ** -149, -(2.0 ** -149)):
        x = np.zeros((16, 1), np.float32)
        x[0, 0] = v
        for mask in (0, 1):
            y = oracle.rht_columnwise(x, mask)[0]
            neg = (v < 0) != bool(mask & 1)
            assert np.all(y == 0) and np.all(np.signbit(y) == neg)
    # the same next to terms 2^149 times larger that cancel in the odd outputs (a block far
    # outside binary64's exact range): those are +-2^-151 again, H[i][2] = (-1)^popcount(i & 2)
    for v in (2.0 ** -149, -(2.0 ** -149)):
        x = np.zeros((16, 1), np.float32)
        x[0:3, 0] = [1.0, 1.0, v]
        y = oracle.rht_columnwise(x, 0)[0]
        for i in range(1, 16, 2):
            neg = (v < 0) != bool(i & 2)
            assert y[i] == 0 and np.signbit(y[i]) == neg


def test_sum_beyond_binary32_range_is_infinite():
    big = np.float32(workloads.bf16_bits_to_f32(np.array([0x7F7F], np.uint16))[0])
    x = np.full((16, 1), big, np.float32)
    with np.errstate(over="ignore"):
        y = oracle.rht_columnwise(x, 0)[0]
    assert y[0] == np.inf and np.all(y[1:] == 0)        # 16 * big / 4 > FLT_MAX


def test_binary64_values_refuse_blocks_outside_the_exact_range():
    x = np.zeros((16, 1), np.float32)
    x[0:3, 0] = [1.0, 2.0 ** -24, 2.0 ** -70]
    try:
        oracle.rht_columnwise_f64(x, 0)
    except ValueError:
        return
    raise AssertionError("the binary64 values of a wide block were returned as exact")
