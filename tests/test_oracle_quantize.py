"""Pins for the oracle's two-level block quantization (CPU only).

The pages fix the storage cost (4.5 bits per element, a 3.56x shrink vs BF16), 16-element
blocks with an E4M3 scale plus one FP32 tensor scale, and 16x16 weight blocks that give
identical values in the forward and backward pass. Those facts, plus invariants of the
scale rule (power-of-two equivariance, block maxima landing on the largest element, tensor
amax landing on the largest scale), pin the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from oracle.formats import E2M1_GRID


def _x(shape, seed, std=1.0, outliers=True):
    bits = (workloads.with_outliers_bf16(shape, seed) if outliers
            else workloads.normal_bf16(shape, seed, std))
    return workloads.bf16_bits_to_f32(bits)


def test_storage_is_4p5_bits_per_element():
    x = _x((64, 256), 1)
    for codes, scales, _ in (oracle.quantize_1x16(x), oracle.quantize_16x16(x)):
        bits = 8 * (codes.nbytes + scales.nbytes)
        assert bits / x.size == 4.5
        assert round(16 / (bits / x.size), 2) == 3.56        # shrink vs BF16


def test_tensor_amax_maps_to_largest_element_and_scale():
    for seed in range(5):
        x = _x((32, 128), 10 + seed)
        A = float(np.abs(x).max())
        for codes, scales, s_dec in (oracle.quantize_1x16(x), oracle.quantize_16x16(x)):
            c = oracle.unpack_nibbles(codes)
            i, j = np.unravel_index(np.argmax(np.abs(x)), x.shape)
            assert c[i, j] & 7 == 7
            assert (c[i, j] >> 3) == int(x[i, j] < 0)
            assert scales[i, j // 16] == 0x7E
            assert np.float32(s_dec[0]) == np.float32(np.float32(A) / np.float32(2688))


def test_block_max_element_encodes_to_six():
    # For every block whose E4M3 scale is normal, the element attaining the block amax is +-6:
    # the scale is within 2^-4 of a_b/6 relative, so a_b * r_b lies in [5.65, 6.38].
    x = _x((128, 512), 21)
    for quant, blk_rows in ((oracle.quantize_1x16, 1), (oracle.quantize_16x16, 16)):
        codes, scales, _ = quant(x)
        c = oracle.unpack_nibbles(codes)
        R, C = x.shape
        for bi in range(0, R, blk_rows):
            for bj in range(0, C, 16):
                tile = np.abs(x[bi:bi + blk_rows, bj:bj + 16])
                if scales[bi, bj // 16] < 0x08:
                    continue
                ii, jj = np.unravel_index(np.argmax(tile), tile.shape)
                assert c[bi + ii, bj + jj] & 7 == 7


def test_power_of_two_equivariance():
    # Scaling the input by 2^k leaves codes and block scales unchanged and scales s_dec by
    # 2^k: catches a reversed encode/decode scale or a misplaced constant.
    x = _x((64, 256), 31)
    base = oracle.quantize_1x16(x)
    for k in (-20, -3, 5, 40):
        xs = (x * np.float32(2.0 ** k)).astype(np.float32)
        got = oracle.quantize_1x16(xs)
        assert np.array_equal(got[0], base[0]) and np.array_equal(got[1], base[1])
        assert got[2][0] == np.float32(base[2][0] * np.float32(2.0 ** k))


def test_dequantized_error_within_half_gap():
    x = _x((64, 512), 41)
    codes, scales, s_dec = oracle.quantize_1x16(x)
    xhat = oracle.dequantize(codes, scales, s_dec)
    s = np.repeat(oracle.e4m3_decode(scales), 16, axis=1)
    c = oracle.unpack_nibbles(codes)
    gap = np.where((c & 7) >= 6, 2.0, np.where((c & 7) >= 4, 1.0, 0.5))
    # rounding error in the element domain is at most half a gap (or the saturation at 6,
    # which is below half the top gap); tolerance covers the FP32 scale products.
    err = np.abs(xhat - x.astype(np.float64))
    bound = 0.5 * gap * s * float(s_dec[0]) * (1 + 1e-6) + 1e-30
    assert np.all(err <= bound)


def test_zero_tensor_and_tiny_blocks():
    x = np.zeros((16, 64), np.float32)
    x[3, 5] = -0.0
    codes, scales, s_dec = oracle.quantize_1x16(x)
    assert s_dec[0] == 1.0 and not scales.any()
    c = oracle.unpack_nibbles(codes)
    assert c[3, 5] == 8 and (c.sum() == 8)
    # A block far below the tensor amax gets scale 0 and signed-zero codes.
    y = np.zeros((1, 32), np.float32)
    y[0, 0] = 1e4
    y[0, 16:] = np.float32(1e-4) * np.sign(np.arange(16) - 7.5).astype(np.float32)
    codes, scales, _ = oracle.quantize_1x16(y)
    c = oracle.unpack_nibbles(codes)
    assert scales[0, 1] == 0
    assert np.array_equal(c[0, 16:], np.where(y[0, 16:] < 0, 8, 0))


def test_16x16_scale_shared_by_tile_rows():
    x = _x((64, 128), 51)
    _, scales, _ = oracle.quantize_16x16(x)
    for r0 in range(0, 64, 16):
        assert np.all(scales[r0:r0 + 16] == scales[r0])


def test_16x16_is_transpose_invariant():
    # The 2D weight blocks give the same values to the forward (W) and backward (W^T) GEMMs.
    for seed in range(3):
        w = _x((96, 160), 60 + seed)
        c, s, sd = oracle.quantize_16x16(w)
        ct, st, sdt = oracle.quantize_16x16(np.ascontiguousarray(w.T))
        assert np.array_equal(oracle.unpack_nibbles(ct), oracle.unpack_nibbles(c).T)
        assert np.array_equal(st[::16], s[::16].T)
        assert sd[0] == sdt[0]
        assert np.array_equal(oracle.dequantize(ct, st, sdt), oracle.dequantize(c, s, sd).T)


def test_row_subsets_match_full_tensor():
    x = _x((64, 128), 71)
    A = oracle.amax(x)
    rows = np.array([3, 17, 40, 63])
    for rnd in ("rn", "sr"):
        full = oracle.quantize_1x16(x, rnd, seed=99, offset=5)
        sub = oracle.quantize_1x16(x[rows], rnd, seed=99, offset=5, amax_vals=A, row_ids=rows)
        assert np.array_equal(sub[0], full[0][rows]) and np.array_equal(sub[1], full[1][rows])
    g = np.arange(32, 48)
    full = oracle.quantize_16x16(x)
    sub = oracle.quantize_16x16(x[g], amax_vals=A, row_ids=g)
    assert np.array_equal(sub[0], full[0][g]) and np.array_equal(sub[1], full[1][g])


def test_segments_equal_separate_tensors():
    x = _x((96, 64), 81)
    seg = np.array([0, 16, 16, 64, 96])          # includes an empty segment
    codes, scales, s_dec = oracle.quantize_1x16(x, segments=seg)
    assert s_dec.shape == (4,) and s_dec[1] == 1.0
    for g in range(4):
        lo, hi = seg[g], seg[g + 1]
        if hi == lo:
            continue
        c, s, sd = oracle.quantize_1x16(x[lo:hi])
        assert np.array_equal(codes[lo:hi], c) and np.array_equal(scales[lo:hi], s)
        assert s_dec[g] == sd[0]
    codes, scales, s_dec = oracle.quantize_16x16(x, segments=seg)
    for g in range(4):
        lo, hi = seg[g], seg[g + 1]
        if hi > lo:
            c, s, sd = oracle.quantize_16x16(x[lo:hi])
            assert np.array_equal(codes[lo:hi], c) and s_dec[g] == sd[0]


def test_sr_only_changes_rounding_direction():
    x = _x((32, 256), 91, std=1e-3, outliers=False)
    rn = oracle.quantize_1x16(x, "rn")
    sr = oracle.quantize_1x16(x, "sr", seed=1, offset=0)
    assert np.array_equal(rn[1], sr[1]) and rn[2][0] == sr[2][0]
    s = np.repeat(oracle.e4m3_decode(sr[1]), 16, axis=1)
    y = x.astype(np.float64) / (s * float(sr[2][0]))
    q = np.abs(oracle.e2m1_decode(oracle.unpack_nibbles(sr[0])))
    a = np.minimum(np.abs(y), 6)
    lo = np.array([E2M1_GRID[E2M1_GRID <= v * (1 - 1e-6)].max() if v > 0 else 0 for v in a.ravel()])
    assert np.all(q.ravel() >= lo - 1e-12)
    # a different offset changes some codes, the same offset reproduces them
    sr2 = oracle.quantize_1x16(x, "sr", seed=1, offset=0)
    sr3 = oracle.quantize_1x16(x, "sr", seed=1, offset=1)
    assert np.array_equal(sr[0], sr2[0]) and not np.array_equal(sr[0], sr3[0])


def test_sr_tensor_mean_is_unbiased():
    x = _x((16, 64), 95, outliers=False)
    acc = np.zeros(x.shape)
    n = 1024
    for off in range(n):
        c, s, sd = oracle.quantize_1x16(x, "sr", seed=7, offset=off)
        acc += oracle.dequantize(c, s, sd)
    mean = acc / n
    c, s, sd = oracle.quantize_1x16(x, "rn")
    unit = np.repeat(oracle.e4m3_decode(s), 16, axis=1) * float(sd[0])
    # Elements pushed past 6 by the nearest-rounded block scale saturate (a deterministic
    # clip, not a rounding decision); everywhere else |E - x| <= gap/256 (bias) + 5 sigma.
    inside = np.abs(x) / unit < 6.0 * (1 - 1e-6)
    assert inside.mean() > 0.9
    err = np.abs(mean - x)[inside]
    assert np.all(err <= unit[inside] * (2 / 256 + 5 * 1.0 / np.sqrt(n)))
    rn_err = np.abs(oracle.dequantize(c, s, sd) - x)[inside].mean()
    assert err.mean() < 0.25 * rn_err


@pytest.mark.parametrize("shape", [(16, 16), (48, 32)])
def test_fp32_input_path(shape):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(shape).astype(np.float32)
    c, s, sd = oracle.quantize_1x16(x)
    assert c.shape == (shape[0], shape[1] // 2) and s.shape == (shape[0], shape[1] // 16)


def test_column_segments_one_range_is_the_plain_quantization():
    x = _x((32, 96), 91)
    for rnd in ("rn", "sr"):
        got = oracle.quantize_1x16_colsegments(x, [0, 96], rnd, seed=4, offset=9)
        want = oracle.quantize_1x16(x, rnd, seed=4, offset=9)
        for g, w in zip(got, want):
            assert np.array_equal(np.asarray(g), np.asarray(w))


def test_column_segments_rn_are_separate_tensors():
    # with nearest rounding nothing depends on a block's position, so each column range is
    # the plain quantization of its own columns with its own tensor scale; an empty range
    # keeps the unit decode scale
    x = _x((24, 112), 92)
    seg = [0, 32, 32, 80, 112]
    codes, scales, s_dec = oracle.quantize_1x16_colsegments(x, seg)
    assert s_dec[1] == 1.0
    for g in range(4):
        lo, hi = seg[g], seg[g + 1]
        if hi == lo:
            continue
        c, s, sd = oracle.quantize_1x16(x[:, lo:hi])
        assert np.array_equal(codes[:, lo // 2:hi // 2], c)
        assert np.array_equal(scales[:, lo // 16:hi // 16], s)
        assert s_dec[g] == sd[0]


def test_column_segments_sr_use_whole_tensor_block_index():
    # giving every range the whole tensor's amax makes the result the plain SR quantization,
    # which numbers blocks over the whole row: the random bytes follow the global position
    x = _x((16, 80), 93)
    a = oracle.amax(x)[0]
    got = oracle.quantize_1x16_colsegments(x, [0, 16, 64, 80], "sr", seed=7, offset=1,
                                           amax_vals=[a, a, a])
    want = oracle.quantize_1x16(x, "sr", seed=7, offset=1)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_colsegments_row_subsets_equal_the_whole_tensor():
    # row subsets (with the full tensor's maxima) give the whole tensor's rows, stochastic
    # rounding included: the block index is the block's place in the whole tensor
    x = workloads.bf16_bits_to_f32(workloads.with_outliers_bf16((24, 96), 61))
    seg = [0, 32, 32, 96]
    full = oracle.quantize_1x16_colsegments(x, seg, "sr", seed=4, offset=9)
    rows = np.array([0, 5, 23])
    a = np.array([np.abs(x[:, seg[g]:seg[g + 1]]).max() if seg[g + 1] > seg[g] else 0.0 for g in range(3)], np.float32)
    sub = oracle.quantize_1x16_colsegments(x[rows], seg, "sr", seed=4, offset=9, amax_vals=a, row_ids=rows)
    assert np.array_equal(sub[0], full[0][rows]) and np.array_equal(sub[1], full[1][rows])
