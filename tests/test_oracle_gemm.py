"""Pins for the oracle's reference GEMM and dequantization (CPU only)."""
from fractions import Fraction

import numpy as np
import torch

import oracle
import workloads


def _quant_pair(seed=0):
    a_bits, w_bits = workloads.tiny()
    a = workloads.bf16_bits_to_f32(a_bits)
    w = workloads.bf16_bits_to_f32(w_bits)
    qa = oracle.quantize_1x16(a)
    qw = oracle.quantize_16x16(w)
    return oracle.dequantize(*qa), oracle.dequantize(*qw)


def test_dequantize_exhaustive_code_scale_pairs():
    # x_hat = e2m1 * e4m3 * s_dec checked against float16 (E2M1 embedding) and torch's
    # float8_e4m3fn decode, for every (code, scale) pair.
    codes = np.arange(16, dtype=np.uint8)
    e2m1 = (np.array([(int(c) & 7) << 9 for c in codes], np.uint16).view(np.float16)
            .astype(np.float64) * 2.0 ** 14 * np.where(codes & 8, -1.0, 1.0))
    e4m3 = (torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
            .to(torch.float32).numpy().astype(np.float64))
    s_dec = np.float32(0.37)
    for s in range(0x7F):
        packed = np.array([[c | (c << 4) for c in codes] * 1], np.uint8)    # 32 elements
        scales = np.full((1, 2), s, np.uint8)
        got = oracle.dequantize(packed, scales, [s_dec])
        ref = np.repeat(e2m1, 2) * e4m3[s] * float(s_dec)
        assert np.array_equal(got[0], ref)


def test_fp64_gemm_matches_exact_rationals():
    ah, bh = _quant_pair()
    d = oracle.gemm_fp64(ah, bh)
    rng = np.random.default_rng(0)
    for _ in range(12):
        m, n = rng.integers(0, 256, 2)
        exact = sum(Fraction(float(ah[m, k])) * Fraction(float(bh[n, k])) for k in range(256))
        assert abs(Fraction(float(d[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 80)


def test_one_hot_operand_selects_columns():
    ah, _ = _quant_pair()
    eye = np.eye(256)
    assert np.array_equal(oracle.gemm_fp64(ah, eye[:8]), ah[:, :8])


def test_bound_is_scaled_abs_product():
    ah, bh = _quant_pair()
    b = oracle.gemm_bound(ah, bh)
    d = oracle.gemm_fp64(ah, bh)
    assert np.all(b >= 0) and np.all(np.abs(d) <= b / 1e-5 * (1 + 1e-12))


def test_grouped_equals_separate():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((40, 32))
    b = rng.standard_normal((3 * 8, 32))
    off = np.array([0, 10, 10, 40])
    d = oracle.grouped_gemm_fp64(a, b, off, 8)
    assert np.array_equal(d[0:10], a[0:10] @ b[0:8].T)
    assert np.array_equal(d[10:40], a[10:40] @ b[16:24].T)


def test_k_grouped_blocks_add_up_to_the_whole_contraction():
    # summing the group blocks over g gives the ungrouped product over the covered columns;
    # the first group (columns before 5) and an empty group contribute their own blocks
    rng = np.random.default_rng(2)
    a = rng.standard_normal((6, 70))
    b = rng.standard_normal((4, 70))
    off = np.array([5, 21, 21, 64, 70])
    d = oracle.grouped_gemm_k_fp64(a, b, off).reshape(4, 6, 4)
    assert np.allclose(d.sum(axis=0), a[:, 5:] @ b[:, 5:].T, rtol=1e-12, atol=1e-12)
    assert np.all(d[1] == 0.0)


def test_k_grouped_exact_on_small_integers():
    # integer operands: every partial sum is exact in binary64, so each block equals the
    # exact integer dot product written out term by term
    rng = np.random.default_rng(3)
    a = rng.integers(-8, 9, (3, 40)).astype(np.float64)
    b = rng.integers(-8, 9, (2, 40)).astype(np.float64)
    off = [0, 16, 40]
    d = oracle.grouped_gemm_k_fp64(a, b, off)
    for g in range(2):
        for i in range(3):
            for j in range(2):
                want = 0
                for k in range(off[g], off[g + 1]):
                    want += int(a[i, k]) * int(b[j, k])
                assert d[g * 3 + i, j] == want
    bound = oracle.grouped_gemm_k_bound(a, b, off)
    assert np.all(bound[3:] == 1e-5 * (np.abs(a[:, 16:]) @ np.abs(b[:, 16:]).T))



def test_round_bf16_matches_torch_cast():
    # library routine: torch's float32 -> bfloat16 conversion (nearest, ties to even)
    rng = np.random.default_rng(5)
    e = rng.integers(-149, 128, 20000)
    x = (rng.uniform(1, 2, 20000) * 2.0 ** e).astype(np.float32) * rng.choice([-1, 1], 20000)
    u = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    ties = np.concatenate([u | 0x8000, u | 0x7FFF, u | 0x8001, u]).view(np.float32)
    x = np.concatenate([x[np.isfinite(x)], ties[np.isfinite(ties)]])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.round_bf16(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_round_bf16_ties_to_even_closed_form():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to the even significand (1);
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -20],
                 np.float32)
    assert list(oracle.round_bf16(x)) == [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7]


def test_bf16_bound_covers_worst_fp32_error_then_rounding():
    # a GPU result within the FP32 bound, pushed to its extremes, then rounded to BF16 stays
    # within the BF16 bound; a one-hot product (exact in FP32 and BF16) is covered too
    ah, bh = _quant_pair()
    d = oracle.gemm_fp64(ah, bh)
    s = oracle.gemm_bound(ah, bh)
    b16 = oracle.gemm_bf16_bound(ah, bh)
    for sign in (-1.0, 1.0):
        d32 = (d + sign * s).astype(np.float32)
        assert np.all(np.abs(oracle.round_bf16(d32).astype(np.float64) - d) <= b16)
    eye = np.eye(256)[:8]
    assert np.all(oracle.round_bf16(oracle.gemm_fp64(ah, eye).astype(np.float32)) == oracle.round_bf16(ah[:, :8].astype(np.float32)))
    # the bound is not loose by orders of magnitude: at most 2^-7 relative above the FP32 one
    assert np.all(b16 <= s + 2.0 ** -7 * (np.abs(d) + s) + 2.0 ** -134)


def test_accumulate_exact_on_small_integers():
    rng = np.random.default_rng(9)
    a = rng.integers(-6, 7, (5, 32)).astype(np.float64)
    b = rng.integers(-6, 7, (4, 32)).astype(np.float64)
    d_old = rng.integers(-1000, 1000, (5, 4)).astype(np.float64)
    want = np.array([[int(d_old[m, n]) + sum(int(a[m, k]) * int(b[n, k]) for k in range(32)) for n in range(4)]
                     for m in range(5)], np.float64)
    assert np.array_equal(oracle.gemm_accumulate_fp64(d_old, a, b), want)
    # one binary32 rounding of the sum stays inside the accumulate bound
    d32 = (oracle.gemm_accumulate_fp64(d_old, a, b) * (1 + 2.0 ** -24)).astype(np.float32)
    assert np.all(np.abs(d32 - want) <= oracle.gemm_accumulate_bound(d_old, a, b))
