"""Random Hadamard transform of the wgrad operands (oracle; test infrastructure only).

What the pages fix
  * "Nemotron NVFP4" explainer, "Why 4-bit training normally falls apart - and the three
    fixes": the weight-gradient GEMM's inputs are multiplied by a random Hadamard matrix,
    which spreads an outlier over its block before quantization and is undone analytically.
  * thelatentdaily "What matters for NVFP4 training?", "A methodological warning": the
    rotations use random sign vectors.

Reading R6 (where the pages are silent)
  * The transform acts on blocks of 16 consecutive tokens of one column, i.e. along the
    contraction dimension of the wgrad GEMM, so that Q^T Q = I cancels inside
    dW = dY^T X = (Q dY)^T (Q X) with the same Q on both operands.
  * Q = (1/4) H16 D: D = diag(sigma_j) with sigma_j = -1 iff bit j of a 16-bit sign mask is
    set (one mask per GEMM, shared by both operands and all blocks); H16 is the Sylvester
    Hadamard matrix in natural order, H[i][j] = (-1)^popcount(i & j).
  * Each output is the exact rational y_i = 1/4 * sum_j H[i][j] * sigma_j * v_j rounded once
    to binary32 (nearest, ties to even). An exactly zero sum is +0; a nonzero sum keeps its
    sign when it rounds to zero; a sum beyond the binary32 range rounds to infinity.
  * How the oracle evaluates it: the fast Walsh-Hadamard butterfly in binary64 (terms
    sigma_j * v_j / 4 + 0, which is exact and turns -0 into +0; stages h = 1, 2, 4, 8 replacing
    (u_j, u_{j+h}) by (u_j + u_{j+h}, u_j - u_{j+h})) followed by one rounding to binary32,
    for every block where a range check proves each butterfly step exact: every partial sum
    is a multiple of the smallest nonzero term's last significant bit 2^q and at most
    sum_j |u_j| in magnitude, so all of them are binary64 numbers when
    sum_j |u_j| < 2^(q + 53). With no -0 among the terms no step can produce -0, so the
    butterfly's zeros are +0 as the definition asks. Every other block is summed in exact
    rational arithmetic (fractions.Fraction) and rounded by _round_to_f32.
  * The output is written transposed: y[c, t] for input x[t, c], so that the quantization
    that follows runs along tokens in ordinary 1x16 row blocks.

Reading R23 (the Mosaic variant: thelatentdaily "What matters for NVFP4 training?", the
combined recipe applies random Hadamard transforms on both backward GEMMs, with 1D weight
quantization, which pairs naturally with rotations in the backward pass)
  * dgrad contracts over the layer's output features N: dX = dY W = (dY Q^T)(W^T Q^T)^T
    with Q acting on blocks of 16 consecutive output features. dY's rows are transformed
    in place (each row's 16-blocks, the "rowwise" transform, same butterfly and rounding as
    R6) and quantized 1x16 along the row (SR); W's columns are transformed along N exactly
    as the wgrad operands are along tokens (rht_quantize(W) gives W^T Q^T as [K, N]
    quantized along N).
  * Weights in that variant are quantized 1x16 (1D) for the forward GEMM.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .quantize import quantize_1x16, quantize_1x16_colsegments


def sign_vector(mask: int) -> np.ndarray:
    """sigma_j = -1 where bit j of the 16-bit mask is set, else +1."""
    return np.array([-1.0 if (int(mask) >> j) & 1 else 1.0 for j in range(16)])


def _butterfly16(u: np.ndarray) -> np.ndarray:
    """Unnormalized Walsh-Hadamard butterfly over the last axis (length 16), binary64."""
    u = np.array(u, dtype=np.float64, copy=True)
    lead = u.shape[:-1]
    for h in (1, 2, 4, 8):
        v = u.reshape(lead + (16 // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        u = v.reshape(lead + (16,))
    return u


def hadamard_matrix_from_butterfly() -> np.ndarray:
    """The 16x16 matrix the butterfly applies (column j = butterfly of unit vector e_j)."""
    return _butterfly16(np.eye(16)).T


def _terms(x, sign_mask: int) -> np.ndarray:
    """sigma_j * v_j / 4 (+0, so no term is -0) per block: x[tokens, cols] -> [cols, tokens/16, 16]
    in binary64 (exact: a power-of-two scale of a binary32 value)."""
    x = np.asarray(x, dtype=np.float32)
    t, c = x.shape
    if t % 16:
        raise ValueError("tokens must be a multiple of 16")
    v = x.astype(np.float64).T.reshape(c, t // 16, 16)
    return v * (sign_vector(sign_mask) * 0.25) + 0.0


def _butterfly_exact(u: np.ndarray) -> np.ndarray:
    """Per block (last axis): True when every partial sum of the binary64 butterfly over u is
    exact, i.e. sum |u_j| < 2^(q + 53) with 2^q the smallest last-significant-bit weight of a
    nonzero u_j. The float64 sum of |u_j| is enlarged by 2^-40 to cover its own rounding."""
    a = np.abs(u)
    nz = a != 0
    m, e = np.frexp(np.where(nz, a, 1.0))                 # a = m * 2^e, 0.5 <= m < 1
    mi = (m * 2.0 ** 53).astype(np.int64)                 # integer significand (exact)
    low = mi & -mi                                        # its lowest set bit
    q = e - 53 + np.round(np.log2(low.astype(np.float64))).astype(np.int64)
    qmin = np.where(nz, q, 1 << 20).min(axis=-1)               # all-zero blocks: see below
    total = a.sum(axis=-1) * (1.0 + 2.0 ** -40)
    lim = np.ldexp(1.0, np.clip(qmin + 53, -1074, 1023).astype(np.int64))
    return (~nz.any(axis=-1)) | (total < lim)


def _round_to_f32(q: Fraction) -> np.float32:
    """An exact rational rounded once to binary32: nearest, ties to the even significand;
    +0 for zero, the sign kept for a nonzero value that rounds to zero, infinity beyond the
    largest finite value (IEEE 754 round-to-nearest-even with gradual underflow)."""
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    mag = -q if neg else q
    n, d = mag.numerator, mag.denominator
    e = n.bit_length() - d.bit_length()                   # 2^(e-1) < mag < 2^(e+1)
    if Fraction(2) ** e > mag:
        e -= 1                                            # now 2^e <= mag < 2^(e+1)
    lsb = max(e, -126) - 23                                # weight of the last kept bit
    scaled = mag / Fraction(2) ** lsb                      # mag in units of that bit
    k = scaled.numerator // scaled.denominator
    rest = scaled - k
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and k % 2 == 1):
        k += 1
    val = k * Fraction(2) ** lsb
    if val >= Fraction(2) ** 128:
        out = np.float32(np.inf)
    else:
        out = np.float32(float(val))                       # k < 2^25: exact in binary32
    return -out if neg else out


def _exact_block(v32: np.ndarray, sign_mask: int) -> np.ndarray:
    """The 16 outputs of one block by exact arithmetic: every binary32 value is an integer
    multiple of 2^-149, so 2^151 * sigma_j * v_j / 4 is an integer and each output is an
    integer sum over 2^151, rounded by _round_to_f32."""
    sig = sign_vector(sign_mask)
    h = hadamard_matrix_from_butterfly()
    units = []
    for a in v32:
        n, d = float(a).as_integer_ratio()                # d = 2^k with k <= 149
        units.append(n * ((1 << 149) // d))               # v_j * 2^149
    out = np.empty(16, dtype=np.float32)
    for i in range(16):
        s = sum(int(h[i, j] * sig[j]) * units[j] for j in range(16))
        out[i] = _round_to_f32(Fraction(s, 1 << 151))     # (v-sum * 2^149) / 4 / 2^149
    return out


def rht_columnwise_f64(x, sign_mask: int) -> np.ndarray:
    """0.25 * H16 * D applied to each 16-token block of each column, in binary64, before the
    final rounding: x[tokens, cols] -> [cols, tokens]. Only defined where the butterfly is
    exact (raises otherwise), so these values are the exact products."""
    u = _terms(x, sign_mask)
    if not _butterfly_exact(u).all():
        raise ValueError("a block is outside the range where the binary64 butterfly is exact")
    c, nb, _ = u.shape
    return _butterfly16(u).reshape(c, nb * 16)


def rht_columnwise(x, sign_mask: int) -> np.ndarray:
    """The transform rounded once to float32 (R6). x[tokens, cols] -> y[cols, tokens]."""
    x32 = np.asarray(x, dtype=np.float32)
    u = _terms(x32, sign_mask)
    c, nb, _ = u.shape
    with np.errstate(over="ignore"):
        y = _butterfly16(u).astype(np.float32)
    wide = ~_butterfly_exact(u)
    if wide.any():
        v = x32.T.reshape(c, nb, 16)
        for ci, bi in zip(*np.nonzero(wide)):
            y[ci, bi] = _exact_block(v[ci, bi], sign_mask)
    return y.reshape(c, nb * 16)


def rht_quantize_segments(x, sign_mask: int, token_segments, rounding: str = "rn", seed: int = 0,
                          offset: int = 0):
    """The transform along tokens, then 1x16 quantization of the transposed result with one
    tensor scale per token segment (the tokens of one expert; multiples of 16), each from the
    maximum of its own transformed values (R16). Returns (codes [cols, tokens/2],
    scales [cols, tokens/16], s_dec [G])."""
    y = rht_columnwise(x, sign_mask)
    return quantize_1x16_colsegments(y, token_segments, rounding=rounding, seed=seed, offset=offset)


def rht_quantize(x, sign_mask: int, rounding: str = "rn", seed: int = 0, offset: int = 0,
                 amax_vals=None, col_ids=None):
    """Transform along tokens, then 1x16 quantization of the transposed result.

    x may be a column subset X[:, col_ids]; then amax_vals must hold the amax of the full
    transformed tensor. Returns (codes [cols, tokens/2], scales [cols, tokens/16], s_dec)."""
    y = rht_columnwise(x, sign_mask)
    return quantize_1x16(y, rounding=rounding, seed=seed, offset=offset,
                         amax_vals=amax_vals, row_ids=col_ids)


def rht_rowwise(x, sign_mask: int) -> np.ndarray:
    """R23: the transform of each row's 16-element blocks (the R6 butterfly on x^T), rounded
    once to float32. x[rows, cols] -> y[rows, cols]."""
    x = np.asarray(x, dtype=np.float32)
    return np.ascontiguousarray(rht_columnwise(np.ascontiguousarray(x.T), sign_mask))


def rht_rowwise_quantize(x, sign_mask: int, rounding: str = "rn", seed: int = 0, offset: int = 0,
                         amax_vals=None):
    """R23: rowwise transform, then 1x16 quantization along the rows (tensor scale from the
    transformed values unless amax_vals is given). Returns (codes, scales, s_dec)."""
    return quantize_1x16(rht_rowwise(x, sign_mask), rounding=rounding, seed=seed, offset=offset,
                         amax_vals=amax_vals)
