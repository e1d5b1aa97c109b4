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
  * It is computed by the fast Walsh-Hadamard butterfly in binary64: signs applied first
    (exact), then stages h = 1, 2, 4, 8 replacing (u_j, u_{j+h}) by (u_j + u_{j+h},
    u_j - u_{j+h}) for j with (j & h) == 0, then a multiply by 0.25 (exact), then one
    round-to-nearest-even to binary32. For BF16 inputs whose 16-block exponent spread is at
    most 40 binades every binary64 step is exact, so the result is the correctly rounded
    exact product (pinned against exact rational arithmetic).
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


def rht_columnwise_f64(x, sign_mask: int) -> np.ndarray:
    """0.25 * H16 * D applied to each 16-token block of each column, in binary64, before
    the final rounding. x[tokens, cols] -> [cols, tokens]."""
    x = np.asarray(x, dtype=np.float32)
    t, c = x.shape
    if t % 16:
        raise ValueError("tokens must be a multiple of 16")
    v = x.astype(np.float64).T.reshape(c, t // 16, 16)
    u = v * sign_vector(sign_mask)
    return (_butterfly16(u) * 0.25).reshape(c, t)


def rht_columnwise(x, sign_mask: int) -> np.ndarray:
    """The transform rounded once to float32 (R6). x[tokens, cols] -> y[cols, tokens]."""
    return rht_columnwise_f64(x, sign_mask).astype(np.float32)


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
