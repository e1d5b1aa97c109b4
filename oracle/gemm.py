"""Reference GEMM on dequantized NVFP4 operands (oracle; test infrastructure only).

The pages place the format in the three linear-layer GEMMs of training, forward, backward
(activation gradient) and weight gradient (artiverse.ca "NVIDIA's 4-bit floating point pushes
AI training limits", paragraph on which parts run in 4-bit), and in the expert GEMMs of the
mixture-of-experts layers ("Nemotron NVFP4" explainer, "The model underneath").

Reading R13: D[m, n] = sum_k A_hat[m, k] * B_hat[n, k] with both operands stored along K
("TN"); the reference is computed in binary64 (numpy/BLAS dgemm, whose rounding error
~K * 2^-53 is far below the acceptance bound). A GPU result D (FP32 accumulation, FP32 output)
is accepted iff |D - D64| <= 1e-5 * sum_k |A_hat[m,k]| |B_hat[n,k]| for every element.
Reading R14: the grouped GEMM is one such GEMM per group g over rows
m_offsets[g]..m_offsets[g+1] of A and rows g*N..(g+1)*N of the stacked B.
Reading R15: the MoE weight gradient groups along the contraction instead: group g sums
over columns k_offsets[g]..k_offsets[g+1] (the tokens routed to expert g) of A [M, K] and
B [N, K] into its own [M, N] block, stacked along rows; an empty group gives zeros.

The linear-layer wrapper around these GEMMs (the forward output feeds the next layer in
16-bit, the weight gradient accumulates into an FP32 main gradient; artiverse.ca page, same
paragraph: only the GEMMs run in 4-bit, the rest of the layer stays in higher precision):
Reading R18: a BF16 output is the binary32 result rounded once more to BF16 (nearest, ties
to even). Against D64 it is accepted within the FP32 bound plus BF16's relative rounding
error 2^-8 of the result (and half its smallest subnormal spacing).
Reading R19: with accumulation the output is D_old + the product in binary32 (one more
rounding of the sum); against D_old + D64 it is accepted within the FP32 bound plus 2^-24 of
the result.
Reading R20: the output's amax is max |D| over the values as stored (after the BF16
rounding for a BF16 output), the tensor amax a later quantization of D needs.
"""
from __future__ import annotations

import numpy as np


def gemm_fp64(a_hat: np.ndarray, b_hat: np.ndarray) -> np.ndarray:
    """D64 = A_hat @ B_hat^T in binary64."""
    return np.asarray(a_hat, np.float64) @ np.asarray(b_hat, np.float64).T


def gemm_bound(a_hat: np.ndarray, b_hat: np.ndarray, rel: float = 1e-5) -> np.ndarray:
    """Per-element acceptance bound rel * sum_k |a||b|."""
    return rel * (np.abs(np.asarray(a_hat, np.float64)) @ np.abs(np.asarray(b_hat, np.float64)).T)


def grouped_gemm_fp64(a_hat, b_hat, m_offsets, n: int) -> np.ndarray:
    """Per-group D_g = A_g @ B_g^T stacked along rows; A_g rows come from m_offsets."""
    off = np.asarray(m_offsets, dtype=np.int64)
    out = np.zeros((int(off[-1]) - int(off[0]), n), dtype=np.float64)
    for g in range(len(off) - 1):
        lo, hi = int(off[g]) - int(off[0]), int(off[g + 1]) - int(off[0])
        if hi > lo:
            out[lo:hi] = gemm_fp64(a_hat[lo:hi], b_hat[g * n:(g + 1) * n])
    return out


def grouped_gemm_bound(a_hat, b_hat, m_offsets, n: int, rel: float = 1e-5) -> np.ndarray:
    off = np.asarray(m_offsets, dtype=np.int64)
    out = np.zeros((int(off[-1]) - int(off[0]), n), dtype=np.float64)
    for g in range(len(off) - 1):
        lo, hi = int(off[g]) - int(off[0]), int(off[g + 1]) - int(off[0])
        if hi > lo:
            out[lo:hi] = gemm_bound(a_hat[lo:hi], b_hat[g * n:(g + 1) * n], rel)
    return out


def grouped_gemm_k_fp64(a_hat, b_hat, k_offsets) -> np.ndarray:
    """R15: D[g*M:(g+1)*M] = A[:, k_g] @ B[:, k_g]^T over k_g = k_offsets[g]..k_offsets[g+1]."""
    a = np.asarray(a_hat, np.float64)
    b = np.asarray(b_hat, np.float64)
    off = np.asarray(k_offsets, dtype=np.int64)
    m, n = a.shape[0], b.shape[0]
    out = np.zeros(((len(off) - 1) * m, n), dtype=np.float64)
    for g in range(len(off) - 1):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            out[g * m:(g + 1) * m] = gemm_fp64(a[:, lo:hi], b[:, lo:hi])
    return out


def grouped_gemm_k_bound(a_hat, b_hat, k_offsets, rel: float = 1e-5) -> np.ndarray:
    a = np.asarray(a_hat, np.float64)
    b = np.asarray(b_hat, np.float64)
    off = np.asarray(k_offsets, dtype=np.int64)
    m, n = a.shape[0], b.shape[0]
    out = np.zeros(((len(off) - 1) * m, n), dtype=np.float64)
    for g in range(len(off) - 1):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            out[g * m:(g + 1) * m] = gemm_bound(a[:, lo:hi], b[:, lo:hi], rel)
    return out


def round_bf16(x) -> np.ndarray:
    """R18: binary32 values rounded to BF16 (8 significant bits, binary32's exponent range),
    nearest with ties to even, returned as float32. Finite inputs; a value past the largest
    BF16 rounds to infinity as the rule implies."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def gemm_bf16_bound(a_hat, b_hat, rel: float = 1e-5) -> np.ndarray:
    """R18: acceptance bound of a BF16 output against D64 = gemm_fp64(a_hat, b_hat)."""
    s = gemm_bound(a_hat, b_hat, rel)
    return s + 2.0 ** -8 * (np.abs(gemm_fp64(a_hat, b_hat)) + s) + 2.0 ** -134


def gemm_accumulate_fp64(d_old, a_hat, b_hat) -> np.ndarray:
    """R19: D_old + A_hat @ B_hat^T in binary64."""
    return np.asarray(d_old, np.float64) + gemm_fp64(a_hat, b_hat)


def gemm_accumulate_bound(d_old, a_hat, b_hat, rel: float = 1e-5) -> np.ndarray:
    """R19: acceptance bound of an accumulated FP32 output against gemm_accumulate_fp64."""
    s = gemm_bound(a_hat, b_hat, rel)
    return s + 2.0 ** -24 * (np.abs(gemm_accumulate_fp64(d_old, a_hat, b_hat)) + s) + 2.0 ** -150
