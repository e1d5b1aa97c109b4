"""MXFP4 quantization (oracle; test infrastructure only).

The pages set MXFP4 against NVFP4 ("Nemotron NVFP4" explainer, "What NVFP4 actually is" and
the storage-cost comparison below it): the same E2M1 element, but one power-of-two (E8M0)
scale per block of 32 elements and no tensor-level scale, 4.25 bits per element; a coarser,
cheaper format that trains less well (skillainest "NVIDIA researchers unlock 4-bit LLM
training...", the 8B comparison). The pages do not say how the power-of-two scale is chosen.

Reading R22 (the OCP Microscaling Formats v1.0 conversion, the format's public definition):
  block = 32 consecutive elements of a row; amax = max |x| over the block;
  shared exponent e = floor(log2(amax)) - 2 (2 = exponent of E2M1's largest power of two,
  4 <= 6 < 8), clamped to [-127, 127]; amax = 0 gives e = -127;
  scale code = e + 127 (E8M0: value 2^(code - 127); 255 would be NaN and never occurs);
  element = E2M1(x / 2^e) rounded to nearest, ties to even, saturating at 6 (R9), x / 2^e
  taken in binary32 (exact unless it falls below binary32's normal range, where it rounds
  like any binary32 product).
  Stochastic rounding (gradients) uses R10 with the random byte of element j of the
  16-element half-block with linear index b = (row * cols + col) / 16, the same counter
  mapping as the NVFP4 path.
So the block's largest element lands in [4, 8) before rounding and encodes as 4 or 6.
Layout: codes [rows, cols/2] (element 2i in the low nibble, as NVFP4), scales [rows, cols/32]
E8M0 codes.
"""
from __future__ import annotations

import numpy as np

from .formats import e2m1_decode, e2m1_encode_rn, e2m1_encode_sr
from .philox import block_random_bytes
from .quantize import pack_nibbles, unpack_nibbles

MX_BLOCK = 32
E8M0_BIAS = 127


def e8m0_decode(codes) -> np.ndarray:
    """Value 2^(code - 127) of each E8M0 code as float64 (NaN for 255)."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - E8M0_BIAS))


def mx_shared_exponent(amax) -> np.ndarray:
    """R22: floor(log2(amax)) - 2 clamped to [-127, 127]; -127 for amax = 0."""
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(a)                      # a = m * 2^ex, m in [0.5, 1): floor(log2 a) = ex - 1
    e = np.where(a > 0, ex.astype(np.int64) - 1 - 2, -E8M0_BIAS)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS)


def quantize_mxfp4(x, rounding: str = "rn", seed: int = 0, offset: int = 0):
    """x[rows, cols] (cols % 32 == 0) -> (codes [rows, cols/2] uint8, scales [rows, cols/32]
    uint8 E8M0)."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    if cols % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    nb = cols // MX_BLOCK
    xb = x.reshape(rows, nb, MX_BLOCK)
    amax = np.abs(xb).max(axis=2) if x.size else np.zeros((rows, nb), np.float32)
    e = mx_shared_exponent(amax)                                  # [rows, nb]
    with np.errstate(under="ignore"):
        y = (xb.astype(np.float64) * np.ldexp(1.0, -e)[:, :, None]).astype(np.float32)
    y16 = y.reshape(rows * cols // 16, 16)
    if rounding == "rn":
        codes = e2m1_encode_rn(y16)
    elif rounding == "sr":
        rbytes = block_random_bytes(np.arange(rows * cols // 16, dtype=np.int64), seed, offset)
        codes = e2m1_encode_sr(y16, rbytes)
    else:
        raise ValueError(rounding)
    return pack_nibbles(codes.reshape(rows, cols)), (e + E8M0_BIAS).astype(np.uint8)


def dequantize_mxfp4(codes_packed, scales) -> np.ndarray:
    """x_hat = e2m1(code) * 2^(scale - 127) in float64 (exact)."""
    c = unpack_nibbles(codes_packed)
    s = np.repeat(e8m0_decode(scales), MX_BLOCK, axis=1)
    return e2m1_decode(c) * s
