"""E2M1 element and E4M3 scale codecs (oracle; test infrastructure only).

Format facts from the pages
  * "Nemotron NVFP4" explainer, "What NVFP4 actually is": the element is E2M1 (one sign,
    two exponent and one mantissa bit); the block scale is FP8 E4M3.
  * skillainest "NVIDIA researchers unlock 4-bit LLM training...", "How NVFP4 works": a
    4-bit code has 16 bit patterns.

Readings where the pages are silent
  R1  E2M1 is an IEEE-style minifloat with exponent bias 1 and a subnormal at exponent 0:
      magnitude = m/2 for e = 0, (1 + m/2) * 2^(e-1) otherwise; no Inf/NaN. The 8
      magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}; +0 and -0 are both zero.
  R2  E4M3 is the OCP "E4M3FN" variant: bias 7, no Inf, NaN = S.1111.111, largest finite
      value 448, subnormals m * 2^-9. Encoding rounds to nearest, ties to even, saturates to
      448, and never produces a negative scale.
  R9  Deterministic element rounding is round-to-nearest, ties to the even code (mantissa bit
      0), saturating at 6; the sign bit is the sign bit of the input, so negative values that
      round to zero give code 0x8.
  R10 Stochastic rounding takes a = min(|y|, 6); if a is on the grid it is kept; otherwise
      with lo < a < hi the neighbouring grid values and frac = (a - lo) / (hi - lo), it rounds
      up iff frac + r/256 >= 1 for the random byte r in [0, 255]. This is the usual "add
      random bits below the kept precision, then truncate" rule with 8 random bits, so
      P(up) = floor(256 * frac) / 256 and the expected value is within gap/256 of a.
"""
from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0


def _e2m1_magnitudes() -> np.ndarray:
    """Magnitudes of the 8 non-negative E2M1 codes, from the bit fields (R1)."""
    out = np.zeros(8, dtype=np.float64)
    for code in range(8):
        e = (code >> 1) & 0x3
        m = code & 0x1
        out[code] = (m * 0.5) if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return out


E2M1_GRID = _e2m1_magnitudes()          # ascending: code index == rank


def e2m1_decode(codes) -> np.ndarray:
    """Value of each 4-bit code (bit 3 = sign) as float64."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    mag = E2M1_GRID[c & 0x7]
    return np.where(c & 0x8, -mag, mag)


def _sign_bits(y: np.ndarray) -> np.ndarray:
    return np.signbit(np.asarray(y)).astype(np.uint8) << 3


def e2m1_encode_rn(y) -> np.ndarray:
    """Nearest E2M1 code to each float32 value, ties to even code, saturating (R9)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y).astype(np.float64), E2M1_MAX)
    lo = np.clip(np.searchsorted(E2M1_GRID, a, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    d_lo = a - E2M1_GRID[lo]
    d_hi = E2M1_GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    idx = np.where(pick_hi, hi, lo).astype(np.uint8)
    return idx | _sign_bits(y)


def e2m1_encode_sr(y, rbytes) -> np.ndarray:
    """Stochastic rounding of each float32 value with its random byte (R10)."""
    y = np.asarray(y, dtype=np.float32)
    r = np.asarray(rbytes).astype(np.float64)
    a = np.minimum(np.abs(y).astype(np.float64), E2M1_MAX)
    lo = np.clip(np.searchsorted(E2M1_GRID, a, side="right") - 1, 0, 7)
    on_grid = E2M1_GRID[lo] == a
    hi = np.minimum(lo + 1, 7)
    gap = np.where(on_grid, 1.0, E2M1_GRID[hi] - E2M1_GRID[lo])
    frac = np.where(on_grid, 0.0, (a - E2M1_GRID[lo]) / gap)   # exact: gap is a power of 2
    up = (~on_grid) & (frac + r / 256.0 >= 1.0)                  # exact in float64
    idx = np.where(up, hi, lo).astype(np.uint8)
    return idx | _sign_bits(y)


def _e4m3_values() -> np.ndarray:
    """Values of the 256 E4M3 codes (NaN for 0x7F/0xFF), from the bit fields (R2)."""
    out = np.zeros(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = s * m * 2.0 ** -9
        else:
            out[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


E4M3_TABLE = _e4m3_values()
_E4M3_POS = E4M3_TABLE[:0x7F]          # codes 0x00..0x7E, ascending, finite


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code as float64."""
    return E4M3_TABLE[np.asarray(codes).astype(np.int64) & 0xFF]


def e4m3_encode(t) -> np.ndarray:
    """E4M3 code of each non-negative float32 scale: nearest, ties to even, saturating to
    448 (R2). Inputs are block-scale candidates, which are never negative."""
    t = np.asarray(t, dtype=np.float32).astype(np.float64)
    a = np.minimum(t, E4M3_MAX)
    lo = np.clip(np.searchsorted(_E4M3_POS, a, side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    return np.where(pick_hi, hi, lo).astype(np.uint8)
