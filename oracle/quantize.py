"""Two-level NVFP4 block quantization (oracle; test infrastructure only).

What the pages fix
  * "Nemotron NVFP4" explainer, "What NVFP4 actually is": elements are E2M1, each block of 16
    elements shares an E4M3 scale, and the whole tensor shares one FP32 scale; storage is
    4 + 8/16 = 4.5 bits per element.
  * artiverse.ca "NVIDIA's 4-bit floating point pushes AI training limits": per-block scales
    combined with a per-tensor adjustment; weights use 16x16 blocks instead of 1x16 so the
    forward and backward passes see the same values; stochastic rounding only on gradients.

Readings (where the pages are silent; labels R3-R8, R11, R12, shared with the other oracle modules)
  R3  BF16 input widens exactly to FP32; FP32 input is used as is.
  R4  A = max |x| over the tensor (per segment for expert-stacked tensors). If A == 0 then
      s_enc = s_dec = 1; else s_enc = fl32(2688 / A) (clamped to FLT_MAX) and
      s_dec = fl32(A / 2688). 2688 = 6 * 448, so the tensor's largest magnitude maps to the
      largest element times the largest scale. s_dec is the stored FP32 tensor scale.
  R5  The block amax a_b is max |x| over 16 consecutive elements of a row (1x16) or over an
      aligned 16x16 tile (2D weight blocks).
  R7  t_b = fl32(fl32(a_b / 6) * s_enc); the stored block scale is S_b = E4M3(t_b) (RNE,
      saturating).
  R8  If S_b decodes to 0 every element of the block encodes as a signed zero. Otherwise
      r_b = min(fl32(s_enc / dec(S_b)), FLT_MAX) and each element is y = fl32(x * r_b),
      which is then rounded to E2M1 (RN, or SR with the block's Philox bytes).
  R11 codes[r, c/2] holds element c (even) in the low nibble and c+1 in the high nibble;
      scales are [rows, cols/16] row-major; a 16x16 tile's scale is repeated in each of its
      16 rows, so every NVFP4 tensor has the same layout. The transposed emission of a
      16x16-quantized W is by definition the 16x16 quantization of W^T.
  R12 The dequantized value is e2m1(code) * e4m3(S_b) * s_dec (exact in float64).
"""
from __future__ import annotations

import numpy as np

from .formats import (E2M1_MAX, E4M3_MAX, e2m1_decode, e2m1_encode_rn, e2m1_encode_sr,
                      e4m3_decode, e4m3_encode)
from .philox import block_random_bytes

F32 = np.float32
FLT_MAX = np.finfo(np.float32).max
SCALE_NUMERATOR = F32(E2M1_MAX * E4M3_MAX)      # 2688, exact in float32


def _as_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)


def _segment_of_rows(row_ids: np.ndarray, segments) -> np.ndarray:
    if segments is None:
        return np.zeros(row_ids.shape, dtype=np.int64)
    seg = np.asarray(segments, dtype=np.int64)
    s = np.searchsorted(seg, row_ids, side="right") - 1
    if np.any(s < 0) or np.any(s >= len(seg) - 1):
        raise ValueError("row outside the segment table")
    return s


def amax(x, segments=None) -> np.ndarray:
    """max |x| over the whole tensor, or per row segment (R4). Returns float32 [nseg]."""
    x = _as_f32(x)
    if segments is None:
        return np.array([np.abs(x).max() if x.size else 0.0], dtype=F32)
    seg = np.asarray(segments, dtype=np.int64)
    out = np.zeros(len(seg) - 1, dtype=F32)
    for g in range(len(seg) - 1):
        part = x[seg[g]:seg[g + 1]]
        out[g] = np.abs(part).max() if part.size else F32(0)
    return out


def global_scales(a) -> tuple[np.ndarray, np.ndarray]:
    """(s_enc, s_dec) from the tensor amax values (R4)."""
    a = _as_f32(a)
    with np.errstate(divide="ignore", over="ignore"):
        s_enc = np.where(a == 0, F32(1), SCALE_NUMERATOR / np.where(a == 0, F32(1), a))
        s_dec = np.where(a == 0, F32(1), a / SCALE_NUMERATOR)
    s_enc = np.minimum(s_enc.astype(F32), F32(FLT_MAX))
    return s_enc.astype(F32), s_dec.astype(F32)


def _encode_blocks(xb: np.ndarray, a_b: np.ndarray, s_enc: np.ndarray, rounding: str,
                   rbytes: np.ndarray | None):
    """Encode blocks xb [n, 16] (float32) with block amax a_b [n] and tensor encode scale
    s_enc [n]. Returns (codes [n, 16] uint8, scale codes [n] uint8)  (R7, R8)."""
    t = (a_b / F32(6.0)).astype(F32)
    t = (t * s_enc).astype(F32)
    S = e4m3_encode(t)
    dS = e4m3_decode(S).astype(F32)                       # exact in float32
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        r = np.where(dS > 0, s_enc / np.where(dS > 0, dS, F32(1)), F32(0)).astype(F32)
    r = np.minimum(r, F32(FLT_MAX)).astype(F32)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (xb * r[:, None]).astype(F32)
    if rounding == "rn":
        codes = e2m1_encode_rn(y)
    elif rounding == "sr":
        codes = e2m1_encode_sr(y, rbytes)
    else:
        raise ValueError(rounding)
    zero_scale = (dS == 0)[:, None]
    signed_zero = np.signbit(xb).astype(np.uint8) << 3
    codes = np.where(zero_scale, signed_zero, codes).astype(np.uint8)
    return codes, S


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[rows, cols] 4-bit codes -> [rows, cols/2] bytes, even column in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def quantize_1x16(x, rounding: str = "rn", seed: int = 0, offset: int = 0, segments=None,
                  amax_vals=None, row_ids=None):
    """Quantize x[rows, cols] along cols in 1x16 blocks.

    x may be a subset of the tensor's rows: then ``row_ids`` gives their global indices (used
    for the segment lookup and the stochastic-rounding block index, R10) and ``amax_vals``
    must hold the full tensor's amax per segment. ``cols`` is the full row length.
    Returns (codes [rows, cols/2] uint8, scales [rows, cols/16] uint8, s_dec [nseg] f32)."""
    x = _as_f32(x)
    rows, cols = x.shape
    if cols % 16:
        raise ValueError("cols must be a multiple of 16")
    row_ids = np.arange(rows, dtype=np.int64) if row_ids is None else np.asarray(row_ids, np.int64)
    a_t = amax(x, segments) if amax_vals is None else _as_f32(amax_vals).reshape(-1)
    s_enc, s_dec = global_scales(a_t)
    seg = _segment_of_rows(row_ids, segments)
    nb = cols // 16
    xb = x.reshape(rows * nb, 16)
    a_b = np.abs(xb).max(axis=1).astype(F32) if xb.size else np.zeros(0, F32)
    s_enc_b = np.repeat(s_enc[seg], nb)
    rbytes = None
    if rounding == "sr":
        bidx = (row_ids[:, None] * nb + np.arange(nb, dtype=np.int64)[None, :]).reshape(-1)
        rbytes = block_random_bytes(bidx, seed, offset)
    codes, S = _encode_blocks(xb, a_b, s_enc_b, rounding, rbytes)
    return pack_nibbles(codes.reshape(rows, cols)), S.reshape(rows, nb), s_dec


def quantize_1x16_colsegments(x, col_segments, rounding: str = "rn", seed: int = 0,
                              offset: int = 0, amax_vals=None, row_ids=None):
    """1x16 quantization of x[rows, cols] along cols with one tensor scale per range of
    columns (R16): columns col_segments[g]..col_segments[g+1] (multiples of 16, covering
    [0, cols]) use amax_vals[g], by default their own max|x|. This is the transposed
    weight-gradient operand of an expert layer, whose columns are the tokens routed to each
    expert. The stochastic-rounding block index is the block's place in the whole tensor,
    as in quantize_1x16; x may be a subset of the tensor's rows given by ``row_ids`` (then
    amax_vals must be given). Returns (codes [rows, cols/2], scales [rows, cols/16], s_dec [G])."""
    x = _as_f32(x)
    rows, cols = x.shape
    seg = np.asarray(col_segments, dtype=np.int64)
    if cols % 16 or np.any(seg % 16) or seg[0] != 0 or seg[-1] != cols or np.any(np.diff(seg) < 0):
        raise ValueError("column segments must be multiples of 16 covering [0, cols]")
    G = len(seg) - 1
    if amax_vals is None:
        if row_ids is not None:
            raise ValueError("a row subset needs the full tensor's amax_vals")
        a_t = np.array([np.abs(x[:, seg[g]:seg[g + 1]]).max() if seg[g + 1] > seg[g] else 0.0
                        for g in range(G)], dtype=F32)
    else:
        a_t = _as_f32(amax_vals).reshape(-1)
    s_enc, s_dec = global_scales(a_t)
    nb = cols // 16
    gid = np.searchsorted(seg, np.arange(nb, dtype=np.int64) * 16, side="right") - 1
    xb = x.reshape(rows * nb, 16)
    a_b = np.abs(xb).max(axis=1).astype(F32) if xb.size else np.zeros(0, F32)
    s_enc_b = np.tile(s_enc[gid], rows)
    rbytes = None
    if rounding == "sr":
        rid = np.arange(rows, dtype=np.int64) if row_ids is None else np.asarray(row_ids, np.int64)
        bidx = (rid[:, None] * nb + np.arange(nb, dtype=np.int64)[None, :]).reshape(-1)
        rbytes = block_random_bytes(bidx, seed, offset)
    codes, S = _encode_blocks(xb, a_b, s_enc_b, rounding, rbytes)
    return pack_nibbles(codes.reshape(rows, cols)), S.reshape(rows, nb), s_dec


def quantize_16x16(x, segments=None, amax_vals=None, row_ids=None):
    """Quantize x[rows, cols] with one scale per aligned 16x16 tile, round-to-nearest
    (weights). The scale is stored once per row of the tile (R11).

    As for quantize_1x16, x may be a subset of rows made of whole aligned 16-row groups."""
    x = _as_f32(x)
    rows, cols = x.shape
    if rows % 16 or cols % 16:
        raise ValueError("rows and cols must be multiples of 16")
    row_ids = np.arange(rows, dtype=np.int64) if row_ids is None else np.asarray(row_ids, np.int64)
    if np.any(row_ids[0::16] % 16) or np.any(np.diff(row_ids.reshape(-1, 16), axis=1) != 1):
        raise ValueError("rows must come in aligned groups of 16")
    a_t = amax(x, segments) if amax_vals is None else _as_f32(amax_vals).reshape(-1)
    s_enc, s_dec = global_scales(a_t)
    seg = _segment_of_rows(row_ids, segments)
    nb = cols // 16
    tiles = np.abs(x).reshape(rows // 16, 16, nb, 16).max(axis=(1, 3)).astype(F32)
    a_b = np.repeat(tiles, 16, axis=0).reshape(-1)        # one entry per (row, 16-col block)
    s_enc_b = np.repeat(s_enc[seg], nb)
    codes, S = _encode_blocks(x.reshape(rows * nb, 16), a_b, s_enc_b, "rn", None)
    return pack_nibbles(codes.reshape(rows, cols)), S.reshape(rows, nb), s_dec


def dequantize(codes_packed, scales, s_dec, segments=None, row_ids=None) -> np.ndarray:
    """x_hat = e2m1(code) * e4m3(S_b) * s_dec in float64 (R12)."""
    c = unpack_nibbles(codes_packed)
    rows, cols = c.shape
    row_ids = np.arange(rows, dtype=np.int64) if row_ids is None else np.asarray(row_ids, np.int64)
    seg = _segment_of_rows(row_ids, segments)
    s = e4m3_decode(np.asarray(scales)).astype(np.float64)
    s_full = np.repeat(s, 16, axis=1)
    sd = np.asarray(s_dec, dtype=np.float32).astype(np.float64)[seg][:, None]
    return e2m1_decode(c) * s_full * sd
