"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module only draws random numbers and rounds them to BF16 storage; it holds none of
the NVFP4 arithmetic (no scales, no encoding, no transform), so both the CPU oracle and the
HIP path can consume its outputs without sharing any of the method's code.

Every tensor is produced on the CPU with ``numpy.random.default_rng(seed)`` in float32 and
then rounded to BF16 with round-to-nearest-even, so it is identical on every machine.
BF16 tensors are returned as ``uint16`` bit patterns (row-major).

Workload shapes (the dense layer is the one a 12B-class hybrid model uses for its MLP
up-projection; the MoE layer mirrors an expert layer with 128 experts, top-6 routing):
  tiny    A[256,256], W[256,256] ~ N(0,1) with 0.1% of entries scaled x50
  fprop   X[8192,5120] ~ N(0,1) + 0.1% x50 outliers ; W[20480,5120] ~ N(0, 0.02)
  dgrad   dY[8192,20480] ~ N(0, 1e-3)
  wgrad   dY and X as above, 16-bit random sign mask for the Hadamard transform
  moe     16384 tokens pick 6 of 128 experts (Gumbel top-6 over Zipf(1.1) weights);
          X[98304,2688] ~ N(0,1) in expert-sorted order; W[128*1856, 2688] ~ N(0,1)
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "normal_bf16", "with_outliers_bf16",
    "tiny", "fprop", "dgrad", "wgrad_sign_mask", "moe_routing", "moe",
    "SEEDS", "SR_SEED_DGRAD", "SR_SEED_WGRAD", "SR_OFFSET_WGRAD",
    "exponent_spread_bf16", "exponent_spread_f32", "hadamard_edge_blocks_bf16", "WIDE_SPREADS",
]

SEEDS = {
    "tiny_a": 101, "tiny_w": 102,
    "fprop_x": 201, "fprop_w": 202,
    "dgrad_dy": 301,
    "moe_dy": 504,
    "wgrad_sign": 401,
    "moe_route": 501, "moe_x": 502, "moe_w": 503,
}
SR_SEED_DGRAD = 0x5EED0003
SR_SEED_WGRAD = 0x5EED0004
SR_OFFSET_WGRAD = 1 << 32

MOE_EXPERTS = 128
MOE_TOKENS = 16384
MOE_TOPK = 6
MOE_HIDDEN = 2688
MOE_FFN = 1856


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (nearest, ties to even) and return the 16-bit patterns.

    Inputs must be finite (the generators never produce NaN/Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_f32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def normal_bf16(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) entries rounded to BF16 bits."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(_normal_f32(rng, shape, std))


def with_outliers_bf16(shape, seed: int, frac: float = 1e-3, factor: float = 50.0) -> np.ndarray:
    """N(0,1) entries where exactly round(frac * numel) distinct entries are scaled by factor
    before the BF16 rounding."""
    rng = np.random.default_rng(seed)
    x = _normal_f32(rng, shape, 1.0)
    n = x.size
    k = int(round(frac * n))
    idx = rng.choice(n, size=k, replace=False)
    flat = x.reshape(-1)
    flat[idx] *= np.float32(factor)
    return f32_to_bf16_bits(x)


def tiny():
    """A[256,256] (activations, 1x16 blocks) and W[256,256] (weights, 16x16 blocks)."""
    a = with_outliers_bf16((256, 256), SEEDS["tiny_a"])
    w = with_outliers_bf16((256, 256), SEEDS["tiny_w"])
    return a, w


def fprop(m: int = 8192, n: int = 20480, k: int = 5120):
    """Activations X[m,k] with outliers and weights W[n,k] ~ N(0, 0.02)."""
    x = with_outliers_bf16((m, k), SEEDS["fprop_x"])
    w = normal_bf16((n, k), SEEDS["fprop_w"], std=0.02)
    return x, w


def dgrad(m: int = 8192, n: int = 20480):
    """Output gradient dY[m,n] ~ N(0, 1e-3) (1e-3 read as the standard deviation)."""
    return normal_bf16((m, n), SEEDS["dgrad_dy"], std=1e-3)


def wgrad_sign_mask() -> int:
    """The 16-bit sign mask of the random Hadamard transform used for the wgrad operands."""
    return int(np.random.default_rng(SEEDS["wgrad_sign"]).integers(0, 65536))


def moe_routing(tokens: int = MOE_TOKENS, experts: int = MOE_EXPERTS, topk: int = MOE_TOPK,
                zipf_s: float = 1.1, seed: int = SEEDS["moe_route"]) -> np.ndarray:
    """Rows per expert for top-k routing with Zipf-like expert popularity.

    Each token draws Gumbel noise over log-weights p_e ~ rank^-s and keeps its top-k experts
    (sampling k distinct experts without replacement, proportional to p). Returns the int64
    row offsets [experts+1] of the expert-sorted activation matrix."""
    rng = np.random.default_rng(seed)
    ranks = np.arange(1, experts + 1, dtype=np.float64)
    logp = -zipf_s * np.log(ranks)
    logp -= np.log(np.exp(logp).sum())
    g = rng.gumbel(size=(tokens, experts)) + logp[None, :]
    top = np.argsort(-g, axis=1)[:, :topk]
    counts = np.bincount(top.reshape(-1), minlength=experts).astype(np.int64)
    offsets = np.zeros(experts + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    return offsets


def moe(rows_w_per_expert: int = MOE_FFN, hidden: int = MOE_HIDDEN):
    """Expert-sorted activations X[sum M_g, hidden], stacked expert weights W[G*ffn, hidden]
    and the row offsets of X per expert."""
    offsets = moe_routing()
    total = int(offsets[-1])
    x = normal_bf16((total, hidden), SEEDS["moe_x"])
    w = normal_bf16((MOE_EXPERTS * rows_w_per_expert, hidden), SEEDS["moe_w"])
    return x, w, offsets


# Exponent spreads (binades between a block's largest and smallest nonzero value) around the
# limits where a 16-term sum needs more than binary32's 24 or binary64's 53 bits, up to the
# whole finite range.
WIDE_SPREADS = (0, 6, 11, 12, 13, 14, 16, 24, 25, 26, 40, 41, 42, 60, 120, 253)


def exponent_spread_bf16(tokens: int, cols: int, seed: int, spreads=WIDE_SPREADS) -> np.ndarray:
    """BF16 bits [tokens, cols] built per 16-token block of each column: a top exponent field
    F (mostly mid-range, sometimes 249..251 or very small) and a spread s drawn from `spreads`;
    fields uniform in [F - s, F] with F present, random signs and mantissas, about 5% exact
    zeros; fields that fall to 0 or below give subnormals. Used to exercise blocks whose
    16-term sums need more bits than binary32 or binary64 hold."""
    if tokens % 16:
        raise ValueError("tokens must be a multiple of 16")
    rng = np.random.default_rng(seed)
    nb = tokens // 16
    spread = rng.choice(np.asarray(spreads, dtype=np.int64), size=(nb, cols))
    top = rng.integers(60, 200, size=(nb, cols))
    edge = rng.random((nb, cols))
    top = np.where(edge < 0.1, rng.integers(249, 252, size=(nb, cols)), top)
    top = np.where((edge >= 0.1) & (edge < 0.15), rng.integers(1, 14, size=(nb, cols)), top)
    field = top[:, None, :] - rng.integers(0, spread[:, None, :] + 1, size=(nb, 16, cols))
    first = rng.integers(0, 16, size=(nb, cols))
    field[np.arange(nb)[:, None], first, np.arange(cols)[None, :]] = top
    field = np.clip(field, 0, 254)
    mant = rng.integers(0, 128, size=(nb, 16, cols))
    mant = np.where(field == 0, np.maximum(mant, 1), mant)          # field 0: nonzero subnormal
    sign = rng.integers(0, 2, size=(nb, 16, cols))
    bits = (sign << 15) | (field << 7) | mant
    bits = np.where(rng.random((nb, 16, cols)) < 0.05, 0, bits)
    return bits.reshape(tokens, cols).astype(np.uint16)


def pad_offsets(offsets, multiple: int = 64) -> np.ndarray:
    """Offsets of the same groups with each group's size rounded up to a multiple (the padded
    token layout of the expert backward pass: every expert's tokens start on a 64-token
    boundary)."""
    sizes = np.diff(np.asarray(offsets, dtype=np.int64))
    padded = (sizes + multiple - 1) // multiple * multiple
    out = np.zeros(len(sizes) + 1, dtype=np.int64)
    np.cumsum(padded, out=out[1:])
    return out


def scatter_rows(bits: np.ndarray, offsets, padded_offsets) -> np.ndarray:
    """Rows of group g moved from offsets[g].. to padded_offsets[g]..; padding rows are zero."""
    out = np.zeros((int(padded_offsets[-1]), bits.shape[1]), dtype=bits.dtype)
    for g in range(len(offsets) - 1):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        out[int(padded_offsets[g]):int(padded_offsets[g]) + hi - lo] = bits[lo:hi]
    return out


def moe_backward(x_bits: np.ndarray, offsets, ffn: int = MOE_FFN, pad: int = 64):
    """The expert layer's backward inputs in the padded token layout: X and the output gradient
    dY[tokens, ffn] ~ N(0, 1e-3) (its rows of real tokens; padding rows zero), and the padded
    offsets."""
    off_pad = pad_offsets(offsets, pad)
    dy = normal_bf16((int(offsets[-1]), ffn), SEEDS["moe_dy"], std=1e-3)
    return scatter_rows(x_bits, offsets, off_pad), scatter_rows(dy, offsets, off_pad), off_pad



def exponent_spread_f32(tokens: int, cols: int, seed: int, spreads=WIDE_SPREADS) -> np.ndarray:
    """float32 [tokens, cols] built like exponent_spread_bf16 with 23 random mantissa bits:
    per 16-token block of a column a top exponent field and a spread, fields uniform below the
    top (subnormals where they reach 0), random signs, about 5% exact zeros."""
    if tokens % 16:
        raise ValueError("tokens must be a multiple of 16")
    rng = np.random.default_rng(seed)
    nb = tokens // 16
    spread = rng.choice(np.asarray(spreads, dtype=np.int64), size=(nb, cols))
    top = rng.integers(60, 200, size=(nb, cols))
    edge = rng.random((nb, cols))
    top = np.where(edge < 0.1, rng.integers(249, 252, size=(nb, cols)), top)
    top = np.where((edge >= 0.1) & (edge < 0.15), rng.integers(1, 14, size=(nb, cols)), top)
    field = top[:, None, :] - rng.integers(0, spread[:, None, :] + 1, size=(nb, 16, cols))
    first = rng.integers(0, 16, size=(nb, cols))
    field[np.arange(nb)[:, None], first, np.arange(cols)[None, :]] = top
    field = np.clip(field, 0, 254).astype(np.uint32)
    mant = rng.integers(0, 1 << 23, size=(nb, 16, cols)).astype(np.uint32)
    mant = np.where(field == 0, np.maximum(mant, 1), mant).astype(np.uint32)
    sign = rng.integers(0, 2, size=(nb, 16, cols)).astype(np.uint32)
    bits = (sign << np.uint32(31)) | (field << np.uint32(23)) | mant
    bits = np.where(rng.random((nb, 16, cols)) < 0.05, np.uint32(0), bits).astype(np.uint32)
    return bits.reshape(tokens, cols).view(np.float32)


def hadamard_edge_blocks_bf16(seed: int = 0) -> np.ndarray:
    """BF16 bits [16 * n, 1]: one 16-token block per column entry of a list of hand-made
    blocks for the Hadamard transform's corner cases: all zeros (some -0), a pair that cancels,
    a lone value, a value and its negation among zeros, tiny values far below large ones
    (1, 2^-24, 2^-70 as in a tie broken by a far term), exact ties next to cancelling far
    terms, sums one to three bits wider than binary64, the smallest subnormal, the largest
    finite values (sums beyond binary32's range), every exponent field once, and random
    blocks with one term 100 or more binades below the rest. Returned as rows of one column
    per block stacked along tokens."""
    rng = np.random.default_rng(seed)

    def b(vals):
        v = np.zeros(16, np.float32)
        v[:len(vals)] = np.asarray(vals, np.float32)
        return f32_to_bf16_bits(v)

    blocks = [
        np.zeros(16, np.uint16),
        np.full(16, 0x8000, np.uint16),                                   # all -0
        np.where(np.arange(16) % 3 == 0, 0x8000, 0).astype(np.uint16),
        b([1.0, 1.0]), b([1.0, -1.0]), b([3.0]), b([0.0, -5.0]),
        b([1.0, 2.0 ** -24, 2.0 ** -70]), b([1.0, -(2.0 ** -24), 2.0 ** -70]),
        b([1.0, 2.0 ** -24, -(2.0 ** -70)]), b([2.0 ** 100, 2.0 ** -100, 2.0 ** -126]),
        b([1.0, 2.0 ** -24, 2.0 ** -70, -(2.0 ** -70)]),                 # exact ties, far terms
        b([1.0, 2.0 ** -23, 2.0 ** -24, 2.0 ** -70, -(2.0 ** -70)]),
        b([1.0, 2.0 ** -24, 2.0 ** -53]), b([1.0, 2.0 ** -24, 2.0 ** -54]),  # 54..56-bit sums
        b([1.0, 2.0 ** -24, 2.0 ** -55]), b([1.0, 2.0 ** -24, -(2.0 ** -53)]),
        np.array([1] + [0] * 15, np.uint16),                             # 2^-133
        np.array([0x8001] + [1] * 15, np.uint16),
        np.full(16, 0x7F7F, np.uint16),                                   # largest finite
        np.where(np.arange(16) % 2 == 0, 0x7F7F, 0xFF7F).astype(np.uint16),
        np.array([0x7F7F, 0x0001] + [0] * 14, np.uint16),
    ]
    fields = np.arange(0, 255, dtype=np.uint16)                          # every exponent field
    fb = ((fields << 7) | rng.integers(0, 128, fields.size).astype(np.uint16)).astype(np.uint16)
    fb = np.concatenate([fb, np.zeros((-fb.size) % 16, np.uint16)])
    blocks += list(fb.reshape(-1, 16))
    for _ in range(48):
        v = (rng.integers(100, 140, 16) << 7) | rng.integers(0, 128, 16)
        v[rng.integers(0, 16)] = rng.integers(0, 20) << 7 | rng.integers(1, 128)
        v |= rng.integers(0, 2, 16) << 15
        blocks.append(v.astype(np.uint16))
    return np.concatenate(blocks).astype(np.uint16).reshape(-1, 1)
