"""Philox4x32-10 counter-based generator and the per-block random bytes of stochastic
rounding (oracle; test infrastructure only).

The pages only say that gradients are rounded stochastically so that the rounding is
unbiased in expectation ("Nemotron NVFP4" explainer, "Why 4-bit training normally falls
apart - and the three fixes"; artiverse.ca stabilizer paragraph). The generator is a reading:
Philox4x32 with 10 rounds as published by Salmon, Moraes, Dror and Shaw, "Parallel random
numbers: as easy as 1, 2, 3" (SC'11). One round maps counter (c0,c1,c2,c3) and key (k0,k1) to
  (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0))
with M0 = 0xD2511F53, M1 = 0xCD9E8D57; between rounds the key is bumped by the Weyl
constants (0x9E3779B9, 0xBB67AE85).

Reading R10 (counter mapping): the quantization block with linear index b (row-major over
the OUTPUT tensor's [rows, cols/16] block grid) uses key = (lo32(seed), hi32(seed)) and
counter = (lo32(b), hi32(b), lo32(offset), hi32(offset)). The 128 output bits give one byte
per element: element j of the block (j = 0..15 along the quantized dimension) uses byte
j % 4 (little-endian) of word j // 4.
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorized Philox4x32-10. All arguments are uint32 scalars or arrays (broadcast);
    returns four uint32 arrays."""
    c0, c1, c2, c3 = (np.asarray(v, dtype=np.uint64) & _MASK32 for v in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK32
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        p0 = m0 * c0                      # < 2^64, exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return tuple(v.astype(np.uint32) for v in (c0, c1, c2, c3))


def block_random_bytes(block_index, seed: int, offset: int) -> np.ndarray:
    """Random bytes [n, 16] (uint8) for the quantization blocks with the given linear
    indices (R10)."""
    b = np.asarray(block_index, dtype=np.uint64).reshape(-1)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    offset = int(offset) & 0xFFFFFFFFFFFFFFFF
    w = philox4x32_10(b & _MASK32, b >> np.uint64(32),
                      np.uint64(offset & 0xFFFFFFFF), np.uint64(offset >> 32),
                      np.uint64(seed & 0xFFFFFFFF), np.uint64(seed >> 32))
    words = np.stack([np.broadcast_to(x, b.shape) for x in w], axis=1)  # [n, 4]
    out = np.empty((b.size, 16), dtype=np.uint8)
    for j in range(16):
        out[:, j] = (words[:, j // 4] >> np.uint32(8 * (j % 4))) & np.uint32(0xFF)
    return out
