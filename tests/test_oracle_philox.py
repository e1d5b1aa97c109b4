"""Pins for the oracle's Philox4x32-10 (CPU only): the published known-answer vectors."""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(t, 16) for t in line.split()])
    return rows


def test_known_answer_vectors():
    rows = _kat()
    assert len(rows) == 3
    for v in rows:
        out = oracle.philox4x32_10(*v[:6])
        assert [int(o) for o in out] == v[6:]


def test_vectorized_matches_scalar():
    rng = np.random.default_rng(5)
    ctr = rng.integers(0, 2 ** 32, size=(64, 4), dtype=np.uint64)
    key = rng.integers(0, 2 ** 32, size=2, dtype=np.uint64)
    vec = oracle.philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], key[0], key[1])
    for i in range(64):
        sc = oracle.philox4x32_10(*ctr[i], key[0], key[1])
        assert [int(w[i]) for w in vec] == [int(s) for s in sc]


def test_block_bytes_layout():
    seed, offset = 0x0123456789ABCDEF, (7 << 32) | 9
    b = np.array([0, 1, (1 << 33) + 5])
    got = oracle.block_random_bytes(b, seed, offset)
    for i, bi in enumerate(b.tolist()):
        w = oracle.philox4x32_10(bi & 0xFFFFFFFF, bi >> 32, offset & 0xFFFFFFFF, offset >> 32,
                                 seed & 0xFFFFFFFF, seed >> 32)
        raw = b"".join(int(x).to_bytes(4, "little") for x in w)
        assert bytes(got[i]) == raw
