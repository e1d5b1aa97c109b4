"""CPU test of the library's exact Hadamard path (csrc/rht_exact.h), compiled for the host.

The kernels send blocks whose 16 values span too many binades for a binary64 butterfly to be
exact through nvfp4::exact_quarter_sum. That code has no device builtins, so it is built here
as a host program (tests/host/rht_exact_host.hip) and compared bit for bit with the oracle's
transform on every kind of block: BF16 and FP32 blocks of any exponent spread, the corner
blocks (ties broken by far terms, exact ties, cancellations, signed zeros, underflow,
overflow) and ordinary Gaussian blocks."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def exact_bin(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("rht_exact") / "rht_exact_host")
    src = os.path.join(HERE, "host", "rht_exact_host.hip")
    subprocess.run([hipcc, "-x", "hip", "--cuda-host-only", "-O2", "-std=c++17", src, "-o", out],
                   check=True, capture_output=True, text=True)
    return out


def _run(binary, x, mask):
    """x[tokens, cols] float32 -> the host program's y[cols, tokens] (same layout as the oracle)."""
    x = np.ascontiguousarray(x, np.float32)
    t, c = x.shape
    blocks = x.T.reshape(c, t // 16, 16).reshape(-1, 16).view(np.uint32)
    lines = [str(len(blocks))] + [f"{mask:x} " + " ".join(f"{w:08x}" for w in b) for b in blocks]
    res = subprocess.run([binary], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True)
    got = np.array([int(w, 16) for w in res.stdout.split()], dtype=np.uint32)
    return got.view(np.float32).reshape(c, t)


def _check(binary, x, masks):
    for mask in masks:
        with np.errstate(over="ignore"):
            want = oracle.rht_columnwise(x, mask)
        got = _run(binary, x, mask)
        bad = np.argwhere(got.view(np.uint32) != want.view(np.uint32))
        assert bad.size == 0, (f"mask {mask:#x}: {len(bad)} mismatches, first {tuple(bad[0])}: "
                               f"got {got[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}")


def test_exact_path_corner_blocks(exact_bin):
    x = workloads.bf16_bits_to_f32(workloads.hadamard_edge_blocks_bf16(3))
    _check(exact_bin, x, (0, 0x6E04, 0xFFFF, 0x8001))


def test_exact_path_any_spread_bf16(exact_bin):
    x = workloads.bf16_bits_to_f32(workloads.exponent_spread_bf16(256, 32, 41))
    _check(exact_bin, x, (0, workloads.wgrad_sign_mask()))


def test_exact_path_any_spread_fp32(exact_bin):
    x = workloads.exponent_spread_f32(256, 32, 42)
    _check(exact_bin, x, (0x1234, 0xFFFF))
    tiny = np.zeros((32, 2), np.float32)                   # underflow to signed zeros
    tiny[0:3, 0] = [1.0, 1.0, -(2.0 ** -149)]
    tiny[16:19, 1] = [2.0 ** 60, -(2.0 ** 60), 2.0 ** -149]
    _check(exact_bin, tiny, (0, 0x0004))


def test_exact_path_gaussian_blocks(exact_bin):
    x = workloads.bf16_bits_to_f32(workloads.with_outliers_bf16((256, 32), 43))
    _check(exact_bin, x, (0, workloads.wgrad_sign_mask()))
