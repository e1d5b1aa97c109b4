"""Shared helpers for the GPU parity tests: move seeded inputs to the device, pull NVFP4
buffers back, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads


def log(msg: str):
    print(f"[case] {msg}", flush=True)


def to_device_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_device_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(q):
    torch.cuda.synchronize()
    return (q.codes.cpu().numpy(), q.scales.cpu().numpy(), q.global_scale.cpu().numpy())


def assert_bytes_equal(got, want, what: str):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {got[i]!r} want {want[i]!r}")


def assert_quant_equal(gpu, ref, what: str, rows=None):
    """gpu = (codes, scales, gscale) from the device; ref = oracle triple (rows subset)."""
    gc, gs, gg = gpu
    rc, rs, rg = ref
    if rows is not None:
        gc, gs = gc[rows], gs[rows]
    assert_bytes_equal(gc, rc, what + " codes")
    assert_bytes_equal(gs, rs, what + " scales")
    assert_bytes_equal(gg.view(np.uint32), np.asarray(rg, np.float32).view(np.uint32), what + " global scale")


def assert_gemm_within_bound(d_gpu: np.ndarray, a_hat: np.ndarray, b_hat: np.ndarray, what: str,
                             rel: float = 1e-5):
    d64 = oracle.gemm_fp64(a_hat, b_hat)
    bound = oracle.gemm_bound(a_hat, b_hat, rel)
    err = np.abs(d_gpu.astype(np.float64) - d64)
    ok = err <= bound
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} elements out of bound; first {i}: "
                             f"gpu {d_gpu[i]!r} ref {d64[i]!r} bound {bound[i]!r}")
    return float((err / np.maximum(bound / rel, 1e-300)).max())


def f32(bits):
    return workloads.bf16_bits_to_f32(bits)
