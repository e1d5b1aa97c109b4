"""GPU parity of the Mosaic variant's pieces (R23): the rowwise Hadamard transform + 1x16
quantization of the activation gradient (bit-exact against the oracle, with its amax), and
the activation-gradient GEMM with both operands rotated along the output features (within the
bound of the FP64 GEMM of the oracle's operands; the rotation cancels)."""
import numpy as np
import pytest
import torch

import bit_block_scaled_quantize_amd as nv
import oracle
import workloads
from helpers import (assert_bytes_equal, assert_gemm_within_bound, assert_quant_equal, f32, host, log,
                     to_device_bf16, to_device_f32)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("shape", [(1, 16), (37, 160), (130, 2048), (64, 5120), (3, 2688)])
@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_rows_rht_quantize_bf16(shape, rounding):
    log(f"rows rht {shape} {rounding}")
    bits = workloads.with_outliers_bf16(shape, 900 + shape[0])
    mask = workloads.wgrad_sign_mask()
    dev = to_device_bf16(bits)
    q = nv.rht_rows_quantize(dev, mask, rounding, seed=0x5EED0003, offset=5)
    ref = oracle.rht_rowwise_quantize(f32(bits), mask, rounding, seed=0x5EED0003, offset=5)
    assert_quant_equal(host(q), ref, f"rows rht {shape} {rounding}")
    a = nv.amax(dev, rht=2, sign_mask=mask)
    torch.cuda.synchronize()
    want = oracle.amax(oracle.rht_rowwise(f32(bits), mask))
    assert_bytes_equal(a.cpu().numpy().view(np.uint32), want.view(np.uint32), "rotated amax")


@pytest.mark.parametrize("mask", [0, 0xFFFF, 0x8001, 0x6E04])
def test_rows_rht_quantize_fp32_strided(mask):
    log(f"rows rht fp32 {mask:#x}")
    rng = np.random.default_rng(mask + 3)
    x = (rng.standard_normal((45, 200)) * 3).astype(np.float32)
    x[2, 16:32] = 0.0
    dev = to_device_f32(x)[:, :192]
    q = nv.rht_rows_quantize(dev, mask, "sr", seed=9, offset=1 << 33)
    assert_quant_equal(host(q), oracle.rht_rowwise_quantize(x[:, :192], mask, "sr", seed=9, offset=1 << 33),
                       "rows rht fp32")


def test_rows_rht_every_bf16_pattern_blocks():
    # every finite BF16 pattern, 16 random ones per block: blocks of any exponent spread, most
    # beyond binary64's exact range, against the oracle's correctly rounded transform
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    u = u[((u >> 7) & 0xFF) != 0xFF]
    n = len(u) // 256 * 256
    rng = np.random.default_rng(1)
    bits = rng.permutation(u[:n]).reshape(-1, 256)
    q = nv.rht_rows_quantize(to_device_bf16(bits), 0x6E04, "rn")
    assert_quant_equal(host(q), oracle.rht_rowwise_quantize(f32(bits), 0x6E04, "rn"), "every bf16")


@pytest.mark.parametrize("mnk", [(64, 96, 128), (300, 520, 1024), (1000, 700, 1344)])
def test_mosaic_dgrad_gemm(mnk):
    """dX = dY W with dY rotated rowwise (SR) and W rotated along N (RN): the GEMM of the two
    is within bound of the FP64 product of the oracle's operands, and close to dY W."""
    m, k, n = mnk                                   # dY [m, n], W [n, k] -> dX [m, k]
    log(f"mosaic dgrad {mnk}")
    mask = workloads.wgrad_sign_mask()
    dy_bits = workloads.normal_bf16((m, n), 950 + m, std=1e-3)
    w_bits = workloads.normal_bf16((n, k), 951 + k, std=0.02)
    qa = nv.rht_rows_quantize(to_device_bf16(dy_bits), mask, "sr", seed=3, offset=0)
    qb = nv.rht_quantize(to_device_bf16(w_bits), mask, "rn")
    ra = oracle.rht_rowwise_quantize(f32(dy_bits), mask, "sr", seed=3, offset=0)
    rb = oracle.rht_quantize(f32(w_bits), mask, "rn")
    assert_quant_equal(host(qa), ra, "rotated dY")
    assert_quant_equal(host(qb), rb, "rotated W^T")
    d = nv.gemm(qa, qb)
    torch.cuda.synchronize()
    ah, bh = oracle.dequantize(*ra), oracle.dequantize(*rb)
    got = d.cpu().numpy()
    assert_gemm_within_bound(got, ah, bh, f"mosaic dgrad {mnk}")
    ref = f32(dy_bits).astype(np.float64) @ f32(w_bits).astype(np.float64)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 0.2


@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_rows_rht_wide_spreads(rounding):
    """Rowwise transform of blocks of any exponent spread: BF16 (rows of the spread
    generator's columns), FP32 with 23-bit mantissas, and the corner blocks as rows."""
    mask = 0x6E04
    bf = np.ascontiguousarray(workloads.exponent_spread_bf16(256, 64, 81).T)      # [64, 256]
    corner = workloads.hadamard_edge_blocks_bf16(6).reshape(-1, 16)
    corner = corner[~((corner & 0x7FFF) >= 0x7F00).any(axis=1)]
    corner = corner[: len(corner) // 4 * 4].reshape(-1, 64)                          # 4 blocks per row
    fp = np.ascontiguousarray(workloads.exponent_spread_f32(128, 48, 82).T)         # [48, 128]
    for name, dev, host_x in (("bf16 spread", to_device_bf16(bf), f32(bf)),
                              ("corner rows", to_device_bf16(corner), f32(corner)),
                              ("fp32 spread", to_device_f32(fp), fp)):
        log(f"rows rht {name} {rounding}")
        q = nv.rht_rows_quantize(dev, mask, rounding, seed=7, offset=3)
        assert_quant_equal(host(q), oracle.rht_rowwise_quantize(host_x, mask, rounding, seed=7, offset=3),
                           f"rows rht {name} {rounding}")
        a = nv.amax(dev, rht=2, sign_mask=mask)
        torch.cuda.synchronize()
        want = oracle.amax(oracle.rht_rowwise(host_x, mask))
        assert_bytes_equal(a.cpu().numpy().view(np.uint32), want.view(np.uint32), f"rotated amax {name}")
