"""GPU parity of the linear-layer GEMM outputs (nvfp4_gemm_ex): BF16 output, accumulation into
an FP32 output and the fused output amax, against the oracle's FP64 reference (R18, R19) on
operands checked bit-exact first, and bit for bit against the FP32 GEMM where the readings fix
the relation (the BF16 output is the FP32 result rounded; the accumulated output is D_old plus
the FP32 result; the amax is the maximum of what was stored)."""
import numpy as np
import pytest
import torch

import bit_block_scaled_quantize_amd as nv
import oracle
import workloads
from helpers import assert_bytes_equal, assert_quant_equal, f32, host, log, to_device_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _operands(m, n, k, seed):
    a_bits = workloads.with_outliers_bf16((m, k), seed)
    w_bits = workloads.normal_bf16((n, k), seed + 1, std=0.02)
    qa, _ = nv.quantize(to_device_bf16(a_bits), "1x16", "rn")
    qb, _ = nv.quantize(to_device_bf16(w_bits), "1x16", "rn")
    ra, rb = oracle.quantize_1x16(f32(a_bits)), oracle.quantize_1x16(f32(w_bits))
    assert_quant_equal(host(qa), ra, "A")
    assert_quant_equal(host(qb), rb, "B")
    return qa, qb, oracle.dequantize(*ra), oracle.dequantize(*rb)


def _bf16_values(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16


# A last round of at most a quarter of the 256 CUs: 256 x 64 column quarters over all of K;
# (2304, 2560, 256), 90 tiles: split along K (workspace + fixup); K = 128: one step, no split;
# K % 64 != 0: the general kernel
SHAPES = [(300, 520, 512), (257, 33, 128), (1000, 700, 1344), (130, 257, 272), (64, 64, 2688),
          (2304, 2560, 256)]


@pytest.mark.parametrize("mnk", SHAPES)
def test_bf16_output_and_amax(mnk):
    m, n, k = mnk
    log(f"gemm_ex bf16 {mnk}")
    qa, qb, ah, bh = _operands(m, n, k, 300 + m + k)
    d32 = nv.gemm(qa, qb)
    amax = torch.full((1,), -1.0, device="cuda")
    d16 = nv.gemm_ex(qa, qb, out_dtype=torch.bfloat16, amax_out=amax)
    torch.cuda.synchronize()
    got = _bf16_values(d16).view(np.float32)
    # R18 against the FP64 reference
    bound = oracle.gemm_bf16_bound(ah, bh)
    assert np.all(np.abs(got.astype(np.float64) - oracle.gemm_fp64(ah, bh)) <= bound)
    # the FP32 result rounded once to BF16, bit for bit
    assert_bytes_equal(got.view(np.uint32), oracle.round_bf16(d32.cpu().numpy()).view(np.uint32), "bf16 = rn(fp32)")
    # R20: the maximum of the stored values
    assert amax.cpu().numpy()[0] == np.abs(got).max()


@pytest.mark.parametrize("mnk", SHAPES)
def test_fp32_output_amax_matches_plain_gemm(mnk):
    m, n, k = mnk
    log(f"gemm_ex fp32 {mnk}")
    qa, qb, ah, bh = _operands(m, n, k, 400 + n + k)
    d32 = nv.gemm(qa, qb).cpu().numpy()
    amax = torch.empty((1,), device="cuda")
    out = torch.full((m, n + 3), 7.0, device="cuda")
    nv.gemm_ex(qa, qb, out=out[:, :n], amax_out=amax)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, n:] == 7.0)
    assert_bytes_equal(o[:, :n].view(np.uint32), d32.view(np.uint32), "gemm_ex fp32 = gemm")
    assert amax.cpu().numpy()[0] == np.abs(d32).max()


@pytest.mark.parametrize("mnk", SHAPES)
def test_fp32_accumulate(mnk):
    m, n, k = mnk
    log(f"gemm_ex accumulate {mnk}")
    qa, qb, ah, bh = _operands(m, n, k, 500 + m + n)
    rng = np.random.default_rng(m * n)
    d_old = (rng.standard_normal((m, n)) * 0.5).astype(np.float32)
    d32 = nv.gemm(qa, qb).cpu().numpy()
    out = torch.from_numpy(d_old.copy()).cuda()
    amax = torch.empty((1,), device="cuda")
    nv.gemm_ex(qa, qb, out=out, accumulate=True, amax_out=amax)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # R19 against D_old + D64
    bound = oracle.gemm_accumulate_bound(d_old, ah, bh)
    assert np.all(np.abs(got.astype(np.float64) - oracle.gemm_accumulate_fp64(d_old, ah, bh)) <= bound)
    # one FP32 addition of the FP32 product, bit for bit
    assert_bytes_equal(got.view(np.uint32), (d_old + d32).view(np.uint32), "D_old + D")
    assert amax.cpu().numpy()[0] == np.abs(got).max()
    # a second accumulation adds again
    nv.gemm_ex(qa, qb, out=out, accumulate=True)
    torch.cuda.synchronize()
    assert_bytes_equal(out.cpu().numpy().view(np.uint32), ((d_old + d32) + d32).view(np.uint32), "twice")


def test_fp32_accumulate_keeps_subnormals():
    """D += A B^T (one K step, no split: each element gets one float atomic add) with a product of
    exact zeros on a D holding subnormals of both signs, normals and signed zeros: one IEEE
    addition per element, bit for bit (subnormals kept, -0 + 0 = +0)."""
    m, n, k = 300, 520, 128
    qa, _ = nv.quantize(to_device_bf16(workloads.normal_bf16((m, k), 3)), "1x16", "rn")
    qb, _ = nv.quantize(torch.zeros((n, k), dtype=torch.bfloat16, device="cuda"), "1x16", "rn")
    rng = np.random.default_rng(9)
    bits = rng.integers(1, 1 << 23, (m, n), dtype=np.uint32)              # subnormal magnitudes
    bits |= rng.integers(0, 2, (m, n)).astype(np.uint32) << 31
    d_old = bits.view(np.float32).copy()
    d_old[::7] = rng.standard_normal(d_old[::7].shape).astype(np.float32)
    d_old[1, :] = 0.0
    d_old[2, :] = -0.0
    out = torch.from_numpy(d_old.copy()).cuda()
    nv.gemm_ex(qa, qb, out=out, accumulate=True)
    d = nv.gemm(qa, qb)
    torch.cuda.synchronize()
    d = d.cpu().numpy()
    assert np.all(d == 0.0)
    assert_bytes_equal(out.cpu().numpy().view(np.uint32), (d_old + d).view(np.uint32), "subnormals")


def test_empty_output_clears_amax():
    full = nv.NVFP4Tensor.empty(16, 128)
    qa = nv.NVFP4Tensor(full.codes, full.scales, full.global_scale, 0, 128)   # M = 0
    qb, _ = nv.quantize(to_device_bf16(workloads.normal_bf16((32, 128), 7)), "1x16", "rn")
    amax = torch.full((1,), 5.0, device="cuda")
    out = torch.full((4, 32), 3.0, dtype=torch.bfloat16, device="cuda")
    nv.gemm_ex(qa, qb, out=out, out_dtype=torch.bfloat16, amax_out=amax)
    torch.cuda.synchronize()
    assert amax.cpu().numpy()[0] == 0.0
    assert torch.all(out == 3.0)                                         # nothing written


@pytest.mark.parametrize("shape", [(8192, 5120, 20480), (20480, 5120, 8192)])
def test_full_size_bf16_and_accumulate(shape):
    """The dense layer's activation-gradient and weight-gradient shapes (partial last rounds:
    128 tiles split along K through the workspace, 64 tiles cut into column quarters): BF16 = rn(FP32 result) and D_old + FP32 result on every
    element; the FP32 result itself is checked against the oracle on sampled elements by the
    dense GEMM tests."""
    m, n, k = shape
    log(f"gemm_ex full size {shape}")
    g = torch.Generator(device="cuda").manual_seed(m + n)
    a = (torch.randn((m, k), device="cuda", generator=g)).to(torch.bfloat16)
    b = (torch.randn((n, k), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    qa, _ = nv.quantize(a, "1x16", "rn")
    qb, _ = nv.quantize(b, "1x16", "rn")
    del a, b
    d32 = nv.gemm(qa, qb)
    amax = torch.empty((1,), device="cuda")
    d16 = nv.gemm_ex(qa, qb, out_dtype=torch.bfloat16, amax_out=amax)
    torch.cuda.synchronize()
    want16 = oracle.round_bf16(d32.cpu().numpy())
    got16 = _bf16_values(d16).view(np.float32)
    assert_bytes_equal(got16.view(np.uint32), want16.view(np.uint32), "full bf16")
    assert amax.cpu().numpy()[0] == np.abs(got16).max()
    del d16
    acc = torch.full((m, n), 0.25, device="cuda")
    nv.gemm_ex(qa, qb, out=acc, accumulate=True)
    torch.cuda.synchronize()
    assert_bytes_equal(acc.cpu().numpy().view(np.uint32),
                       (np.float32(0.25) + d32.cpu().numpy()).view(np.uint32), "full accumulate")
