"""GPU parity of the MXFP4 path (E8M0 scale per 32 elements): quantization bit-exact against
the oracle (RN and SR, BF16 and FP32, ragged shapes, every exponent range)."""
import numpy as np
import pytest
import torch

import bit_block_scaled_quantize_amd as nv
import oracle
import workloads
from helpers import assert_bytes_equal, f32, log, to_device_bf16, to_device_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _host(q):
    torch.cuda.synchronize()
    return q.codes.cpu().numpy(), q.scales_by_row().cpu().numpy()


def _same(q, ref, what):
    c, s = _host(q)
    assert_bytes_equal(c, ref[0], what + " codes")
    assert_bytes_equal(s, ref[1], what + " scales")


@pytest.mark.parametrize("shape", [(1, 32), (3, 96), (37, 160), (130, 2048), (64, 5120), (257, 2688)])
@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_mx_quantize_bf16(shape, rounding):
    log(f"mx bf16 {shape} {rounding}")
    bits = workloads.with_outliers_bf16(shape, 700 + shape[0])
    q = nv.mx_quantize(to_device_bf16(bits), rounding, seed=0x5EED, offset=3)
    _same(q, oracle.quantize_mxfp4(f32(bits), rounding, seed=0x5EED, offset=3), f"mx {shape} {rounding}")


@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_mx_quantize_fp32_strided_and_wide_exponents(rounding):
    log(f"mx fp32 {rounding}")
    rng = np.random.default_rng(17)
    rows, cols, ld = 45, 192, 200
    x = (rng.standard_normal((rows, ld)) * np.ldexp(1.0, rng.integers(-150, 126, (rows, 1)))).astype(np.float32)
    x[0, :32] = 0.0
    x[1, :32] = -0.0
    x[2, 5] = np.float32(3.0e38)
    x[3, :64] = np.float32(2.0 ** -149)
    dev = to_device_f32(x)[:, :cols]
    q = nv.mx_quantize(dev, rounding, seed=99, offset=1 << 33)
    _same(q, oracle.quantize_mxfp4(x[:, :cols], rounding, seed=99, offset=1 << 33), f"mx fp32 {rounding}")


@pytest.mark.parametrize("dtype,shape", [("fp32", (64, 96)), ("fp32", (32, 2560)), ("bf16", (256, 32)),
                                         ("bf16", (96, 1408))])
def test_mx_quantize_contiguous_short_and_partial_rows(dtype, shape):
    """Contiguous FP32 and BF16 inputs, rows down to one 32-block and rows that end inside a
    128-column K step: every scale lands at its row and block of the K-step layout."""
    log(f"mx flat {dtype} {shape}")
    if dtype == "fp32":
        x = np.random.default_rng(shape[1]).standard_normal(shape).astype(np.float32)
        dev = to_device_f32(x)
    else:
        x = workloads.with_outliers_bf16(shape, 900 + shape[0])
        dev = to_device_bf16(x)
        x = f32(x)
    for rounding in ("rn", "sr"):
        q = nv.mx_quantize(dev, rounding, seed=21, offset=5)
        _same(q, oracle.quantize_mxfp4(x, rounding, seed=21, offset=5), f"mx flat {dtype} {shape} {rounding}")


def test_mx_quantize_every_bf16_pattern():
    # all 65536 BF16 bit patterns except NaN/Inf, in blocks with a shared top exponent spread
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    e = (u >> 7) & 0xFF
    u = u[e != 0xFF]
    n = len(u) // 32 * 32
    bits = u[:n].reshape(-1, 128)[: (n // 128)]
    q = nv.mx_quantize(to_device_bf16(bits), "rn")
    _same(q, oracle.quantize_mxfp4(f32(bits), "rn"), "every bf16")


def test_mx_validation_errors():
    x = torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nv.NVFP4Error):
        nv.mx_quantize(x)                                  # cols % 32


def _mx_pair(m, n, k, seed):
    a_bits = workloads.with_outliers_bf16((m, k), seed)
    b_bits = workloads.normal_bf16((n, k), seed + 1, std=0.02)
    qa = nv.mx_quantize(to_device_bf16(a_bits), "rn")
    qb = nv.mx_quantize(to_device_bf16(b_bits), "sr", seed=4, offset=2)
    ra = oracle.quantize_mxfp4(f32(a_bits))
    rb = oracle.quantize_mxfp4(f32(b_bits), "sr", seed=4, offset=2)
    _same(qa, ra, "A")
    _same(qb, rb, "B")
    return qa, qb, oracle.dequantize_mxfp4(*ra), oracle.dequantize_mxfp4(*rb)


@pytest.mark.parametrize("mnk", [(1, 1, 128), (37, 70, 256), (256, 256, 128), (300, 520, 640),
                                 (513, 1024, 2688), (1000, 33, 5120)])
def test_mx_gemm_within_bound(mnk):
    from helpers import assert_gemm_within_bound
    m, n, k = mnk
    log(f"mx gemm {mnk}")
    qa, qb, ah, bh = _mx_pair(m, n, k, 800 + m + k)
    out = torch.full((m, n + 3), -5.0, device="cuda")
    nv.mx_gemm(qa, qb, out=out[:, :n])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, n:] == -5.0)
    assert_gemm_within_bound(o[:, :n], ah, bh, f"mx gemm {mnk}")


def test_mx_gemm_unsupported_k():
    qa = nv.MXFP4Tensor.empty(16, 96)
    qb = nv.MXFP4Tensor.empty(16, 96)
    with pytest.raises(nv.NVFP4Error):
        nv.mx_gemm(qa, qb)


@pytest.mark.parametrize("shape", [(32, 1), (64, 3), (96, 130), (256, 128), (288, 257), (2048, 640)])
@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_mx_quantize_columns_bf16(shape, rounding):
    """x^T quantized without materializing it: equal to the oracle's row-wise MXFP4 of x^T
    (ragged column tiles, rows not a multiple of the 256-row tile, SR counters of the output)."""
    log(f"mx columns bf16 {shape} {rounding}")
    bits = workloads.with_outliers_bf16(shape, 760 + shape[1])
    q = nv.mx_quantize_columns(to_device_bf16(bits), rounding, seed=0x5EED, offset=9)
    ref = oracle.quantize_mxfp4(np.ascontiguousarray(f32(bits).T), rounding, seed=0x5EED, offset=9)
    _same(q, ref, f"mx columns {shape} {rounding}")


@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_mx_quantize_columns_fp32_strided_and_every_exponent(rounding):
    """FP32 input with a row stride and an odd column count; and every finite BF16 pattern laid
    out in columns (every exponent range, subnormals, zeros)."""
    log(f"mx columns fp32 strided {rounding}")
    rng = np.random.default_rng(77)
    full = (rng.standard_normal((160, 100)) * np.exp2(rng.integers(-40, 40, (160, 1)))).astype(np.float32)
    x = full[:, :77]
    q = nv.mx_quantize_columns(to_device_f32(full)[:, :77], rounding, seed=3, offset=1 << 40)
    _same(q, oracle.quantize_mxfp4(np.ascontiguousarray(x.T), rounding, seed=3, offset=1 << 40), "mx columns fp32")
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    u = u[((u >> 7) & 0xFF) != 0xFF]
    n = len(u) // 2048 * 2048
    bits = np.random.default_rng(2).permutation(u[:n]).reshape(-1, 64)          # [1020, 64]
    bits = bits[: len(bits) // 32 * 32]
    log(f"mx columns every bf16 pattern {rounding}")
    q = nv.mx_quantize_columns(to_device_bf16(bits), rounding, seed=5)
    _same(q, oracle.quantize_mxfp4(np.ascontiguousarray(f32(bits).T), rounding, seed=5), "mx columns every pattern")


def test_mx_columns_feed_the_backward_gemms():
    """The dgrad and wgrad operands made by the column quantization give the same GEMMs as the
    row-wise quantization of torch's transposes (bit-identical operands, identical outputs)."""
    log("mx columns in the backward GEMMs")
    w = to_device_bf16(workloads.normal_bf16((256, 384), 780, std=0.02))      # W [N, K]
    dy = to_device_bf16(workloads.normal_bf16((512, 256), 781, std=1e-3))     # dY [M, N]
    qwt_c = nv.mx_quantize_columns(w, "rn")                                  # W^T [K, N]
    qwt_t = nv.mx_quantize(w.t().contiguous(), "rn")
    qdy = nv.mx_quantize(dy, "sr", seed=1)
    a, b = nv.mx_gemm(qdy, qwt_c), nv.mx_gemm(qdy, qwt_t)
    torch.cuda.synchronize()
    assert torch.equal(qwt_c.codes, qwt_t.codes) and torch.equal(qwt_c.scales_by_row(), qwt_t.scales_by_row())
    assert torch.equal(a, b)
