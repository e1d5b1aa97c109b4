"""GPU parity of the quantize kernels with the oracle: bit-exact codes, scales and tensor
scales, on ragged shapes, both input dtypes, both rounding modes, segments, and the edge
cases of the scale rule (zero tensors, subnormal inputs and amax, huge values, signed
zeros). All calls go through the C ABI via the binding."""
import numpy as np
import pytest
import torch

import bit_block_scaled_quantize_amd as nv
import oracle
import workloads
from helpers import (assert_bytes_equal, assert_quant_equal, f32, host, log, to_device_bf16,
                     to_device_f32)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(shape, seed, std=1.0, outliers=True):
    return (workloads.with_outliers_bf16(shape, seed) if outliers
            else workloads.normal_bf16(shape, seed, std))


SHAPES = [(1, 16), (3, 48), (17, 1040), (64, 256), (130, 80), (33, 2048)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_1x16_bf16(shape, rounding):
    log(f"1x16 bf16 {shape} {rounding}")
    bits = _bits(shape, 1000 + shape[0] * 7 + shape[1])
    q, _ = nv.quantize(to_device_bf16(bits), "1x16", rounding, seed=0xABCDEF0123, offset=77)
    ref = oracle.quantize_1x16(f32(bits), rounding, seed=0xABCDEF0123, offset=77)
    assert_quant_equal(host(q), ref, f"1x16 {shape} {rounding}")


@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_1x16_fp32_with_row_stride(rounding):
    log(f"1x16 fp32 strided {rounding}")
    rng = np.random.default_rng(5)
    full = (rng.standard_normal((40, 160)) * rng.uniform(0.01, 100, (40, 1))).astype(np.float32)
    x = full[:, :96]
    xd = to_device_f32(full)[:, :96]
    q, _ = nv.quantize(xd, "1x16", rounding, seed=3, offset=(5 << 32) | 1)
    ref = oracle.quantize_1x16(x, rounding, seed=3, offset=(5 << 32) | 1)
    assert_quant_equal(host(q), ref, f"1x16 fp32 {rounding}")


def test_1x16_all_bf16_patterns():
    # Every finite BF16 pattern, 16 per block, quantized against several tensor amax values
    # (amax_in), so every element meets many block and tensor scales.
    log("1x16 exhaustive bf16 patterns")
    pats = np.arange(65536, dtype=np.uint32)
    expo = (pats >> 7) & 0xFF
    rng = np.random.default_rng(9)
    # exponent windows so that each trial spans a different set of block / tensor scales
    windows = [(0, 254), (117, 137), (200, 254), (0, 30), (120, 130)]
    for trial, (lo, hi) in enumerate(windows):
        sel = pats[(expo >= lo) & (expo <= hi)].astype(np.uint16)
        sel = sel if trial == 0 else sel[rng.permutation(len(sel))]
        sel = np.concatenate([sel, np.zeros((-len(sel)) % 256, np.uint16)])
        bits = sel.reshape(-1, 256)
        x = f32(bits)
        amax = oracle.amax(x)
        for rnd in ("rn", "sr"):
            for use_amax_in in (False, True):
                amax_d = torch.from_numpy(amax).cuda() if use_amax_in else None
                q, _ = nv.quantize(to_device_bf16(bits), "1x16", rnd, seed=11, offset=trial, amax=amax_d)
                ref = oracle.quantize_1x16(x, rnd, seed=11, offset=trial, amax_vals=amax)
                assert_quant_equal(host(q), ref, f"exhaustive window {lo}-{hi} {rnd} amax_in={use_amax_in}")


def test_1x16_scale_edge_cases():
    cases = {
        "zeros": np.zeros((4, 32), np.float32),
        "signed_zeros": np.where(np.arange(128).reshape(4, 32) % 3 == 0, -0.0, 0.0).astype(np.float32),
        "subnormal_amax": np.full((2, 32), 1e-40, np.float32) * np.sign(np.arange(64).reshape(2, 32) - 31.5).astype(np.float32),
        "tiny_blocks": np.concatenate([np.full((1, 16), 1e4, np.float32), np.full((1, 16), 1e-4, np.float32)], axis=1),
        "huge": np.array([[3.0e38, -1e38] + [1.0] * 14], np.float32),
        "one_hot": np.eye(16, 64, dtype=np.float32) * 5.0,
        "midpoints": np.array([[0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 2], np.float32),
    }
    for name, x in cases.items():
        for rnd in ("rn", "sr"):
            log(f"1x16 edge {name} {rnd}")
            q, _ = nv.quantize(to_device_f32(x), "1x16", rnd, seed=1, offset=2)
            ref = oracle.quantize_1x16(x, rnd, seed=1, offset=2)
            assert_quant_equal(host(q), ref, f"edge {name} {rnd}")


def test_1x16_segments_and_amax_api():
    log("1x16 segments")
    bits = _bits((200, 96), 44)
    seg = np.array([0, 0, 16, 17, 100, 100, 200], np.int64)      # empty and ragged segments
    segd = torch.from_numpy(seg).cuda()
    x = f32(bits)
    a = nv.amax(to_device_bf16(bits), segd)
    torch.cuda.synchronize()
    assert_bytes_equal(a.cpu().numpy().view(np.uint32), oracle.amax(x, seg).view(np.uint32), "segment amax")
    for rnd in ("rn", "sr"):
        q, _ = nv.quantize(to_device_bf16(bits), "1x16", rnd, seed=9, offset=0, segments=segd)
        ref = oracle.quantize_1x16(x, rnd, seed=9, offset=0, segments=seg)
        assert_quant_equal(host(q), ref, f"segments {rnd}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("nseg,pad", [(7, 0), (300, 16), (1500, 0), (3000, 8)])
def test_segment_amax_many_segments(dtype, nseg, pad):
    """Per-segment maxima with many segments, empty ones included: offset tables searched in
    LDS (up to 1023 segments) and in global memory, workgroups whose rows cross more segments
    than their window of per-segment maxima, rows with a stride (pad columns between rows).
    Every segment's maximum bit-exact against the oracle."""
    log(f"segment amax nseg={nseg} pad={pad} {dtype}")
    rng = np.random.default_rng(nseg + pad)
    rows, cols = 6000, 48
    seg = np.concatenate([[0], np.sort(rng.integers(0, rows + 1, nseg - 1)), [rows]]).astype(np.int64)
    x = f32(workloads.normal_bf16((rows, cols), 700 + nseg))
    x *= (np.float32(2.0) ** rng.integers(-30, 30, rows).astype(np.float32))[:, None]
    x = f32(workloads.f32_to_bf16_bits(x)) if dtype == "bf16" else x
    full = np.zeros((rows, cols + pad), np.float32)
    full[:, :cols] = x
    full[:, cols:] = 1e30                                     # must not count: past each row
    if dtype == "bf16":
        dev = to_device_bf16(workloads.f32_to_bf16_bits(full))[:, :cols]
    else:
        dev = torch.from_numpy(full).cuda()[:, :cols]
    a = nv.amax(dev, torch.from_numpy(seg).cuda())
    torch.cuda.synchronize()
    assert_bytes_equal(a.cpu().numpy().view(np.uint32), oracle.amax(x, seg).view(np.uint32),
                       f"segment amax nseg={nseg}")


@pytest.mark.parametrize("shape", [(16, 16), (48, 80), (64, 1024), (160, 528)])
def test_16x16_with_transpose(shape):
    log(f"16x16 {shape}")
    bits = _bits(shape, 2000 + shape[1], outliers=True)
    x = f32(bits)
    q, qt = nv.quantize(to_device_bf16(bits), "16x16", "rn", emit_transposed=True)
    ref = oracle.quantize_16x16(x)
    assert_quant_equal(host(q), ref, f"16x16 {shape}")
    reft = oracle.quantize_16x16(np.ascontiguousarray(x.T), amax_vals=oracle.amax(x))
    assert_quant_equal(host(qt), reft, f"16x16 transposed {shape}")


def test_16x16_fp32_segments():
    log("16x16 fp32 segments")
    rng = np.random.default_rng(8)
    x = rng.standard_normal((96, 64)).astype(np.float32) * np.repeat(rng.uniform(0.1, 10, 6), 16)[:, None].astype(np.float32)
    seg = np.array([0, 32, 32, 96], np.int64)
    q, _ = nv.quantize(to_device_f32(x), "16x16", "rn", segments=torch.from_numpy(seg).cuda())
    assert_quant_equal(host(q), oracle.quantize_16x16(x, segments=seg), "16x16 segments")


@pytest.mark.parametrize("shape", [(16, 1), (32, 7), (256, 129), (48, 513), (64, 200), (32, 130)])
@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_rht_quantize(shape, rounding):
    log(f"rht {shape} {rounding}")
    bits = _bits(shape, 3000 + shape[1], outliers=True)
    x = f32(bits)
    mask = workloads.wgrad_sign_mask()
    q = nv.rht_quantize(to_device_bf16(bits), mask, rounding, seed=0x5EED, offset=1 << 32)
    ref = oracle.rht_quantize(x, mask, rounding, seed=0x5EED, offset=1 << 32)
    assert_quant_equal(host(q), ref, f"rht {shape} {rounding}")
    a = nv.amax(to_device_bf16(bits), rht=True, sign_mask=mask)
    torch.cuda.synchronize()
    assert a.cpu().numpy()[0] == oracle.amax(oracle.rht_columnwise(x, mask))[0]


@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_rht_exponent_spread(rounding):
    """Blocks of every exponent spread up to the whole BF16 range (each side of the range
    tests of the binary32 and binary64 butterflies, and the exact path beyond), plus zeros,
    subnormals and fields up to 251, bit-exact against the oracle's correctly rounded
    transform."""
    log(f"rht exponent spread {rounding}")
    bits = workloads.exponent_spread_bf16(512, 272, 77)
    x = f32(bits)
    mask = workloads.wgrad_sign_mask()
    q = nv.rht_quantize(to_device_bf16(bits), mask, rounding, seed=0x5EED, offset=3)
    ref = oracle.rht_quantize(x, mask, rounding, seed=0x5EED, offset=3)
    assert_quant_equal(host(q), ref, f"rht spread {rounding}")
    a = nv.amax(to_device_bf16(bits), rht=True, sign_mask=mask)
    torch.cuda.synchronize()
    assert a.cpu().numpy()[0] == oracle.amax(oracle.rht_columnwise(x, mask))[0]


@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_rht_exponent_spread_fp32(rounding):
    """FP32 inputs with 23-bit mantissas and exponent spreads up to the whole range (the
    binary64 butterfly is exact only up to about 25 binades): bit-exact, amax too."""
    log(f"rht fp32 exponent spread {rounding}")
    x = workloads.exponent_spread_f32(256, 144, 79)
    mask = 0x6E04
    q = nv.rht_quantize(to_device_f32(x), mask, rounding, seed=0x5EED, offset=11)
    ref = oracle.rht_quantize(x, mask, rounding, seed=0x5EED, offset=11)
    assert_quant_equal(host(q), ref, f"rht fp32 spread {rounding}")
    a = nv.amax(to_device_f32(x), rht=True, sign_mask=mask)
    torch.cuda.synchronize()
    assert a.cpu().numpy()[0] == oracle.amax(oracle.rht_columnwise(x, mask))[0]


def _corner_block_columns(finite_only: bool):
    """The hand-made corner blocks as the columns of a [16, n] BF16 tensor; without the
    blocks whose transform exceeds the binary32 range when finite_only."""
    blocks = workloads.hadamard_edge_blocks_bf16(5).reshape(-1, 16)
    if finite_only:
        big = ((blocks & 0x7FFF) >= 0x7F00).any(axis=1)
        blocks = blocks[~big]
    return np.ascontiguousarray(blocks.T)


@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_rht_corner_blocks(rounding):
    """Ties broken by terms 46+ binades below, exact ties next to cancelling far terms, sums
    one to three bits wider than binary64, all-zero blocks with -0 inputs (their outputs are
    +0, so codes carry no sign), subnormals, one block per exponent field: bit-exact for
    several sign masks."""
    bits = _corner_block_columns(finite_only=True)
    x = f32(bits)
    for mask in (0, 0x6E04, 0xFFFF):
        log(f"rht corner blocks {rounding} mask {mask:#x}")
        q = nv.rht_quantize(to_device_bf16(bits), mask, rounding, seed=0x5EED, offset=2)
        ref = oracle.rht_quantize(x, mask, rounding, seed=0x5EED, offset=2)
        assert_quant_equal(host(q), ref, f"rht corner blocks {rounding} {mask:#x}")


def test_rht_corner_blocks_per_block_amax():
    """max|y| of each corner block alone, including blocks whose transform is beyond the
    binary32 range (infinite maximum), against the oracle."""
    bits = _corner_block_columns(finite_only=False)
    mask = 0x6E04
    want = np.abs(oracle.rht_columnwise(f32(bits), mask)).reshape(bits.shape[1], 16).max(axis=1)
    got = np.empty_like(want)
    for c in range(bits.shape[1]):
        col = np.ascontiguousarray(bits[:, c:c + 1])
        got[c] = nv.amax(to_device_bf16(col), rht=True, sign_mask=mask).cpu().numpy()[0]
    assert_bytes_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32), "corner block amax")


def test_rht_exponent_spread_per_block_amax():
    """max |y| of single 16-token blocks (one column each): the transform's largest output
    per block, exact against the oracle."""
    bits = workloads.exponent_spread_bf16(16, 48, 78)
    mask = workloads.wgrad_sign_mask()
    for c in range(48):
        col = np.ascontiguousarray(bits[:, c:c + 1])
        a = nv.amax(to_device_bf16(col), rht=True, sign_mask=mask)
        torch.cuda.synchronize()
        want = oracle.amax(oracle.rht_columnwise(f32(col), mask))[0]
        assert a.cpu().numpy()[0] == want, f"column {c}"


@pytest.mark.parametrize("shape,dtype,ld", [((16, 1), "bf16", 1), ((48, 513), "bf16", 514),
                                            ((256, 129), "fp32", 129), ((512, 272), "bf16", 272),
                                            ((4096, 1040), "bf16", 1040)])
def test_amax_pair(shape, dtype, ld):
    """nvfp4_amax_pair equals max|x| and max|Hx| of the oracle, and the two single maxima of
    the library, bit for bit (ragged column tiles, odd row strides, FP32 input)."""
    log(f"amax pair {shape} {dtype} ld={ld}")
    tokens, cols = shape
    bits = workloads.exponent_spread_bf16(tokens, ld, 90 + cols) if cols >= 16 else _bits((tokens, ld), 91)
    full = f32(bits)
    x = np.ascontiguousarray(full[:, :cols])
    mask = workloads.wgrad_sign_mask()
    if dtype == "bf16":
        dev = to_device_bf16(bits)[:, :cols]
    else:
        dev = to_device_f32(full)[:, :cols]
    got = nv.amax_pair(dev, mask)
    hx = nv.amax(dev, rht=True, sign_mask=mask)
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    want = np.array([oracle.amax(x)[0], oracle.amax(oracle.rht_columnwise(x, mask))[0]], np.float32)
    assert_bytes_equal(g.view(np.uint32), want.view(np.uint32), f"amax pair {shape}")
    assert g[1] == hx.cpu().numpy()[0]
    if cols % 16 == 0 and ld % (8 if dtype == "bf16" else 4) == 0:   # the rowwise amax's layout
        assert g[0] == nv.amax(dev).cpu().numpy()[0]


def _pair_vs_oracle(bits, what):
    mask = workloads.wgrad_sign_mask()
    got = nv.amax_pair(to_device_bf16(bits), mask)
    torch.cuda.synchronize()
    xf = f32(bits)
    want = np.array([oracle.amax(xf)[0], oracle.amax(oracle.rht_columnwise(xf, mask))[0]], np.float32)
    assert_bytes_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32), what)


@pytest.mark.parametrize("tokens,cols", [(2048, 1024), (1024, 1000), (4096, 160)])
def test_amax_pair_gaussian(tokens, cols):
    """The BF16 pair on Gaussian data at sizes spanning many tiles, with column tiles cut by the
    last column: bit for bit against the oracle."""
    log(f"amax pair gaussian {tokens}x{cols}")
    x = (np.random.default_rng(tokens + cols).standard_normal((tokens, cols)) * 1e-3).astype(np.float32)
    _pair_vs_oracle((x.view(np.uint32) >> 16).astype(np.uint16), f"amax pair {tokens}x{cols}")


def _planted_block(case):
    j = np.arange(16)
    if case == "zero":
        return np.zeros(16, np.uint16)
    if case.startswith("field"):                    # 3 binades wide, smallest exponent field f
        f = int(case[5:])
        return (((f + j % 3) << 7) | ((37 * j) & 0x7F) | np.where(j % 2 == 1, 0x8000, 0)).astype(np.uint16)
    spread = int(case[6:])                          # one value 2^spread above the others
    v = (((127 - spread) << 7) | ((29 * j) & 0x7F) | np.where(j % 3 == 1, 0x8000, 0)).astype(np.uint16)
    v[5] = 0x3F80
    return v


@pytest.mark.parametrize("case", ["zero", "field9", "field10", "field11", "spread11", "spread12",
                                  "spread13", "spread14", "spread30", "spread60", "spread118"])
@pytest.mark.parametrize("col", [0, 1])
def test_amax_pair_single_block(case, col):
    """One 16-token block beside a zero column, so its maximum is the result: all zero, tiny
    blocks (smallest exponent field 9, 10, 11), one value 11 to 118 binades above the others
    (the binary64 butterfly's range and past it, the exact sums), in the even and the odd
    column of a lane's pair."""
    log(f"amax pair single block {case} col {col}")
    bits = np.zeros((16, 2), np.uint16)
    bits[:, col] = _planted_block(case)
    _pair_vs_oracle(bits, f"single block {case} col {col}")


@pytest.mark.parametrize("n,k,G", [(48, 272, 3), (1856, 160, 2), (16, 32, 5), (320, 144, 3), (64, 400, 5)])
def test_16x16_segments_with_transpose(n, k, G):
    """An expert weight stack [G*n, k] quantized in 16x16 tiles with one tensor scale per
    expert, and every expert's transpose stacked [G*k, n] (the grouped activation-gradient
    GEMM's operand): bit-exact against the oracle, expert by expert."""
    log(f"16x16 segments + transpose n={n} k={k} G={G}")
    bits = workloads.with_outliers_bf16((G * n, k), 96 + n)
    x = f32(bits)
    x *= np.repeat(np.float32(2.0) ** np.arange(G, dtype=np.float32), n)[:, None]
    bits = workloads.f32_to_bf16_bits(x)
    x = f32(bits)
    seg = np.arange(G + 1, dtype=np.int64) * n
    q, qt = nv.quantize(to_device_bf16(bits), "16x16", "rn", emit_transposed=True,
                        segments=torch.from_numpy(seg).cuda())
    assert_quant_equal(host(q), oracle.quantize_16x16(x, segments=seg), "segmented W")
    codes_t, scales_t, gs_t = host(qt)
    for g in range(G):
        xg = x[g * n:(g + 1) * n]
        ref = oracle.quantize_16x16(np.ascontiguousarray(xg.T), amax_vals=oracle.amax(xg))
        assert_quant_equal((codes_t[g * k:(g + 1) * k], scales_t[g * k:(g + 1) * k], gs_t[g:g + 1]),
                           ref, f"W_{g}^T")


@pytest.mark.parametrize("rounding", ["rn", "sr"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("data", ["gauss", "spread"])
def test_rht_quantize_token_segments(rounding, dtype, data):
    """The expert-segmented transform-and-quantize (MoE weight gradient): one tensor scale per
    token range (an empty range included), bit-exact against the oracle; the segmented amax
    of the transformed tensor too. Gaussian inputs with outliers, or blocks of any exponent
    spread."""
    log(f"rht segments {rounding} {dtype} {data}")
    bits = (workloads.with_outliers_bf16((512, 272), 95) if data == "gauss"
            else workloads.exponent_spread_bf16(512, 272, 97))
    x = f32(bits)
    mask = workloads.wgrad_sign_mask()
    seg = np.array([0, 48, 48, 160, 496, 512], np.int64)
    segd = torch.from_numpy(seg).cuda()
    dev = to_device_bf16(bits) if dtype == "bf16" else to_device_f32(x)
    q = nv.rht_quantize(dev, mask, rounding, seed=0x5EED, offset=77, segments=segd)
    ref = oracle.rht_quantize_segments(x, mask, seg, rounding, seed=0x5EED, offset=77)
    assert_quant_equal(host(q), ref, f"rht segments {rounding} {dtype}")
    a = nv.amax(dev, segments=segd, rht=True, sign_mask=mask)
    torch.cuda.synchronize()
    y = oracle.rht_columnwise(x, mask)
    want = np.array([np.abs(y[:, seg[g]:seg[g + 1]]).max() if seg[g + 1] > seg[g] else 0.0
                     for g in range(len(seg) - 1)], np.float32)
    assert_bytes_equal(a.cpu().numpy().view(np.uint32), want.view(np.uint32), "segment rht amax")


def test_rht_fp32_masks():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((64, 40)) * 3).astype(np.float32)
    for mask in (0, 0xFFFF, 0x8001):
        log(f"rht fp32 mask {mask:#x}")
        q = nv.rht_quantize(to_device_f32(x), mask, "rn")
        assert_quant_equal(host(q), oracle.rht_quantize(x, mask, "rn"), f"rht fp32 {mask:#x}")


def test_dequantize_matches_oracle():
    log("dequantize")
    bits = _bits((64, 128), 55)
    q, _ = nv.quantize(to_device_bf16(bits), "1x16", "rn")
    y = nv.dequantize(q)
    torch.cuda.synchronize()
    ref = oracle.dequantize(*oracle.quantize_1x16(f32(bits))).astype(np.float32)
    assert_bytes_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32), "dequantize")


def test_empty_inputs_are_no_ops():
    """Zero rows (torch hands over NULL data pointers): every entry point returns without
    touching memory; the amax of nothing is 0."""
    log("empty inputs")
    mask = workloads.wgrad_sign_mask()
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, qt = nv.quantize(x, "16x16", "rn", emit_transposed=True)
    assert q.rows == 0 and qt.cols == 0
    nv.quantize(x, "1x16", "sr", seed=1)
    nv.rht_quantize(x, mask, "sr")
    nv.rht_rows_quantize(x, mask, "rn")
    nv.mx_quantize(x)
    a = torch.full((1,), 7.0, device="cuda")
    nv.amax(x, out=a)
    p = torch.full((2,), 7.0, device="cuda")
    nv.amax_pair(x, mask, out=p)
    assert nv.dequantize(q).shape == (0, 64)
    # GEMMs with no rows on either side
    qb, _ = nv.quantize(to_device_bf16(workloads.normal_bf16((32, 64), 5)), "1x16", "rn")
    assert nv.gemm(q, qb).shape == (0, 32)
    assert nv.gemm(qb, q).shape == (32, 0)
    assert nv.gemm_ex(q, qb, out_dtype=torch.bfloat16).shape == (0, 32)
    off = torch.zeros((3,), dtype=torch.int64, device="cuda")
    qw, _ = nv.quantize(to_device_bf16(workloads.normal_bf16((64, 64), 6)), "1x16", "rn",
                        segments=torch.tensor([0, 32, 64], dtype=torch.int64, device="cuda"))
    assert nv.grouped_gemm(off, nv.NVFP4Tensor.empty(0, 64, 2), qw, 32).shape == (0, 32)
    torch.cuda.synchronize()
    assert a.item() == 0.0 and p.cpu().tolist() == [0.0, 0.0]


def test_side_stream_matches_default_stream():
    """Every call takes the stream it is given: the layer's chain (amax pair, 1x16 SR, 16x16 with
    transpose, Hadamard along tokens, GEMM) issued on a side stream, with its inputs written on
    the default stream just before, gives bit-identical results to the same chain on the
    default stream. The stochastic bits depend on the counter offset only: the same seed and
    offset repeat the codes, another offset changes some."""
    log("side stream")
    mask = workloads.wgrad_sign_mask()
    x_bits = _bits((256, 512), 91)
    w_bits = _bits((384, 512), 92)

    def chain(stream):
        x = to_device_bf16(x_bits)
        w = to_device_bf16(w_bits)
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
            pair = nv.amax_pair(x, mask, stream=stream)
            qx, _ = nv.quantize(x, "1x16", "sr", seed=5, offset=9, amax=pair[0:1], stream=stream)
            qw, qwt = nv.quantize(w, "16x16", "rn", emit_transposed=True, stream=stream)
            qh = nv.rht_quantize(x, mask, "rn", amax=pair[1:2], stream=stream)
            d = nv.gemm(qx, qw, stream=stream)
        if stream is not None:
            stream.synchronize()
        torch.cuda.synchronize()
        return [t.cpu() for t in (pair, qx.codes, qx.scales, qw.codes, qwt.codes, qh.codes, qh.scales, d)]

    ref = chain(None)
    side = chain(torch.cuda.Stream())
    for i, (a, b) in enumerate(zip(ref, side)):
        assert torch.equal(a, b), f"output {i} differs between streams"
    x = to_device_bf16(x_bits)
    q1, _ = nv.quantize(x, "1x16", "sr", seed=5, offset=9)
    q2, _ = nv.quantize(x, "1x16", "sr", seed=5, offset=9)
    q3, _ = nv.quantize(x, "1x16", "sr", seed=5, offset=10)
    torch.cuda.synchronize()
    assert torch.equal(q1.codes, q2.codes)
    assert not torch.equal(q1.codes, q3.codes)
    assert torch.equal(q1.scales, q3.scales)


def test_side_stream_temporaries_outlive_the_call():
    """stream= without entering a stream context: the binding's workspaces and default outputs
    must belong to that stream. The side stream is held back by a sleep kernel so its kernels
    run after the call has returned and the workspace has been freed; the default stream then
    allocates buffers of the same sizes and fills them with garbage before anything is
    synchronized. Results must still equal the oracle (quantize's partial maxima live in its
    workspace; the BF16 GEMM's K-split halves live in its workspace)."""
    log("side stream temporaries")
    x_bits = _bits((512, 1024), 93)
    w_bits = _bits((320, 1024), 94)
    x_dev, w_dev = to_device_bf16(x_bits), to_device_bf16(w_bits)
    ref_x = oracle.quantize_1x16(f32(x_bits), "sr", seed=11, offset=4)
    ref_w = oracle.quantize_16x16(f32(w_bits))
    qx0, _ = nv.quantize(x_dev, "1x16", "sr", seed=11, offset=4)
    qw0, _ = nv.quantize(w_dev, "16x16", "rn")
    d_ref = nv.gemm_ex(qx0, qw0, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(side):
            torch.cuda._sleep(100_000_000)                  # tens of milliseconds, bounded
        qx, _ = nv.quantize(x_dev, "1x16", "sr", seed=11, offset=4, stream=side)
        qw, _ = nv.quantize(w_dev, "16x16", "rn", stream=side)
        d = nv.gemm_ex(qx, qw, out_dtype=torch.bfloat16, stream=side)
        junk = [torch.full((n,), 0x7F, dtype=torch.uint8, device="cuda")
                for n in (nv.workspace_size(nv.OP_QUANTIZE, 512, 1024),
                          nv.workspace_size(nv.OP_QUANTIZE, 320, 1024),
                          max(nv.workspace_size(nv.OP_GEMM_EX, 512, 320), 1), 512 * 512, 320 * 512)]
        side.synchronize()
        torch.cuda.synchronize()
        del junk
        assert_quant_equal(host(qx), ref_x, "side-stream 1x16 SR")
        assert_quant_equal(host(qw), ref_w, "side-stream 16x16")
        assert torch.equal(d.cpu(), d_ref.cpu()), "side-stream BF16 GEMM differs"
