"""GPU parity of the block-scaled GEMM and grouped GEMM: every output element within
1e-5 * sum_k |a||b| of the binary64 GEMM of the oracle's dequantized operands (operands are
first checked bit-exact against the oracle, so the reference uses the oracle's own bytes)."""
import numpy as np
import pytest
import torch

import bit_block_scaled_quantize_amd as nv
import oracle
import workloads
from helpers import (assert_gemm_within_bound, assert_quant_equal, f32, host, log,
                     to_device_bf16, to_device_f32)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pair(m, n, k, seed, rnd_a="rn", wblk="16x16"):
    a_bits = workloads.with_outliers_bf16((m, k), seed)
    w_bits = workloads.normal_bf16((n, k), seed + 1, std=0.02)
    qa, _ = nv.quantize(to_device_bf16(a_bits), "1x16", rnd_a, seed=5, offset=0)
    ra = oracle.quantize_1x16(f32(a_bits), rnd_a, seed=5, offset=0)
    assert_quant_equal(host(qa), ra, "A")
    if wblk == "16x16" and n % 16 == 0:
        qb, _ = nv.quantize(to_device_bf16(w_bits), "16x16", "rn")
        rb = oracle.quantize_16x16(f32(w_bits))
    else:
        qb, _ = nv.quantize(to_device_bf16(w_bits), "1x16", "rn")
        rb = oracle.quantize_1x16(f32(w_bits))
    assert_quant_equal(host(qb), rb, "B")
    return qa, qb, oracle.dequantize(*ra), oracle.dequantize(*rb)


def test_tiny_config_end_to_end():
    # 256 x 256 activations (1x16, RN) and weights (16x16, RN), GEMM 256^3.
    log("tiny end to end")
    a_bits, w_bits = workloads.tiny()
    qa, _ = nv.quantize(to_device_bf16(a_bits), "1x16", "rn")
    qw, qwt = nv.quantize(to_device_bf16(w_bits), "16x16", "rn", emit_transposed=True)
    ra = oracle.quantize_1x16(f32(a_bits))
    rw = oracle.quantize_16x16(f32(w_bits))
    assert_quant_equal(host(qa), ra, "tiny A")
    assert_quant_equal(host(qw), rw, "tiny W")
    assert_quant_equal(host(qwt), oracle.quantize_16x16(f32(w_bits).T.copy()), "tiny W^T")
    d = nv.gemm(qa, qw)
    torch.cuda.synchronize()
    assert_gemm_within_bound(d.cpu().numpy(), oracle.dequantize(*ra), oracle.dequantize(*rw), "tiny gemm")


@pytest.mark.parametrize("mnk", [(1, 1, 16), (17, 33, 48), (130, 257, 272), (64, 128, 512),
                                 (256, 200, 2688), (129, 130, 1040),
                                 # K % 64 == 0: the 256 x 256 LDS-staged kernel, with ragged
                                 # M/N edges and a partial last 128-wide K step
                                 (300, 520, 192), (257, 33, 64), (1000, 700, 1344),
                                 (513, 1024, 5120)])
def test_gemm_ragged(mnk):
    m, n, k = mnk
    log(f"gemm {mnk}")
    qa, qb, ah, bh = _pair(m, n, k, 100 + m + n + k)
    d = nv.gemm(qa, qb)
    torch.cuda.synchronize()
    assert_gemm_within_bound(d.cpu().numpy(), ah, bh, f"gemm {mnk}")


def test_gemm_output_row_stride_and_sr_operand():
    log("gemm ldd + SR operand")
    qa, qb, ah, bh = _pair(70, 90, 320, 7, rnd_a="sr", wblk="1x16")
    out = torch.full((70, 128), -7.0, dtype=torch.float32, device="cuda")
    nv.gemm(qa, qb, out=out[:, :90])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, 90:] == -7.0)
    assert_gemm_within_bound(o[:, :90], ah, bh, "gemm ldd")
    # odd row stride and a D that is not 16-byte aligned, neighbours untouched
    out2 = torch.full((70, 131), -7.0, dtype=torch.float32, device="cuda")
    nv.gemm(qa, qb, out=out2[:, 1:91])
    torch.cuda.synchronize()
    o2 = out2.cpu().numpy()
    assert np.all(o2[:, 0] == -7.0) and np.all(o2[:, 91:] == -7.0)
    assert np.array_equal(o2[:, 1:91], o[:, :90])


def test_gemm_k_split_tail_output_stride():
    """90 tiles of 256 x 256 on 256 CUs leave a last round of more than a quarter of them: those
    tiles are zeroed and split along K in two halves added with atomics. Into an odd row stride
    at a D off 16-byte alignment (zeroed by scalar stores) the result equals the compact one bit
    for bit, within the bound, and the neighbouring columns stay untouched."""
    m, n, k = 2304, 2560, 256
    log(f"gemm K-split tail, strided D {(m, n, k)}")
    qa, qb, ah, bh = _pair(m, n, k, 41)
    d = nv.gemm(qa, qb)
    out = torch.full((m, n + 3), -7.0, dtype=torch.float32, device="cuda")
    nv.gemm(qa, qb, out=out[:, 1:n + 1])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, 0] == -7.0) and np.all(o[:, n + 1:] == -7.0)
    ref = d.cpu().numpy()
    assert np.array_equal(o[:, 1:n + 1], ref)
    assert_gemm_within_bound(ref, ah, bh, "gemm K-split tail")


def test_column_quarters_equal_whole_tiles():
    """A GEMM whose tiles leave a last round of at most a quarter of the CUs computes it as 256 x
    64 column quarters; every output element still sums the same products in the same order as
    in a whole 256 x 256 tile. So a 600 x 700 GEMM (9 tiles, all in quarters) equals bit for bit
    the same rows and columns of a 4096 x 4096 GEMM of the same operands (256 whole tiles, one
    round on 256 CUs)."""
    log("column quarters = whole tiles")
    m = n = 4096
    k = 256
    rng = np.random.default_rng(77)
    qa, _ = nv.quantize(torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).cuda(), "1x16", "rn")
    qb, _ = nv.quantize(torch.from_numpy(rng.standard_normal((n, k)).astype(np.float32)).cuda(), "1x16", "sr",
                        seed=3)
    big = nv.gemm(qa, qb)
    sa = nv.NVFP4Tensor(qa.codes, qa.scales, qa.global_scale, 600, k)
    sb = nv.NVFP4Tensor(qb.codes, qb.scales, qb.global_scale, 700, k)
    small = nv.gemm(sa, sb)
    torch.cuda.synchronize()
    assert torch.equal(small, big[:600, :700])


def test_gemm_zero_and_one_hot():
    log("gemm special operands")
    k = 64
    x = np.zeros((16, k), np.float32)
    eye = np.eye(32, k, dtype=np.float32) * 3.0
    qa, _ = nv.quantize(torch.from_numpy(x).cuda(), "1x16", "rn")
    qb, _ = nv.quantize(torch.from_numpy(eye).cuda(), "1x16", "rn")
    d = nv.gemm(qa, qb)
    torch.cuda.synchronize()
    assert np.all(d.cpu().numpy() == 0.0)
    rng = np.random.default_rng(3)
    y = rng.standard_normal((40, k)).astype(np.float32)
    qy, _ = nv.quantize(torch.from_numpy(y).cuda(), "1x16", "rn")
    d = nv.gemm(qy, qb)
    torch.cuda.synchronize()
    yh = oracle.dequantize(*oracle.quantize_1x16(y))
    eh = oracle.dequantize(*oracle.quantize_1x16(eye))
    assert_gemm_within_bound(d.cpu().numpy(), yh, eh, "one hot")


def test_grouped_gemm_ragged_groups():
    log("grouped gemm")
    G, n, k = 6, 48, 96
    off = np.array([0, 0, 5, 140, 141, 141, 300], np.int64)      # empty, tiny and >128 groups
    x_bits = workloads.normal_bf16((int(off[-1]), k), 61)
    w_bits = workloads.normal_bf16((G * n, k), 62)
    offd = torch.from_numpy(off).cuda()
    wseg = np.arange(G + 1, dtype=np.int64) * n
    qx, _ = nv.quantize(to_device_bf16(x_bits), "1x16", "rn", segments=offd)
    qw, _ = nv.quantize(to_device_bf16(w_bits), "16x16", "rn", segments=torch.from_numpy(wseg).cuda())
    rx = oracle.quantize_1x16(f32(x_bits), segments=off)
    rw = oracle.quantize_16x16(f32(w_bits), segments=wseg)
    assert_quant_equal(host(qx), rx, "grouped X")
    assert_quant_equal(host(qw), rw, "grouped W")
    d = nv.grouped_gemm(offd, qx, qw, n)
    torch.cuda.synchronize()
    xh = oracle.dequantize(*rx, segments=off)
    wh = oracle.dequantize(*rw, segments=wseg)
    d64 = oracle.grouped_gemm_fp64(xh, wh, off, n)
    bound = oracle.grouped_gemm_bound(xh, wh, off, n)
    assert np.all(np.abs(d.cpu().numpy() - d64) <= bound)


@pytest.mark.parametrize("rows", [[3, 0, 200, 0], [700], [0, 0, 0, 1]])
def test_grouped_gemm_fewer_slots_than_xcds(rows):
    """The LDS-staged grouped kernel when the groups need fewer 256-row slots than the chip has
    XCDs (the slots are split over the XCDs by count, so some XCDs get none): every row
    within bound, the columns past N untouched."""
    log(f"grouped gemm few slots {rows}")
    n, k = 208, 128                      # N: the weights' 16x16 segments need multiples of 16
    G = len(rows)
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    x_bits = workloads.normal_bf16((int(off[-1]), k), 81 + G)
    w_bits = workloads.normal_bf16((G * n, k), 82 + G)
    offd = torch.from_numpy(off).cuda()
    wseg = np.arange(G + 1, dtype=np.int64) * n
    qx, _ = nv.quantize(to_device_bf16(x_bits), "1x16", "rn", segments=offd)
    qw, _ = nv.quantize(to_device_bf16(w_bits), "16x16", "rn", segments=torch.from_numpy(wseg).cuda())
    rx = oracle.quantize_1x16(f32(x_bits), segments=off)
    rw = oracle.quantize_16x16(f32(w_bits), segments=wseg)
    out = torch.full((int(off[-1]), n + 3), -5.0, dtype=torch.float32, device="cuda")
    nv.grouped_gemm(offd, qx, qw, n, out=out[:, :n])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, n:] == -5.0)
    xh = oracle.dequantize(*rx, segments=off)
    wh = oracle.dequantize(*rw, segments=wseg)
    d64 = oracle.grouped_gemm_fp64(xh, wh, off, n)
    bound = oracle.grouped_gemm_bound(xh, wh, off, n)
    assert np.all(np.abs(o[:, :n] - d64) <= bound)


@pytest.mark.parametrize("n,k", [(320, 192), (64, 128), (112, 2688), (576, 64), (352, 1856)])
def test_grouped_gemm_tile_shapes(n, k):
    """The LDS-staged grouped kernel (K % 64 == 0) with every tile shape it picks: full
    256 x 256 tiles, 128-row tiles for a group's last slot of at most 128 rows, and 64- or
    128-wide tiles for a last column of at most 64 or 128, over empty, tiny, exactly-128/256
    and multi-slot groups. Every row within bound, and each group's rows equal to the plain
    GEMM of that group's operands bit for bit."""
    log(f"grouped gemm tiles n={n} k={k}")
    rows = [0, 5, 130, 128, 300, 513, 256, 1, 0, 129]
    G = len(rows)
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    x_bits = workloads.normal_bf16((int(off[-1]), k), 71 + n)
    w_bits = workloads.with_outliers_bf16((G * n, k), 72 + k)
    offd = torch.from_numpy(off).cuda()
    wseg = np.arange(G + 1, dtype=np.int64) * n
    qx, _ = nv.quantize(to_device_bf16(x_bits), "1x16", "rn", segments=offd)
    qw, _ = nv.quantize(to_device_bf16(w_bits), "16x16", "rn", segments=torch.from_numpy(wseg).cuda())
    rx = oracle.quantize_1x16(f32(x_bits), segments=off)
    rw = oracle.quantize_16x16(f32(w_bits), segments=wseg)
    assert_quant_equal(host(qx), rx, "grouped X")
    assert_quant_equal(host(qw), rw, "grouped W")
    out = torch.full((int(off[-1]), n + 3), -5.0, dtype=torch.float32, device="cuda")
    d = nv.grouped_gemm(offd, qx, qw, n, out=out[:, :n])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, n:] == -5.0)
    xh = oracle.dequantize(*rx, segments=off)
    wh = oracle.dequantize(*rw, segments=wseg)
    d64 = oracle.grouped_gemm_fp64(xh, wh, off, n)
    bound = oracle.grouped_gemm_bound(xh, wh, off, n)
    assert np.all(np.abs(o[:, :n] - d64) <= bound)
    del d
    # each group's rows equal the plain GEMM of that group's operands bit for bit: the tile
    # shapes differ, the products and their order per element do not
    for g in range(G):
        r0, r1 = int(off[g]), int(off[g + 1])
        if r1 == r0:
            continue
        ag = nv.NVFP4Tensor(qx.codes[r0:r1], qx.scales[r0:r1], qx.global_scale[g:g + 1], r1 - r0, k)
        bg = nv.NVFP4Tensor(qw.codes[g * n:(g + 1) * n], qw.scales[g * n:(g + 1) * n],
                            qw.global_scale[g:g + 1], n, k)
        dg = nv.gemm(ag, bg)
        torch.cuda.synchronize()
        assert torch.equal(dg, out[r0:r1, :n]), f"group {g}"


def test_grouped_gemm_clustered_short_groups():
    """48 groups, the first 24 of 300-900 rows and the last 24 of 1-128 rows (so every short
    slot sits at the end of the slot numbering), N = 1856 (seven full column tiles and a 64-wide
    last one): the XCDs take equal runs of one slot order with the short slots spread through
    it and split runs inside slots. Every group's rows equal the plain GEMM of its operands bit
    for bit, all rows are within bound of the FP64 GEMM, and the columns past N stay untouched."""
    n, k = 1856, 128
    rng = np.random.default_rng(90)
    rows = list(rng.integers(300, 901, 24)) + list(rng.integers(1, 129, 24))
    G = len(rows)
    log(f"grouped gemm clustered short groups G={G} rows={sum(rows)}")
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    x_bits = workloads.normal_bf16((int(off[-1]), k), 91)
    w_bits = workloads.normal_bf16((G * n, k), 92)
    offd = torch.from_numpy(off).cuda()
    wseg = np.arange(G + 1, dtype=np.int64) * n
    qx, _ = nv.quantize(to_device_bf16(x_bits), "1x16", "rn", segments=offd)
    qw, _ = nv.quantize(to_device_bf16(w_bits), "16x16", "rn", segments=torch.from_numpy(wseg).cuda())
    out = torch.full((int(off[-1]), n + 2), -5.0, dtype=torch.float32, device="cuda")
    nv.grouped_gemm(offd, qx, qw, n, out=out[:, :n])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, n:] == -5.0)
    rx = oracle.quantize_1x16(f32(x_bits), segments=off)
    rw = oracle.quantize_16x16(f32(w_bits), segments=wseg)
    xh = oracle.dequantize(*rx, segments=off)
    wh = oracle.dequantize(*rw, segments=wseg)
    d64 = oracle.grouped_gemm_fp64(xh, wh, off, n)
    bound = oracle.grouped_gemm_bound(xh, wh, off, n)
    assert np.all(np.abs(o[:, :n] - d64) <= bound)
    for g in range(G):
        r0, r1 = int(off[g]), int(off[g + 1])
        ag = nv.NVFP4Tensor(qx.codes[r0:r1], qx.scales[r0:r1], qx.global_scale[g:g + 1], r1 - r0, k)
        bg = nv.NVFP4Tensor(qw.codes[g * n:(g + 1) * n], qw.scales[g * n:(g + 1) * n],
                            qw.global_scale[g:g + 1], n, k)
        dg = nv.gemm(ag, bg)
        torch.cuda.synchronize()
        assert torch.equal(dg, out[r0:r1, :n]), f"group {g}"


@pytest.mark.parametrize("m,n,offs", [
    (300, 520, [0, 64, 64, 448, 1024, 1920]),     # empty group, half steps at both ends
    (256, 256, [128, 192, 1856]),                 # groups not starting at 0 / ending before K
    (70, 33, [0, 1920]),                          # one group, ragged M and N
    (513, 300, [0, 640, 1280, 1344, 1920]),       # a 64-wide group inside one K step
    (448, 384, [0, 512, 1920]),                   # last row tile 192 high, last column 128 wide
    # 24 groups x 5 row tiles (the last 76 high): 120 tiles on 32 workgroups, each walking four
    # tiles whose shapes change along the walk (DMA of the next tile prefetched only between
    # tiles of one shape), with empty groups and 64-wide groups between them
    (1100, 200, [0, 64, 64, 192, 256, 448, 448, 512, 640, 704, 768, 1024, 1024, 1088, 1152, 1280,
                 1344, 1408, 1408, 1536, 1600, 1664, 1728, 1856, 1920]),
    # 5 x 3 = 15 tiles per group: one whole run of 8 tile ids, whose XCD regions rotate with the
    # group index, and a partial run of 7 that keeps its order; 11 groups cover every rotation
    (1100, 600, [0, 128, 256, 256, 640, 768, 1024, 1152, 1280, 1536, 1792, 1920]),
])
def test_grouped_gemm_k(m, n, offs):
    """GEMMs grouped along K (MoE weight gradient): each group's block against the FP64
    reference on the group's columns, per-group global scales, a padded output row stride."""
    log(f"grouped gemm K {m}x{n} {offs}")
    k = 1920
    G = len(offs) - 1
    rng = np.random.default_rng(m + n + G)
    a = (rng.standard_normal((m, k)) * 2).astype(np.float32)
    b = rng.standard_normal((n, k)).astype(np.float32)
    qa, _ = nv.quantize(to_device_f32(a), "1x16", "rn")
    qb, _ = nv.quantize(to_device_f32(b), "1x16", "sr", seed=5)
    ra = oracle.quantize_1x16(a)
    rb = oracle.quantize_1x16(b, "sr", seed=5)
    assert_quant_equal(host(qa), ra, "A")
    assert_quant_equal(host(qb), rb, "B")
    sa = np.array([2.0 ** (g % 3 - 1) for g in range(G)], np.float32) * ra[2][0]
    sb = np.array([3.0 if g % 2 else 0.75 for g in range(G)], np.float32) * rb[2][0]
    qa.global_scale = torch.from_numpy(sa).cuda()
    qb.global_scale = torch.from_numpy(sb).cuda()
    # dequantized operands with group g's columns scaled by its own global scale
    ah = oracle.dequantize(ra[0], ra[1], np.ones(1, np.float32))
    bh = oracle.dequantize(rb[0], rb[1], np.ones(1, np.float32))
    colscale_a = np.ones(k)
    colscale_b = np.ones(k)
    for g in range(G):
        colscale_a[offs[g]:offs[g + 1]] = sa[g]
        colscale_b[offs[g]:offs[g + 1]] = sb[g]
    ah = ah * colscale_a
    bh = bh * colscale_b
    out = torch.full((G * m, n + 5), -3.0, dtype=torch.float32, device="cuda")
    nv.grouped_gemm_k(torch.tensor(offs, dtype=torch.int64, device="cuda"), qa, qb, out=out[:, :n])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, n:] == -3.0)
    d64 = oracle.grouped_gemm_k_fp64(ah, bh, offs)
    bound = oracle.grouped_gemm_k_bound(ah, bh, offs)
    assert np.all(np.abs(o[:, :n] - d64) <= bound)
    for g in range(G):
        if offs[g + 1] == offs[g]:
            assert np.all(o[g * m:(g + 1) * m, :n] == 0.0)


def _colseg_dequant(q, segments):
    """Dequantized [rows, cols] of a tensor with one global scale per column segment."""
    codes, scales, gs = q
    y = oracle.dequantize(codes, scales, np.ones(1, np.float32))
    col = np.ones(y.shape[1])
    for g in range(len(segments) - 1):
        col[segments[g]:segments[g + 1]] = gs[g]
    return y * col


def test_moe_backward_chain():
    """The expert layer's backward pass end to end on a small layer (4 experts, one empty,
    hidden 256, expert FFN 192, tokens padded to 64 per expert): weights in 16x16 tiles with
    their per-expert transposes, dY in 1x16 SR per expert for the grouped activation-gradient
    GEMM; dY and X transformed and quantized per expert along tokens for the weight-gradient
    GEMM grouped along K. Every quantized operand is bit-exact against the oracle and both
    GEMMs are within the bound of the FP64 reference on those operands."""
    log("moe backward chain")
    G, hidden, ffn = 4, 256, 192
    off = np.array([0, 37, 37, 167, 231], np.int64)
    x_bits = workloads.normal_bf16((231, hidden), 501)
    w_bits = workloads.normal_bf16((G * ffn, hidden), 502)
    x_pad, dy_pad, off_pad = workloads.moe_backward(x_bits, off, ffn=ffn, pad=64)
    tp = int(off_pad[-1])
    offd = torch.from_numpy(off_pad).cuda()
    wseg = np.arange(G + 1, dtype=np.int64) * ffn
    mask = workloads.wgrad_sign_mask()
    wq, wqt = nv.quantize(to_device_bf16(w_bits), "16x16", "rn", emit_transposed=True,
                          segments=torch.from_numpy(wseg).cuda())
    dyq, _ = nv.quantize(to_device_bf16(dy_pad), "1x16", "sr", seed=21, segments=offd)
    dyt = nv.rht_quantize(to_device_bf16(dy_pad), mask, "sr", seed=22, offset=5, segments=offd)
    xt = nv.rht_quantize(to_device_bf16(x_pad), mask, "rn", segments=offd)
    dx = nv.grouped_gemm(offd, dyq, wqt, hidden)
    dw = nv.grouped_gemm_k(offd, dyt, xt)
    torch.cuda.synchronize()

    w, dy, x = f32(w_bits), f32(dy_pad), f32(x_pad)
    r_dyq = oracle.quantize_1x16(dy, "sr", seed=21, segments=off_pad)
    assert_quant_equal(host(dyq), r_dyq, "dY 1x16 SR per expert")
    wt = np.concatenate([w[g * ffn:(g + 1) * ffn].T for g in range(G)])
    wt_amax = oracle.amax(w, wseg)
    r_wt = [oracle.quantize_16x16(np.ascontiguousarray(w[g * ffn:(g + 1) * ffn].T), amax_vals=wt_amax[g:g + 1])
            for g in range(G)]
    r_wqt = (np.concatenate([r[0] for r in r_wt]), np.concatenate([r[1] for r in r_wt]),
             np.concatenate([r[2] for r in r_wt]))
    assert_quant_equal(host(wqt), r_wqt, "W^T per expert")
    r_dyt = oracle.rht_quantize_segments(dy, mask, off_pad, "sr", seed=22, offset=5)
    r_xt = oracle.rht_quantize_segments(x, mask, off_pad, "rn")
    assert_quant_equal(host(dyt), r_dyt, "H dY^T per expert")
    assert_quant_equal(host(xt), r_xt, "H X^T per expert")

    # dgrad: per expert g, dX_g = dY_g W_g (W_g^T stacked as B, N = hidden)
    a_hat = oracle.dequantize(*r_dyq, segments=off_pad)
    wt_seg = np.arange(G + 1, dtype=np.int64) * hidden
    b_hat = oracle.dequantize(*r_wqt, segments=wt_seg)
    d64 = oracle.grouped_gemm_fp64(a_hat, b_hat, off_pad, hidden)
    bound = oracle.grouped_gemm_bound(a_hat, b_hat, off_pad, hidden)
    assert np.all(np.abs(dx.cpu().numpy() - d64) <= bound)
    assert np.all(dx.cpu().numpy()[37:64] == 0.0)                        # padding rows
    # wgrad: per expert g, dW_g = (H dY_g)^T (H X_g) over the expert's tokens
    ah = _colseg_dequant(r_dyt, off_pad)
    bh = _colseg_dequant(r_xt, off_pad)
    d64 = oracle.grouped_gemm_k_fp64(ah, bh, off_pad)
    bound = oracle.grouped_gemm_k_bound(ah, bh, off_pad)
    got = dw.cpu().numpy()
    assert got.shape == (G * ffn, hidden)
    assert np.all(np.abs(got - d64) <= bound)
    assert np.all(got[ffn:2 * ffn] == 0.0)                               # the empty expert
    # the transform cancels: the product is the unrotated dY_g^T X_g up to the FP4 noise of
    # the two operands (about 0.17 relative here; a transform that did not cancel is near 1.4)
    ref = np.concatenate([dy[off_pad[g]:off_pad[g + 1]].T.astype(np.float64) @
                          x[off_pad[g]:off_pad[g + 1]].astype(np.float64) for g in range(G)])
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < 0.25, rel


@pytest.mark.parametrize("mnk", [(513, 1024, 5120), (1000, 700, 1344), (2304, 2560, 1024)])
def test_gemm_reproducible(mnk):
    """The same GEMM twice gives bitwise identical D, also where tiles of a partial last round
    are split along K and added into D with atomics."""
    m, n, k = mnk
    log(f"gemm reproducible {mnk}")
    rng = np.random.default_rng(m + n + k)
    qa, _ = nv.quantize(torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).cuda(), "1x16", "rn")
    qb, _ = nv.quantize(torch.from_numpy(rng.standard_normal((n, k)).astype(np.float32)).cuda(), "1x16", "rn")
    d1 = nv.gemm(qa, qb)
    d2 = nv.gemm(qa, qb)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2)


def test_output_row_pitch_past_the_buffer_range():
    """Outputs with a row pitch above 2^20 elements take the indexed store path instead of the
    tile-bounded buffer: plain FP32, BF16 with its amax, D += A B^T and the MXFP4 GEMM give the
    same bits as into a compact output, and the columns beside the view stay untouched."""
    log("gemm outputs with a row pitch past 2^20")
    m, n, k = 300, 520, 128                         # one K step: no tile is split along K
    pitch = (1 << 20) + 96
    qa, qb, _, _ = _pair(m, n, k, 31)
    sentinel = -7.0

    def wide(dtype, fill=sentinel):
        return torch.full((m, pitch), fill, dtype=dtype, device="cuda")

    def check(big, ref, what):
        torch.cuda.synchronize()
        h = big[:, :n + 96].cpu()
        assert torch.equal(h[:, :n], ref.cpu()), what
        assert torch.all(h[:, n:] == sentinel), what + " (beside the view)"

    ref = nv.gemm(qa, qb)
    big = wide(torch.float32)
    nv.gemm(qa, qb, out=big[:, :n])
    check(big, ref, "fp32")

    am_ref = torch.zeros((1,), device="cuda")
    ref16 = nv.gemm_ex(qa, qb, out_dtype=torch.bfloat16, amax_out=am_ref)
    big16 = wide(torch.bfloat16)
    am = torch.zeros((1,), device="cuda")
    nv.gemm_ex(qa, qb, out=big16[:, :n], out_dtype=torch.bfloat16, amax_out=am)
    check(big16, ref16, "bf16")
    assert torch.equal(am.cpu(), am_ref.cpu())

    d_old = torch.randn((m, n), device="cuda")
    acc_ref = d_old.clone()
    nv.gemm_ex(qa, qb, out=acc_ref, accumulate=True)
    bigacc = wide(torch.float32)
    bigacc[:, :n] = d_old
    nv.gemm_ex(qa, qb, out=bigacc[:, :n], accumulate=True)
    check(bigacc, acc_ref, "accumulate")

    xa = to_device_bf16(workloads.normal_bf16((m, k), 32))
    xb = to_device_bf16(workloads.normal_bf16((n, k), 33, std=0.02))
    ma, mb = nv.mx_quantize(xa), nv.mx_quantize(xb)
    mref = nv.mx_gemm(ma, mb)
    bigmx = wide(torch.float32)
    nv.mx_gemm(ma, mb, out=bigmx[:, :n])
    check(bigmx, mref, "mxfp4")
