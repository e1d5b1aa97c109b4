"""GPU parity at the full workload sizes, through the calls and launch configurations the bench
times: the dense layer (tokens 8192, in 5120, out 20480) and the expert layer (128 experts,
98304 routed rows, hidden 2688, expert FFN 1856). Quantized rows and columns are compared
bit for bit with the oracle on seeded samples (the oracle quantizes just those rows with the
full tensor's amax, which it computes itself), tensor maxima in full, and GEMM outputs on
sampled elements against the FP64 dot product of the oracle's own quantized rows."""
import numpy as np
import pytest
import torch

import bit_block_scaled_quantize_amd as nv
import oracle
import workloads
from helpers import assert_bytes_equal, f32, host, log, to_device_bf16

pytestmark = pytest.mark.gpu

M, K_IN, N_OUT = 8192, 5120, 20480
SAMPLE = 48


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def dense():
    x_bits, w_bits = workloads.fprop()
    dy_bits = workloads.dgrad()
    return f32(x_bits), f32(w_bits), f32(dy_bits), x_bits, w_bits, dy_bits


def _rows_equal(gpu, ref, rows, what):
    codes, scales, gs = gpu
    assert_bytes_equal(codes[rows], ref[0], what + " codes")
    assert_bytes_equal(scales[rows], ref[1], what + " scales")
    assert_bytes_equal(gs.view(np.uint32), np.asarray(ref[2], np.float32).view(np.uint32), what + " scale")


def _rht_amax(x, mask, chunk=1024):
    """max |H x| over the whole tensor, column chunk by column chunk (oracle transform)."""
    m = np.float32(0)
    for c in range(0, x.shape[1], chunk):
        m = max(m, np.abs(oracle.rht_columnwise(x[:, c:c + chunk], mask)).max())
    return np.float32(m)


def _check_samples(d, pick, a_rows, b_rows, what):
    """d: GPU output; pick: (m, n) pairs; a_rows(m) / b_rows(n): the oracle's dequantized row."""
    for m_, n_ in pick:
        a, b = a_rows(m_), b_rows(n_)
        ref = float(np.dot(a, b))
        bound = 1e-5 * float(np.dot(np.abs(a), np.abs(b)))
        got = float(d[m_, n_])
        assert abs(got - ref) <= bound, f"{what} [{m_}, {n_}]: gpu {got!r} ref {ref!r} bound {bound!r}"


def test_dense_layer_full_size(dense):
    x, w, dy, x_bits, w_bits, dy_bits = dense
    mask = workloads.wgrad_sign_mask()
    rng = np.random.default_rng(2024)
    log("dense layer full size: quantize")
    X, W, dY = to_device_bf16(x_bits), to_device_bf16(w_bits), to_device_bf16(dy_bits)
    ax, ady = nv.amax_pair(X, mask), nv.amax_pair(dY, mask)
    qx, _ = nv.quantize(X, "1x16", "rn", amax=ax[0:1])
    qw, qwt = nv.quantize(W, "16x16", "rn", emit_transposed=True)
    qdy, _ = nv.quantize(dY, "1x16", "sr", seed=workloads.SR_SEED_DGRAD, offset=0, amax=ady[0:1])
    qhdy = nv.rht_quantize(dY, mask, "sr", seed=workloads.SR_SEED_WGRAD, offset=workloads.SR_OFFSET_WGRAD,
                           amax=ady[1:2])
    qhx = nv.rht_quantize(X, mask, "rn", amax=ax[1:2])
    torch.cuda.synchronize()
    # tensor maxima, in full
    a_x, a_w, a_dy = oracle.amax(x), oracle.amax(w), oracle.amax(dy)
    h_x, h_dy = _rht_amax(x, mask), _rht_amax(dy, mask)
    assert_bytes_equal(ax.cpu().numpy().view(np.uint32), np.array([a_x[0], h_x], np.float32).view(np.uint32), "pair X")
    assert_bytes_equal(ady.cpu().numpy().view(np.uint32), np.array([a_dy[0], h_dy], np.float32).view(np.uint32), "pair dY")
    # sampled rows / columns, bit for bit
    rx = np.sort(rng.choice(M, SAMPLE, replace=False))
    g16 = np.sort(rng.choice(N_OUT // 16, 8, replace=False))
    rw = (g16[:, None] * 16 + np.arange(16)).reshape(-1)
    gt16 = np.sort(rng.choice(K_IN // 16, 8, replace=False))
    cw = (gt16[:, None] * 16 + np.arange(16)).reshape(-1)                    # rows of W^T
    cdy = np.sort(rng.choice(N_OUT, SAMPLE, replace=False))                  # rows of (H dY)^T
    cx = np.sort(rng.choice(K_IN, SAMPLE, replace=False))                    # rows of (H X)^T
    ref_x = oracle.quantize_1x16(x[rx], amax_vals=a_x, row_ids=rx)
    ref_w = oracle.quantize_16x16(w[rw], amax_vals=a_w, row_ids=rw)
    ref_wt = oracle.quantize_16x16(np.ascontiguousarray(w[:, cw].T), amax_vals=a_w, row_ids=cw)
    ref_dy = oracle.quantize_1x16(dy[rx], "sr", seed=workloads.SR_SEED_DGRAD, offset=0, amax_vals=a_dy, row_ids=rx)
    ref_hdy = oracle.rht_quantize(dy[:, cdy], mask, "sr", seed=workloads.SR_SEED_WGRAD,
                                  offset=workloads.SR_OFFSET_WGRAD, amax_vals=np.float32(h_dy), col_ids=cdy)
    ref_hx = oracle.rht_quantize(x[:, cx], mask, "rn", amax_vals=np.float32(h_x), col_ids=cx)
    gx, gw, gwt, gdy, ghdy, ghx = host(qx), host(qw), host(qwt), host(qdy), host(qhdy), host(qhx)
    _rows_equal(gx, ref_x, rx, "X")
    _rows_equal(gw, ref_w, rw, "W")
    _rows_equal(gwt, ref_wt, cw, "W^T")
    _rows_equal(gdy, ref_dy, rx, "dY")
    _rows_equal(ghdy, ref_hdy, cdy, "(H dY)^T")
    _rows_equal(ghx, ref_hx, cx, "(H X)^T")

    log("dense layer full size: GEMMs")
    y = nv.gemm(qx, qw)
    dx = nv.gemm(qdy, qwt)
    dw = nv.gemm(qhdy, qhx)
    torch.cuda.synchronize()
    # the oracle dequantizes its own quantization of each sampled output's operand rows
    sx_d = dict(zip(rx, oracle.dequantize(*ref_x)))
    sw_d = dict(zip(rw, oracle.dequantize(*ref_w)))
    sdy_d = dict(zip(rx, oracle.dequantize(*ref_dy)))
    swt_d = dict(zip(cw, oracle.dequantize(*ref_wt)))
    shdy_d = dict(zip(cdy, oracle.dequantize(*ref_hdy)))
    shx_d = dict(zip(cx, oracle.dequantize(*ref_hx)))
    pick = lambda rows, cols: [(int(a), int(b)) for a, b in zip(rng.choice(rows, 64), rng.choice(cols, 64))]
    _check_samples(y.cpu().numpy(), pick(rx, rw), sx_d.__getitem__, sw_d.__getitem__, "fprop")
    _check_samples(dx.cpu().numpy(), pick(rx, cw), sdy_d.__getitem__, swt_d.__getitem__, "dgrad")
    _check_samples(dw.cpu().numpy(), pick(cdy, cx), shdy_d.__getitem__, shx_d.__getitem__, "wgrad")


def test_moe_layer_full_size():
    log("moe full size")
    x_bits, w_bits, off = workloads.moe()
    G, n, k = workloads.MOE_EXPERTS, workloads.MOE_FFN, workloads.MOE_HIDDEN
    x, w = f32(x_bits), f32(w_bits)
    rng = np.random.default_rng(77)
    offd = torch.from_numpy(off).cuda()
    wseg = np.arange(G + 1, dtype=np.int64) * n
    qx, _ = nv.quantize(to_device_bf16(x_bits), "1x16", "rn", segments=offd)
    qw, _ = nv.quantize(to_device_bf16(w_bits), "16x16", "rn", segments=torch.from_numpy(wseg).cuda())
    d = nv.grouped_gemm(offd, qx, qw, n)
    torch.cuda.synchronize()
    a_x, a_w = oracle.amax(x, off), oracle.amax(w, wseg)
    gx, gw = host(qx), host(qw)
    assert_bytes_equal(gx[2].view(np.uint32), oracle.global_scales(a_x)[1].astype(np.float32).view(np.uint32),
                       "X scale per expert")
    # sampled rows: the first and last row of a few experts (the largest and smallest among them)
    sizes = np.diff(off)
    experts = np.unique(np.concatenate([[np.argmax(sizes), np.argmin(sizes)], rng.choice(G, 6, replace=False)]))
    rx = np.unique(np.concatenate([[off[g], off[g + 1] - 1, rng.integers(off[g], off[g + 1])] for g in experts]))
    ref_x = oracle.quantize_1x16(x[rx], segments=off, amax_vals=a_x, row_ids=rx)
    _rows_equal(gx, ref_x, rx, "expert X")
    g16 = np.unique(np.concatenate([[g * n // 16, (g + 1) * n // 16 - 1] for g in experts]))
    rw = (g16[:, None] * 16 + np.arange(16)).reshape(-1)
    ref_w = oracle.quantize_16x16(w[rw], segments=wseg, amax_vals=a_w, row_ids=rw)
    _rows_equal(gw, ref_w, rw, "expert W")
    sx_d = dict(zip(rx, oracle.dequantize(*ref_x, segments=off, row_ids=rx)))
    sw_d = dict(zip(rw, oracle.dequantize(*ref_w, segments=wseg, row_ids=rw)))
    dh = d.cpu().numpy()
    checked = 0
    for r in rx:
        g = int(np.searchsorted(off, r, side="right") - 1)
        cols = [c - g * n for c in rw if g * n <= c < (g + 1) * n]
        for c in cols[:: max(1, len(cols) // 8)]:
            a, b = sx_d[r], sw_d[g * n + c]
            ref = float(np.dot(a, b))
            bound = 1e-5 * float(np.dot(np.abs(a), np.abs(b)))
            assert abs(float(dh[r, c]) - ref) <= bound, (r, c)
            checked += 1
    assert checked >= 16


def test_two_to_the_31_elements():
    """A 65536 x 32768 BF16 tensor (2^31 elements, 4 GiB): every index past 32 bits. Uniform
    values in [-1, 1] with one spike of 1000, so both tensor maxima come from the spike's block
    (every other transformed block is at most 16 * 1/4 = 4): the oracle computes them from
    that block, checks them in full, and checks sampled rows (1x16) and columns (transform)
    bit for bit, including the spike's."""
    rows, cols = 65536, 32768
    log("2^31 elements")
    g = torch.Generator(device="cuda").manual_seed(31)
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, rows, 4096):
        x[r0:r0 + 4096] = (torch.rand((4096, cols), generator=g, device="cuda") * 2 - 1).to(torch.bfloat16)
    rs, cs = 54321, 23456
    x[rs, cs] = 1000.0
    mask = workloads.wgrad_sign_mask()
    a = nv.amax(x)
    ah = nv.amax(x, rht=True, sign_mask=mask)
    q, _ = nv.quantize(x, "1x16", "rn")
    qh = nv.rht_quantize(x, mask, "rn")
    torch.cuda.synchronize()
    assert a.item() == 1000.0
    tb = rs // 16 * 16
    blk = x[tb:tb + 16, cs:cs + 1].float().cpu().numpy()
    want_h = np.float32(np.abs(oracle.rht_columnwise(blk, mask)).max())
    assert want_h > 4.0
    assert_bytes_equal(ah.cpu().numpy().view(np.uint32), np.array([want_h], np.float32).view(np.uint32), "rht amax")
    rng = np.random.default_rng(31)
    sr = np.unique(np.concatenate([[0, rows - 1, rs], rng.integers(0, rows, 5)]))
    sc = np.unique(np.concatenate([[0, cols - 1, cs], rng.integers(0, cols, 5)]))
    xr = x[torch.from_numpy(sr).cuda()].float().cpu().numpy()
    xc = x[:, torch.from_numpy(sc).cuda()].float().cpu().numpy()
    ref = oracle.quantize_1x16(xr, amax_vals=np.array([1000.0], np.float32), row_ids=sr)
    gq = (q.codes[torch.from_numpy(sr).cuda()].cpu().numpy(), q.scales[torch.from_numpy(sr).cuda()].cpu().numpy(),
          q.global_scale.cpu().numpy())
    assert_bytes_equal(gq[0], ref[0], "rows codes")
    assert_bytes_equal(gq[1], ref[1], "rows scales")
    refh = oracle.rht_quantize(xc, mask, "rn", amax_vals=np.array([want_h], np.float32), col_ids=sc)
    ic = torch.from_numpy(sc).cuda()
    assert_bytes_equal(qh.codes[ic].cpu().numpy(), refh[0], "columns codes")
    assert_bytes_equal(qh.scales[ic].cpu().numpy(), refh[1], "columns scales")
    assert_bytes_equal(qh.global_scale.cpu().numpy().view(np.uint32), np.asarray(refh[2], np.float32).view(np.uint32),
                       "columns scale")


def test_moe_dgrad_full_size():
    """The expert layer's activation gradient at full size on the padded token layout (128
    experts, tokens padded to 64 per expert, N = hidden 2688, K = FFN 1856): dY in 1x16 SR per
    expert, the weights' per-expert transposes from the 16x16 call, then the grouped GEMM (its
    last column tiles are 128 wide). Sampled rows of both operands bit-exact against the
    oracle, sampled outputs within the bound of the FP64 reference."""
    log("moe dgrad full size")
    x_bits, w_bits, off = workloads.moe()
    G, n, k = workloads.MOE_EXPERTS, workloads.MOE_FFN, workloads.MOE_HIDDEN
    _, dy_pad, off_pad = workloads.moe_backward(x_bits, off)
    del x_bits
    rng = np.random.default_rng(78)
    offp = torch.from_numpy(off_pad).cuda()
    wseg = np.arange(G + 1, dtype=np.int64) * n
    qdy, _ = nv.quantize(to_device_bf16(dy_pad), "1x16", "sr", seed=21, segments=offp)
    _, qwt = nv.quantize(to_device_bf16(w_bits), "16x16", "rn", emit_transposed=True,
                         segments=torch.from_numpy(wseg).cuda())
    dx = nv.grouped_gemm(offp, qdy, qwt, k)
    torch.cuda.synchronize()
    dy, w = f32(dy_pad), f32(w_bits)
    a_dy, a_w = oracle.amax(dy, off_pad), oracle.amax(w, wseg)
    sizes = np.diff(off_pad)
    experts = np.unique(np.concatenate([[np.argmax(sizes), np.argmin(sizes)], rng.choice(G, 5, replace=False)]))
    rows = np.unique(np.concatenate([[off_pad[g], off_pad[g + 1] - 1, rng.integers(off_pad[g], off_pad[g + 1])]
                                     for g in experts]))
    ref_dy = oracle.quantize_1x16(dy[rows], "sr", seed=21, segments=off_pad, amax_vals=a_dy, row_ids=rows)
    _rows_equal(host(qdy), ref_dy, rows, "expert dY")
    sdy = dict(zip(rows, oracle.dequantize(*ref_dy, segments=off_pad, row_ids=rows)))
    # columns of dX: 16-aligned groups at the start, the 128-wide last tile and one inside
    c16 = np.array([0, k // 16 - 1, (k - 128) // 16, rng.integers(0, k // 16)])
    gwt = host(qwt)
    checked = 0
    for g in experts:
        wt = w[g * n:(g + 1) * n].T                                # [hidden, ffn] of expert g
        for cg in c16:
            cols = cg * 16 + np.arange(16)
            ref_wt = oracle.quantize_16x16(wt[cols], amax_vals=np.array([a_w[g]], np.float32))
            trows = g * k + cols
            assert_bytes_equal(gwt[0][trows], ref_wt[0], f"expert {g} W^T codes")
            assert_bytes_equal(gwt[1][trows], ref_wt[1], f"expert {g} W^T scales")
            wdq = oracle.dequantize(*ref_wt)
            for r in rows[(rows >= off_pad[g]) & (rows < off_pad[g + 1])]:
                for i in (0, 7, 15):
                    a, b = sdy[r], wdq[i]
                    ref = float(np.dot(a, b))
                    bound = 1e-5 * float(np.dot(np.abs(a), np.abs(b)))
                    assert abs(float(dx[r, cols[i]].item()) - ref) <= bound, (g, r, cols[i])
                    checked += 1
    assert checked >= 48


def test_moe_wgrad_full_size():
    """The expert layer's weight gradient at full size (the GEMM grouped along K): dY and X on
    the padded token layout, transformed along tokens and quantized per expert (nearest; both
    sides take the same per-expert maxima, 4 max|x| per expert, which bounds |H x|), then
    nvfp4_grouped_gemm_k into dW [128 * 1856, 2688] (its last row tiles are 64 high and its
    last column tiles 128 wide). Sampled rows of both transposed operands bit-exact against
    the oracle, sampled dW entries within the bound of the FP64 sum over the expert's
    tokens."""
    log("moe wgrad full size")
    x_bits, _, off = workloads.moe()
    G, n, k = workloads.MOE_EXPERTS, workloads.MOE_FFN, workloads.MOE_HIDDEN
    x_pad, dy_pad, off_pad = workloads.moe_backward(x_bits, off)
    del x_bits
    mask = workloads.wgrad_sign_mask()
    rng = np.random.default_rng(79)
    offp = torch.from_numpy(off_pad).cuda()
    dy, x = f32(dy_pad), f32(x_pad)
    a_dy = (oracle.amax(dy, off_pad) * np.float32(4)).astype(np.float32)
    a_x = (oracle.amax(x, off_pad) * np.float32(4)).astype(np.float32)
    qdy = nv.rht_quantize(to_device_bf16(dy_pad), mask, "rn", segments=offp, amax=torch.from_numpy(a_dy).cuda())
    qx = nv.rht_quantize(to_device_bf16(x_pad), mask, "rn", segments=offp, amax=torch.from_numpy(a_x).cuda())
    dw = nv.grouped_gemm_k(offp, qdy, qx)
    torch.cuda.synchronize()
    i_rows = np.unique(np.concatenate([[0, n - 1, n - 64, n - 65], rng.integers(0, n, 3)]))      # FFN rows
    c_cols = np.unique(np.concatenate([[0, k - 1, k - 128, k - 129], rng.integers(0, k, 3)]))    # hidden
    ref_dy = oracle.quantize_1x16_colsegments(oracle.rht_columnwise(dy[:, i_rows], mask), off_pad, amax_vals=a_dy)
    ref_x = oracle.quantize_1x16_colsegments(oracle.rht_columnwise(x[:, c_cols], mask), off_pad, amax_vals=a_x)
    gdy, gx = host(qdy), host(qx)
    assert_bytes_equal(gdy[0][i_rows], ref_dy[0], "H dY codes")
    assert_bytes_equal(gdy[1][i_rows], ref_dy[1], "H dY scales")
    assert_bytes_equal(gx[0][c_cols], ref_x[0], "H X codes")
    assert_bytes_equal(gx[1][c_cols], ref_x[1], "H X scales")
    dqa = oracle.dequantize(ref_dy[0], ref_dy[1], np.ones(1, np.float32))
    dqb = oracle.dequantize(ref_x[0], ref_x[1], np.ones(1, np.float32))
    sizes = np.diff(off_pad)
    experts = np.unique(np.concatenate([[np.argmax(sizes), np.argmin(sizes)], rng.choice(G, 4, replace=False)]))
    dwh = {}
    checked = 0
    for g in experts:
        t0, t1 = int(off_pad[g]), int(off_pad[g + 1])
        sg = float(ref_dy[2][g]) * float(ref_x[2][g])
        block = dw[g * n:(g + 1) * n].cpu().numpy()
        for a_i, i in enumerate(i_rows):
            for b_i, c in enumerate(c_cols):
                a, b = dqa[a_i, t0:t1], dqb[b_i, t0:t1]
                ref = float(np.dot(a, b)) * sg
                bound = 1e-5 * float(np.dot(np.abs(a), np.abs(b))) * sg
                assert abs(float(block[i, c]) - ref) <= bound, (g, i, c)
                checked += 1
    assert checked >= 100
