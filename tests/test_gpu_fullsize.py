"""GPU parity at the full workload sizes, through the calls and launch configurations the bench
times: the dense layer (tokens 8192, in 5120, out 20480: fprop, dgrad with stochastic rounding,
wgrad with the Hadamard transform) and the expert layer (128 experts, 98304 routed rows, hidden
2688, expert FFN 1856: forward, and the backward on the padded token layout). Every byte of
every quantized operand (codes, block scales, tensor scales) is compared with the oracle, and
every element of every GEMM output with the bound 1e-5 * sum |a||b| around the FP64 product of
the oracle's dequantized operands (BLAS dgemm, row chunks). The oracle runs on row or column
chunks in a thread pool (numpy releases the interpreter lock inside its array operations), sized
to the host's CPU share."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import bit_block_scaled_quantize_amd as nv
import oracle
import workloads
from helpers import assert_bytes_equal, f32, host, log, to_device_bf16

pytestmark = pytest.mark.gpu

M, K_IN, N_OUT = 8192, 5120, 20480
WORKERS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _ranges(n, parts, align=16):
    step = max(align, (n + parts - 1) // parts // align * align)
    return [(a, min(n, a + step)) for a in range(0, n, step)]


def _pmap(fn, items):
    with ThreadPoolExecutor(WORKERS) as ex:
        return list(ex.map(fn, items))


def _cat(parts, i):
    return np.concatenate([p[i] for p in parts], axis=0)


def _q1x16(x, rounding="rn", seed=0, offset=0, segments=None, amax_vals=None):
    """oracle.quantize_1x16 of the whole tensor, row chunks in parallel (the block index of SR
    and the segment of a row come from row_ids, so chunks give the full tensor's bytes)."""
    a = oracle.amax(x, segments) if amax_vals is None else amax_vals
    parts = _pmap(lambda r: oracle.quantize_1x16(x[r[0]:r[1]], rounding, seed, offset, segments, a,
                                                 np.arange(r[0], r[1])), _ranges(len(x), 4 * WORKERS))
    return _cat(parts, 0), _cat(parts, 1), oracle.global_scales(a)[1]


def _q16x16(x, segments=None, amax_vals=None):
    a = oracle.amax(x, segments) if amax_vals is None else amax_vals
    parts = _pmap(lambda r: oracle.quantize_16x16(x[r[0]:r[1]], segments, a, np.arange(r[0], r[1])),
                  _ranges(len(x), 4 * WORKERS))
    return _cat(parts, 0), _cat(parts, 1), oracle.global_scales(a)[1]


def _rht(x, mask):
    """The transformed tensor y [cols, tokens] (oracle), column chunks in parallel."""
    parts = _pmap(lambda r: oracle.rht_columnwise(x[:, r[0]:r[1]], mask), _ranges(x.shape[1], 4 * WORKERS, 1))
    return np.concatenate(parts, axis=0)


def _deq(q, segments=None):
    """oracle.dequantize in row chunks (float64)."""
    codes, scales, s_dec = q
    parts = _pmap(lambda r: oracle.dequantize(codes[r[0]:r[1]], scales[r[0]:r[1]], s_dec, segments,
                                              np.arange(r[0], r[1])), _ranges(len(codes), 4 * WORKERS))
    return np.concatenate(parts, axis=0)


def _same(gpu, ref, what):
    codes, scales, gs = gpu
    assert_bytes_equal(codes, ref[0], what + " codes")
    assert_bytes_equal(scales, ref[1], what + " scales")
    assert_bytes_equal(gs.view(np.uint32), np.asarray(ref[2], np.float32).view(np.uint32), what + " tensor scales")


def _gemm_in_bound(d_gpu, a_hat, b_hat, what, chunk=1024):
    """Every element of d_gpu [M, N] (a GPU tensor) against a_hat @ b_hat^T in FP64 within
    1e-5 * |a_hat| @ |b_hat|^T."""
    b_abs = np.abs(b_hat)
    worst = 0.0
    for r0 in range(0, a_hat.shape[0], chunk):
        r1 = min(a_hat.shape[0], r0 + chunk)
        a = a_hat[r0:r1]
        ref = a @ b_hat.T
        bound = 1e-5 * (np.abs(a) @ b_abs.T)
        got = d_gpu[r0:r1].float().cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        bad = err > bound
        if bad.any():
            i, j = np.argwhere(bad)[0]
            raise AssertionError(f"{what}: {int(bad.sum())} elements out of bound; first [{r0 + i}, {j}]: "
                                 f"gpu {got[i, j]!r} ref {ref[i, j]!r} bound {bound[i, j]!r}")
        worst = max(worst, float((err / np.maximum(bound, 1e-300)).max()))
    log(f"{what}: every element within bound (largest error {worst:.3g} of the bound)")


@pytest.fixture(scope="module")
def dense():
    x_bits, w_bits = workloads.fprop()
    dy_bits = workloads.dgrad()
    return f32(x_bits), f32(w_bits), f32(dy_bits), x_bits, w_bits, dy_bits


def test_dense_layer_full_size(dense):
    x, w, dy, x_bits, w_bits, dy_bits = dense
    mask = workloads.wgrad_sign_mask()
    log("dense layer full size: GPU quantize")
    X, W, dY = to_device_bf16(x_bits), to_device_bf16(w_bits), to_device_bf16(dy_bits)
    ax, ady = nv.amax_pair(X, mask), nv.amax_pair(dY, mask)
    qx, _ = nv.quantize(X, "1x16", "rn", amax=ax[0:1])
    qw, qwt = nv.quantize(W, "16x16", "rn", emit_transposed=True)
    qdy, _ = nv.quantize(dY, "1x16", "sr", seed=workloads.SR_SEED_DGRAD, offset=0, amax=ady[0:1])
    qhdy = nv.rht_quantize(dY, mask, "sr", seed=workloads.SR_SEED_WGRAD, offset=workloads.SR_OFFSET_WGRAD,
                           amax=ady[1:2])
    qhx = nv.rht_quantize(X, mask, "rn", amax=ax[1:2])
    torch.cuda.synchronize()
    del X, W, dY

    log("dense layer full size: oracle X, W, W^T, dY")
    a_x, a_w, a_dy = oracle.amax(x), oracle.amax(w), oracle.amax(dy)
    ref_x = _q1x16(x, amax_vals=a_x)
    _same(host(qx), ref_x, "X 1x16")
    ref_w = _q16x16(w, amax_vals=a_w)
    _same(host(qw), ref_w, "W 16x16")
    ref_wt = _q16x16(np.ascontiguousarray(w.T), amax_vals=a_w)
    _same(host(qwt), ref_wt, "W^T 16x16")
    ref_dy = _q1x16(dy, "sr", seed=workloads.SR_SEED_DGRAD, offset=0, amax_vals=a_dy)
    _same(host(qdy), ref_dy, "dY 1x16 SR")
    log("dense layer full size: oracle Hadamard operands")
    y_dy = _rht(dy, mask)
    h_dy = oracle.amax(y_dy)
    ref_hdy = _q1x16(y_dy, "sr", seed=workloads.SR_SEED_WGRAD, offset=workloads.SR_OFFSET_WGRAD, amax_vals=h_dy)
    del y_dy
    _same(host(qhdy), ref_hdy, "(H dY)^T SR")
    y_x = _rht(x, mask)
    h_x = oracle.amax(y_x)
    ref_hx = _q1x16(y_x, amax_vals=h_x)
    del y_x
    _same(host(qhx), ref_hx, "(H X)^T RN")
    want_ax = np.array([a_x[0], h_x[0]], np.float32)
    want_ady = np.array([a_dy[0], h_dy[0]], np.float32)
    assert_bytes_equal(ax.cpu().numpy().view(np.uint32), want_ax.view(np.uint32), "amax pair X")
    assert_bytes_equal(ady.cpu().numpy().view(np.uint32), want_ady.view(np.uint32), "amax pair dY")

    log("dense layer full size: GEMMs")
    y_d = nv.gemm(qx, qw)
    x_hat, w_hat = _deq(ref_x), _deq(ref_w)
    _gemm_in_bound(y_d, x_hat, w_hat, "fprop 8192x20480x5120")
    del y_d, x_hat, w_hat
    dx_d = nv.gemm(qdy, qwt)
    dy_hat, wt_hat = _deq(ref_dy), _deq(ref_wt)
    _gemm_in_bound(dx_d, dy_hat, wt_hat, "dgrad 8192x5120x20480")
    del dx_d, dy_hat, wt_hat
    dw_d = nv.gemm(qhdy, qhx)
    hdy_hat, hx_hat = _deq(ref_hdy), _deq(ref_hx)
    _gemm_in_bound(dw_d, hdy_hat, hx_hat, "wgrad 20480x5120x8192")


def _grouped_in_bound(d_gpu, a_hat, b_hat, off, n, what):
    """Grouped GEMM: rows off[g]..off[g+1] of d against a_hat rows and b_hat rows g*n..(g+1)*n."""
    rows = 0
    for g in range(len(off) - 1):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi == lo:
            continue
        _gemm_in_bound_quiet(d_gpu[lo:hi], a_hat[lo:hi], b_hat[g * n:(g + 1) * n], f"{what} group {g}")
        rows += hi - lo
    log(f"{what}: every element of {rows} rows within bound")


def _gemm_in_bound_quiet(d_gpu, a_hat, b_hat, what, chunk=2048):
    b_abs = np.abs(b_hat)
    for r0 in range(0, a_hat.shape[0], chunk):
        a = a_hat[r0:r0 + chunk]
        ref = a @ b_hat.T
        bound = 1e-5 * (np.abs(a) @ b_abs.T)
        got = d_gpu[r0:r0 + chunk].float().cpu().numpy().astype(np.float64)
        bad = np.abs(got - ref) > bound
        if bad.any():
            i, j = np.argwhere(bad)[0]
            raise AssertionError(f"{what}: {int(bad.sum())} out of bound; first [{r0 + i}, {j}]: "
                                 f"gpu {got[i, j]!r} ref {ref[i, j]!r} bound {bound[i, j]!r}")


def test_moe_layer_full_size():
    log("moe full size: GPU")
    x_bits, w_bits, off = workloads.moe()
    G, n, k = workloads.MOE_EXPERTS, workloads.MOE_FFN, workloads.MOE_HIDDEN
    offd = torch.from_numpy(off).cuda()
    wseg = np.arange(G + 1, dtype=np.int64) * n
    qx, _ = nv.quantize(to_device_bf16(x_bits), "1x16", "rn", segments=offd)
    qw, qwt = nv.quantize(to_device_bf16(w_bits), "16x16", "rn", emit_transposed=True,
                          segments=torch.from_numpy(wseg).cuda())
    d = nv.grouped_gemm(offd, qx, qw, n)
    torch.cuda.synchronize()
    log("moe full size: oracle X, W, W^T per expert")
    x, w = f32(x_bits), f32(w_bits)
    del x_bits, w_bits
    a_x, a_w = oracle.amax(x, off), oracle.amax(w, wseg)
    ref_x = _q1x16(x, segments=off, amax_vals=a_x)
    _same(host(qx), ref_x, "expert X 1x16")
    ref_w = _q16x16(w, segments=wseg, amax_vals=a_w)
    _same(host(qw), ref_w, "expert W 16x16")
    gwt = host(qwt)
    parts = _pmap(lambda g: oracle.quantize_16x16(np.ascontiguousarray(w[g * n:(g + 1) * n].T),
                                                  amax_vals=a_w[g:g + 1]), range(G))
    _same(gwt, (_cat(parts, 0), _cat(parts, 1), oracle.global_scales(a_w)[1]), "expert W^T 16x16")
    del parts
    log("moe full size: grouped GEMM")
    x_hat = _deq(ref_x, off)
    w_hat = _deq(ref_w, wseg)
    _grouped_in_bound(d, x_hat, w_hat, off, n, "grouped fprop")


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
    expert and the weights' per-expert transposes from the 16x16 call, every byte against the
    oracle; every output of the grouped GEMM (its last column tiles are 128 wide) within the
    bound of the FP64 product."""
    log("moe dgrad full size: GPU")
    x_bits, w_bits, off = workloads.moe()
    G, n, k = workloads.MOE_EXPERTS, workloads.MOE_FFN, workloads.MOE_HIDDEN
    _, dy_pad, off_pad = workloads.moe_backward(x_bits, off)
    del x_bits
    offp = torch.from_numpy(off_pad).cuda()
    wseg = np.arange(G + 1, dtype=np.int64) * n
    qdy, _ = nv.quantize(to_device_bf16(dy_pad), "1x16", "sr", seed=21, segments=offp)
    _, qwt = nv.quantize(to_device_bf16(w_bits), "16x16", "rn", emit_transposed=True,
                         segments=torch.from_numpy(wseg).cuda())
    dx = nv.grouped_gemm(offp, qdy, qwt, k)
    torch.cuda.synchronize()
    log("moe dgrad full size: oracle dY, W^T per expert")
    dy, w = f32(dy_pad), f32(w_bits)
    del dy_pad, w_bits
    a_dy, a_w = oracle.amax(dy, off_pad), oracle.amax(w, wseg)
    ref_dy = _q1x16(dy, "sr", seed=21, segments=off_pad, amax_vals=a_dy)
    _same(host(qdy), ref_dy, "expert dY 1x16 SR")
    parts = _pmap(lambda g: oracle.quantize_16x16(np.ascontiguousarray(w[g * n:(g + 1) * n].T),
                                                  amax_vals=a_w[g:g + 1]), range(G))
    ref_wt = (_cat(parts, 0), _cat(parts, 1), oracle.global_scales(a_w)[1])
    del parts, w
    _same(host(qwt), ref_wt, "expert W^T 16x16")
    log("moe dgrad full size: grouped GEMM")
    tseg = np.arange(G + 1, dtype=np.int64) * k                     # W^T rows of expert g
    _grouped_in_bound(dx, _deq(ref_dy, off_pad), _deq(ref_wt, tseg), off_pad, k, "grouped dgrad")


def test_moe_wgrad_full_size():
    """The expert layer's weight gradient at full size (the GEMM grouped along K): dY and X on
    the padded token layout, transformed along tokens and quantized per expert (dY stochastic,
    X nearest; both sides take the same per-expert maxima, 4 max|x| per expert, which bounds
    |H x|), every byte against the oracle; then nvfp4_grouped_gemm_k into dW [128 * 1856, 2688]
    (its last row tiles are 64 high and its last column tiles 128 wide), every entry within the
    bound of the FP64 sum over the expert's tokens."""
    log("moe wgrad full size: GPU")
    x_bits, _, off = workloads.moe()
    G, n, k = workloads.MOE_EXPERTS, workloads.MOE_FFN, workloads.MOE_HIDDEN
    x_pad, dy_pad, off_pad = workloads.moe_backward(x_bits, off)
    del x_bits
    mask = workloads.wgrad_sign_mask()
    offp = torch.from_numpy(off_pad).cuda()
    dy, x = f32(dy_pad), f32(x_pad)
    a_dy = (oracle.amax(dy, off_pad) * np.float32(4)).astype(np.float32)
    a_x = (oracle.amax(x, off_pad) * np.float32(4)).astype(np.float32)
    qdy = nv.rht_quantize(to_device_bf16(dy_pad), mask, "sr", seed=23, offset=5, segments=offp,
                          amax=torch.from_numpy(a_dy).cuda())
    qx = nv.rht_quantize(to_device_bf16(x_pad), mask, "rn", segments=offp, amax=torch.from_numpy(a_x).cuda())
    dw = nv.grouped_gemm_k(offp, qdy, qx)
    torch.cuda.synchronize()
    del dy_pad, x_pad
    log("moe wgrad full size: oracle Hadamard operands per expert")

    def colseg(y, rounding, seed, offset, amax_vals):
        parts = _pmap(lambda r: oracle.quantize_1x16_colsegments(y[r[0]:r[1]], off_pad, rounding, seed, offset,
                                                                 amax_vals, np.arange(r[0], r[1])),
                      _ranges(len(y), 4 * WORKERS, 1))
        return _cat(parts, 0), _cat(parts, 1), parts[0][2]

    y_dy = _rht(dy, mask)
    ref_dy = colseg(y_dy, "sr", 23, 5, a_dy)
    del y_dy
    _same(host(qdy), ref_dy, "expert (H dY)^T SR")
    y_x = _rht(x, mask)
    ref_x = colseg(y_x, "rn", 0, 0, a_x)
    del y_x
    _same(host(qx), ref_x, "expert (H X)^T RN")
    log("moe wgrad full size: K-grouped GEMM")
    one = np.ones(1, np.float32)
    dqa = _deq((ref_dy[0], ref_dy[1], one))
    dqb = _deq((ref_x[0], ref_x[1], one))
    for g in range(G):
        t0, t1 = int(off_pad[g]), int(off_pad[g + 1])
        sg = float(ref_dy[2][g]) * float(ref_x[2][g])
        _gemm_in_bound_quiet(dw[g * n:(g + 1) * n], dqa[:, t0:t1] * sg, dqb[:, t0:t1], f"K-grouped wgrad expert {g}")
    log(f"K-grouped wgrad: every element of {G * n} x {k} within bound")
