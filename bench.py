"""Benchmark of the NVFP4 training hot path on one MI355X.

One step = the whole path of one dense linear layer (tokens 8192, in 5120, out 20480):
  amax pair of X (max|X|, max|HX|); quantize X (1x16, RN) and W (16x16, RN, + transposed
  copy)                                                              -> fprop GEMM
  amax pair of dY; quantize dY (1x16, SR)                            -> dgrad GEMM (W^T reused)
  Hadamard-transform + quantize dY^T (SR) and X^T (RN) along tokens  -> wgrad GEMM
`value` is the step's GEMM work (3 x 2*M*N*K) divided by the whole step time, inputs already
resident in HBM. Per-kernel times come from HIP events on the stream the kernels run on;
the mixture-of-experts rows (per-expert quantize, grouped GEMM) are timed the same way.

Prints ONE JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense FP16/BF16 MFMA, TFLOP/s
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 (MX-scaled) MFMA, TFLOP/s

M, K_IN, N_OUT = 8192, 5120, 20480

# HBM bytes per launch of the GEMM kernel on this workload (fprop/dgrad/wgrad average), from two
# rocprofv3 counter runs of this script (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same
# counter reads for the 256 MiB copy kernel of --copy-kernel. The figure belongs to the GEMM source
# whose SHA-256 is given; once that source changes it is reported as null until measured again.
GEMM_SOURCE = os.path.join(ROOT, "bit_block_scaled_quantize_amd", "csrc", "gemm.hip")
GEMM_TRAFFIC = {"source_sha256": "41c1d5afc5c57f7afc2fe811bcd6ac8a4f2432c1a7cddd08e958eea81c06c814",
                "bytes_per_launch": 1202316182}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-moe", action="store_true")
    p.add_argument("--no-mx", action="store_true", help="skip the MXFP4 comparison path")
    p.add_argument("--no-mosaic", action="store_true", help="skip the Mosaic recipe variant step")
    p.add_argument("--no-linear", action="store_true",
                   help="skip the linear-layer wrapper step (BF16 outputs, FP32 main gradient)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-reference", action="store_true",
                   help="skip timing the vendor FP16/BF16 GEMMs on the same shapes")
    p.add_argument("--kernel-reps", type=int, default=5, help="cold-cache repetitions per kernel")
    p.add_argument("--copy-kernel", action="store_true",
                   help="first run one plain 256 MiB fp32 copy kernel, the known-size reference "
                        "that scales the HBM byte counters of a profiler run")
    return p.parse_args()


def q_bytes(rows, cols, transposed=False):
    """Algorithmic bytes of one quantize call: read BF16 once, write codes + scales."""
    el = rows * cols
    return el * 2 + el * 0.5625 * (2 if transposed else 1)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; sharding across GPUs is not "
                                   "implemented, so only --gpus 1 is measured"}))
        sys.exit(2)

    import torch

    import bit_block_scaled_quantize_amd as nv
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    t0 = time.time()
    x_bits, w_bits = workloads.fprop()
    dy_bits = workloads.dgrad()
    mask = workloads.wgrad_sign_mask()
    X, W, dY = to_dev(x_bits), to_dev(w_bits), to_dev(dy_bits)
    gen_s = time.time() - t0

    T = nv.NVFP4Tensor
    Xq, Wq, WqT, dYq = T.empty(M, K_IN), T.empty(N_OUT, K_IN), T.empty(K_IN, N_OUT), T.empty(M, N_OUT)
    dYtq, Xtq = T.empty(N_OUT, M), T.empty(K_IN, M)
    Y = torch.empty((M, N_OUT), dtype=torch.float32, device=dev)
    dX = torch.empty((M, K_IN), dtype=torch.float32, device=dev)
    dW = torch.empty((N_OUT, K_IN), dtype=torch.float32, device=dev)
    ws = torch.empty((8192,), dtype=torch.uint8, device=dev)
    flush = torch.empty((512 << 20,), dtype=torch.uint8, device=dev)
    amax_xx = torch.empty((2,), dtype=torch.float32, device=dev)      # max|X|, max|H X|
    amax_dd = torch.empty((2,), dtype=torch.float32, device=dev)      # max|dY|, max|H dY|

    # X and dY are each quantized twice (rowwise for fprop/dgrad, Hadamard-transformed and
    # transposed for wgrad); one amax_pair read of each gives both tensor scales, so those
    # four quantize calls are single encode passes. W (one use) takes the two-pass call.
    stages = [
        ("amax_pair_x", lambda: nv.amax_pair(X, mask, out=amax_xx, workspace=ws)),
        ("quantize_x_1x16_rn", lambda: nv.quantize(X, "1x16", "rn", out=Xq, amax=amax_xx[0:1])),
        ("quantize_w_16x16_rn_t", lambda: nv.quantize(W, "16x16", "rn", emit_transposed=True,
                                                      out=Wq, out_t=WqT, workspace=ws)),
        ("gemm_fprop", lambda: nv.gemm(Xq, Wq, out=Y)),
        ("amax_pair_dy", lambda: nv.amax_pair(dY, mask, out=amax_dd, workspace=ws)),
        ("quantize_dy_1x16_sr", lambda: nv.quantize(dY, "1x16", "sr", seed=workloads.SR_SEED_DGRAD,
                                                    offset=0, out=dYq, amax=amax_dd[0:1])),
        ("gemm_dgrad", lambda: nv.gemm(dYq, WqT, out=dX)),
        ("rht_quantize_dy_sr", lambda: nv.rht_quantize(dY, mask, "sr", seed=workloads.SR_SEED_WGRAD,
                                                       offset=workloads.SR_OFFSET_WGRAD, out=dYtq,
                                                       amax=amax_dd[1:2])),
        ("rht_quantize_x_rn", lambda: nv.rht_quantize(X, mask, "rn", out=Xtq, amax=amax_xx[1:2])),
        ("gemm_wgrad", lambda: nv.gemm(dYtq, Xtq, out=dW)),
    ]
    work = {
        "amax_pair_x": ("GB/s", M * K_IN * 2),
        "amax_pair_dy": ("GB/s", M * N_OUT * 2),
        "quantize_x_1x16_rn": ("GB/s", q_bytes(M, K_IN)),
        "quantize_w_16x16_rn_t": ("GB/s", q_bytes(N_OUT, K_IN, transposed=True)),
        "quantize_dy_1x16_sr": ("GB/s", q_bytes(M, N_OUT)),
        "rht_quantize_dy_sr": ("GB/s", q_bytes(M, N_OUT)),
        "rht_quantize_x_rn": ("GB/s", q_bytes(M, K_IN)),
        "gemm_fprop": ("TFLOP/s", 2.0 * M * N_OUT * K_IN),
        "gemm_dgrad": ("TFLOP/s", 2.0 * M * K_IN * N_OUT),
        "gemm_wgrad": ("TFLOP/s", 2.0 * N_OUT * K_IN * M),
    }
    step_flops = sum(v for u, v in work.values() if u == "TFLOP/s")

    def run_step(events=None):
        for i, (_, fn) in enumerate(stages):
            if events is not None and events[i] is not None:
                events[i][0].record(stream)
            fn()
            if events is not None and events[i] is not None:
                events[i][1].record(stream)

    if args.copy_kernel:
        src = torch.ones((64 << 20,), dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # --- timed region: K whole steps, events around the three GEMM launches only ------------
    def new_events(which):
        return [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 if which(name) else None for name, _ in stages] for _ in range(args.steps)]
    is_gemm = lambda name: name.startswith("gemm_")
    gev = new_events(is_gemm)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(args.steps):
        run_step(gev[s])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    # the other stages' times: a second pass of K steps with events around them (outside the
    # timed region: twenty event markers per step measured 1-2% of the step time)
    qev = new_events(lambda name: not is_gemm(name))
    for s in range(args.steps):
        run_step(qev[s])
    torch.cuda.synchronize()
    ev = [[g if g is not None else q for g, q in zip(gs, qs)] for gs, qs in zip(gev, qev)]
    stage_ms = {name: float(np.mean([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]))
                for i, (name, _) in enumerate(stages)}

    def rate(name, ms):
        unit, amount = work[name]
        if unit == "GB/s":
            val = amount / (ms * 1e-3) / 1e9
            return {"us": round(ms * 1e3, 2), "GB/s": round(val, 1), "frac_hbm": round(val / HBM_PEAK_GBS, 4)}
        val = amount / (ms * 1e-3) / 1e12
        return {"us": round(ms * 1e3, 2), "TFLOP/s": round(val, 1), "frac_mfma_f16": round(val / MFMA_F16_PEAK_TFLOPS, 4)}

    breakdown = {name: rate(name, ms) for name, ms in stage_ms.items()}

    # --- cold-cache timing of each quantize call (inputs in HBM, caches holding other data) --
    # Before every timed call a 512 MB buffer (written once, up front) is read, which evicts the
    # 256 MB Infinity Cache and the L2s without leaving dirty lines whose write-back would
    # overlap the timed kernel. Each quantize is timed three ways: the stand-alone two-pass call
    # (workspace, no amax_in), the encode pass alone (tensor amax supplied, the pass the HBM
    # roofline applies to), and its amax pass alone; the step's amax_pair calls are timed too.
    flush.fill_(1)
    fsum = torch.empty((1,), dtype=torch.int64, device=dev)

    def cold_ms(fn):
        times = []
        for _ in range(args.kernel_reps):
            torch.sum(flush.view(torch.int64), dim=0, out=fsum[0])
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        return float(np.median(times))

    amx_x, amx_w, amx_dy = nv.amax(X), nv.amax(W), nv.amax(dY)
    ramx_dy, ramx_x = nv.amax(dY, rht=True, sign_mask=mask), nv.amax(X, rht=True, sign_mask=mask)
    two_pass = {
        "quantize_x_1x16_rn": lambda: nv.quantize(X, "1x16", "rn", out=Xq, workspace=ws),
        "quantize_w_16x16_rn_t": lambda: nv.quantize(W, "16x16", "rn", emit_transposed=True,
                                                     out=Wq, out_t=WqT, workspace=ws),
        "quantize_dy_1x16_sr": lambda: nv.quantize(dY, "1x16", "sr", seed=workloads.SR_SEED_DGRAD,
                                                   offset=0, out=dYq, workspace=ws),
        "rht_quantize_dy_sr": lambda: nv.rht_quantize(dY, mask, "sr", seed=workloads.SR_SEED_WGRAD,
                                                      offset=workloads.SR_OFFSET_WGRAD, out=dYtq,
                                                      workspace=ws),
        "rht_quantize_x_rn": lambda: nv.rht_quantize(X, mask, "rn", out=Xtq, workspace=ws),
    }
    encode_only = {
        "quantize_x_1x16_rn": lambda: nv.quantize(X, "1x16", "rn", out=Xq, amax=amx_x),
        "quantize_w_16x16_rn_t": lambda: nv.quantize(W, "16x16", "rn", emit_transposed=True,
                                                     out=Wq, out_t=WqT, amax=amx_w),
        "quantize_dy_1x16_sr": lambda: nv.quantize(dY, "1x16", "sr", seed=workloads.SR_SEED_DGRAD,
                                                   offset=0, out=dYq, amax=amx_dy),
        "rht_quantize_dy_sr": lambda: nv.rht_quantize(dY, mask, "sr", seed=workloads.SR_SEED_WGRAD,
                                                      offset=workloads.SR_OFFSET_WGRAD, out=dYtq,
                                                      amax=ramx_dy),
        "rht_quantize_x_rn": lambda: nv.rht_quantize(X, mask, "rn", out=Xtq, amax=ramx_x),
    }
    amax_only = {
        "quantize_x_1x16_rn": (lambda: nv.amax(X, workspace=ws), M * K_IN * 2),
        "quantize_w_16x16_rn_t": (lambda: nv.amax(W, workspace=ws), N_OUT * K_IN * 2),
        "quantize_dy_1x16_sr": (lambda: nv.amax(dY, workspace=ws), M * N_OUT * 2),
        "rht_quantize_dy_sr": (lambda: nv.amax(dY, rht=True, sign_mask=mask, workspace=ws), M * N_OUT * 2),
        "rht_quantize_x_rn": (lambda: nv.amax(X, rht=True, sign_mask=mask, workspace=ws), M * K_IN * 2),
    }
    cold = {}
    for name, fn in two_pass.items():
        row = {"two_pass": rate(name, cold_ms(fn)), "encode_pass": rate(name, cold_ms(encode_only[name]))}
        afn, abytes = amax_only[name]
        ams = cold_ms(afn)
        av = abytes / (ams * 1e-3) / 1e9
        row["amax_pass"] = {"us": round(ams * 1e3, 2), "GB/s": round(av, 1), "frac_hbm": round(av / HBM_PEAK_GBS, 4)}
        cold[name] = row
    for name, fn in stages:
        if name.startswith("amax_pair"):
            cold[name] = rate(name, cold_ms(fn))

    gemm_names = ["gemm_fprop", "gemm_dgrad", "gemm_wgrad"]
    gemm_avg_ms = float(np.mean([stage_ms[n] for n in gemm_names]))
    achieved = (2.0 * M * N_OUT * K_IN) / (gemm_avg_ms * 1e-3) / 1e12

    out = {
        "metric": "NVFP4 GEMM TFLOP/s (fprop/dgrad/wgrad) + quantize GB/s, % of roofline",
        "value": round(step_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16-mfma/fp32-acc",
        "data": "synthetic",
        "config": {"workload": "dense linear layer NVFP4 training step (fprop+dgrad+wgrad), "
                               "tokens 8192, in 5120, out 20480",
                   "tokens": M, "in_features": K_IN, "out_features": N_OUT,
                   "weights": "16x16 blocks", "grad_rounding": "stochastic",
                   "wgrad_transform": "16-point random-sign Hadamard", "parallelism": "none"},
        "roofline": {"bound": "mfma", "kernel": "k_gemm (fprop/dgrad/wgrad average)",
                     "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": gemm_traffic()},
        "breakdown": breakdown,
        "quantize_cold_cache": cold,
        "input_gen_s": round(gen_s, 1),
    }

    if not args.no_linear:
        out["linear_layer"] = bench_linear(nv, workloads, torch, dev, stream, flush, X, W, dY, mask,
                                           step_flops, args)
    if not args.no_mosaic:
        out["mosaic"] = bench_mosaic(nv, workloads, torch, dev, stream, X, W, dY, mask, step_flops, args)
    if not args.no_mx:
        out["mxfp4"] = bench_mx(nv, workloads, torch, dev, stream, flush, X, W, dY, args)
    if not args.no_moe:
        out["moe"] = bench_moe(nv, workloads, torch, dev, stream, flush, args)
    if not args.no_reference:
        out["reference_gemm"] = reference_gemm(torch, dev, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x_bits, w_bits, dy_bits, mask, step_flops)
    print(json.dumps(out))


def gemm_traffic():
    """Counter-derived HBM bytes per GEMM launch, or None when the kernel source differs from the
    one the counters were taken on."""
    import hashlib
    with open(GEMM_SOURCE, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if GEMM_TRAFFIC["source_sha256"] != digest:
        return None
    return GEMM_TRAFFIC["bytes_per_launch"]


def bench_linear(nv, workloads, torch, dev, stream, flush, X, W, dY, mask, step_flops, args):
    """The same layer through the autograd wrapper (NVFP4Linear): forward output and activation
    gradient stored in BF16 with their amax from the GEMM epilogue, the weight gradient
    accumulated into an FP32 main gradient; one step = forward + backward, timed like the main
    step. Also each linear-layer GEMM alone (cold), against the FP32-output GEMM."""
    from bit_block_scaled_quantize_amd.linear import NVFP4Linear
    layer = NVFP4Linear(K_IN, N_OUT, device=dev, sign_mask=mask, seed=workloads.SR_SEED_DGRAD)
    with torch.no_grad():
        layer.weight.copy_(W)
    Xg = X.detach().requires_grad_(True)

    def step():
        Xg.grad = None
        y = layer(Xg)
        y.backward(dY)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    res = {"ms_per_step": round(ms, 4), "TFLOP/s": round(step_flops / (ms * 1e-3) / 1e12, 1),
           "outputs": "y, dX BF16 with fused amax; dW accumulated into FP32 main_grad"}

    T = nv.NVFP4Tensor
    Xq, Wq, WqT, dYq = T.empty(M, K_IN), T.empty(N_OUT, K_IN), T.empty(K_IN, N_OUT), T.empty(M, N_OUT)
    dYtq, Xtq = T.empty(N_OUT, M), T.empty(K_IN, M)
    nv.quantize(X, "1x16", "rn", out=Xq)
    nv.quantize(W, "16x16", "rn", emit_transposed=True, out=Wq, out_t=WqT)
    nv.quantize(dY, "1x16", "sr", seed=1, out=dYq)
    nv.rht_quantize(dY, mask, "sr", seed=2, out=dYtq)
    nv.rht_quantize(X, mask, "rn", out=Xtq)
    amax = torch.empty((1,), dtype=torch.float32, device=dev)
    Y16 = torch.empty((M, N_OUT), dtype=torch.bfloat16, device=dev)
    dX16 = torch.empty((M, K_IN), dtype=torch.bfloat16, device=dev)
    G = torch.zeros((N_OUT, K_IN), dtype=torch.float32, device=dev)
    wsz = max(nv.workspace_size(nv.OP_GEMM_EX, m_, n_) for m_, n_ in ((M, N_OUT), (M, K_IN), (N_OUT, K_IN)))
    ws = torch.empty((max(wsz, 1),), dtype=torch.uint8, device=dev)
    flops = 2.0 * M * N_OUT * K_IN
    calls = {
        "gemm_ex_fprop_bf16_amax": (lambda: nv.gemm_ex(Xq, Wq, out=Y16, out_dtype=torch.bfloat16,
                                                       amax_out=amax, workspace=ws), "TFLOP/s", flops),
        "gemm_ex_dgrad_bf16_amax": (lambda: nv.gemm_ex(dYq, WqT, out=dX16, out_dtype=torch.bfloat16,
                                                       amax_out=amax, workspace=ws), "TFLOP/s", flops),
        "gemm_ex_wgrad_fp32_accumulate": (lambda: nv.gemm_ex(dYtq, Xtq, out=G, accumulate=True,
                                                             workspace=ws), "TFLOP/s", flops),
    }
    fsum = torch.empty((1,), dtype=torch.int64, device=dev)
    res.update(_time_calls(calls, torch, stream, flush, fsum, args))
    return res


def bench_mosaic(nv, workloads, torch, dev, stream, X, W, dY, mask, step_flops, args):
    """The Mosaic recipe variant of the same layer step (Hadamard transforms on both backward
    GEMMs, 1D weights): W 1x16 RN for fprop and W^T transformed along the output features for
    dgrad; dY transformed rowwise (SR) for dgrad and along tokens (SR) for wgrad; X as in the
    main step. Timed like the main step (K steps between events on the kernels' stream)."""
    T = nv.NVFP4Tensor
    Xq, Wq, WqR, dYr = T.empty(M, K_IN), T.empty(N_OUT, K_IN), T.empty(K_IN, N_OUT), T.empty(M, N_OUT)
    dYtq, Xtq = T.empty(N_OUT, M), T.empty(K_IN, M)
    Y = torch.empty((M, N_OUT), dtype=torch.float32, device=dev)
    dX = torch.empty((M, K_IN), dtype=torch.float32, device=dev)
    dW = torch.empty((N_OUT, K_IN), dtype=torch.float32, device=dev)
    ws = torch.empty((8192,), dtype=torch.uint8, device=dev)
    ax = torch.empty((2,), dtype=torch.float32, device=dev)
    ady = torch.empty((2,), dtype=torch.float32, device=dev)
    stages = [
        lambda: nv.amax_pair(X, mask, out=ax, workspace=ws),
        lambda: nv.quantize(X, "1x16", "rn", out=Xq, amax=ax[0:1]),
        lambda: nv.quantize(W, "1x16", "rn", out=Wq, workspace=ws),
        lambda: nv.rht_quantize(W, mask, "rn", out=WqR, workspace=ws),
        lambda: nv.gemm(Xq, Wq, out=Y),
        lambda: nv.amax(dY, rht=2, sign_mask=mask, out=ady[0:1], workspace=ws),
        lambda: nv.amax(dY, rht=True, sign_mask=mask, out=ady[1:2], workspace=ws),
        lambda: nv.rht_rows_quantize(dY, mask, "sr", seed=workloads.SR_SEED_DGRAD, out=dYr, amax=ady[0:1]),
        lambda: nv.gemm(dYr, WqR, out=dX),
        lambda: nv.rht_quantize(dY, mask, "sr", seed=workloads.SR_SEED_WGRAD, offset=workloads.SR_OFFSET_WGRAD,
                                out=dYtq, amax=ady[1:2]),
        lambda: nv.rht_quantize(X, mask, "rn", out=Xtq, amax=ax[1:2]),
        lambda: nv.gemm(dYtq, Xtq, out=dW),
    ]

    def step():
        for fn in stages:
            fn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    return {"ms_per_step": round(ms, 4), "TFLOP/s": round(step_flops / (ms * 1e-3) / 1e12, 1),
            "recipe": "1x16 weights; Hadamard on dgrad (rowwise dY, W along N) and wgrad (along tokens)"}


def bench_mx(nv, workloads, torch, dev, stream, flush, X, W, dY, args):
    """The comparison format of the pages, MXFP4 (E8M0 scale per 32 elements, no tensor scale),
    on the same layer: quantize (single pass: no amax) and the three GEMMs on gfx950's
    block-scaled FP4 matrix instruction, against its 10.1 PFLOP/s peak. Each GEMM operand is
    quantized along its contraction: W, dY and X row-wise for the forward and the gradients' left
    operands, and W^T, dY^T, X^T by the column quantization straight from W, dY and X (no
    transposed copies). Cold caches, median of --kernel-reps."""
    T = nv.MXFP4Tensor
    qX, qW, qdY, qWt = T.empty(M, K_IN), T.empty(N_OUT, K_IN), T.empty(M, N_OUT), T.empty(K_IN, N_OUT)
    qdYt, qXt = T.empty(N_OUT, M), T.empty(K_IN, M)
    for src, q, rnd in ((X, qX, "rn"), (W, qW, "rn"), (dY, qdY, "sr")):
        nv.mx_quantize(src, rnd, seed=7, out=q)
    for src, q, rnd in ((W, qWt, "rn"), (dY, qdYt, "sr"), (X, qXt, "rn")):
        nv.mx_quantize_columns(src, rnd, seed=7, out=q)
    Y = torch.empty((M, N_OUT), dtype=torch.float32, device=dev)
    dX = torch.empty((M, K_IN), dtype=torch.float32, device=dev)
    dW = torch.empty((N_OUT, K_IN), dtype=torch.float32, device=dev)
    flops = 2.0 * M * N_OUT * K_IN
    mxq = lambda rows, cols: rows * cols * (2 + 0.5 + 1.0 / 32)     # BF16 in, codes + E8M0 out
    calls = {
        "mx_quantize_x_rn": (lambda: nv.mx_quantize(X, "rn", out=qX), "GB/s", mxq(M, K_IN)),
        "mx_quantize_dy_sr": (lambda: nv.mx_quantize(dY, "sr", seed=7, out=qdY), "GB/s", mxq(M, N_OUT)),
        "mx_quantize_w_rn": (lambda: nv.mx_quantize(W, "rn", out=qW), "GB/s", mxq(N_OUT, K_IN)),
        "mx_quantize_columns_wt_rn": (lambda: nv.mx_quantize_columns(W, "rn", out=qWt), "GB/s", mxq(N_OUT, K_IN)),
        "mx_quantize_columns_dyt_sr": (lambda: nv.mx_quantize_columns(dY, "sr", seed=7, out=qdYt), "GB/s",
                                       mxq(M, N_OUT)),
        "mx_quantize_columns_xt_rn": (lambda: nv.mx_quantize_columns(X, "rn", out=qXt), "GB/s", mxq(M, K_IN)),
        "mx_gemm_fprop": (lambda: nv.mx_gemm(qX, qW, out=Y), "TFLOP/s", flops),
        "mx_gemm_dgrad": (lambda: nv.mx_gemm(qdY, qWt, out=dX), "TFLOP/s", flops),
        "mx_gemm_wgrad": (lambda: nv.mx_gemm(qdYt, qXt, out=dW), "TFLOP/s", flops),
    }
    fsum = torch.empty((1,), dtype=torch.int64, device=dev)
    res = _time_calls(calls, torch, stream, flush, fsum, args)
    for k in ("mx_gemm_fprop", "mx_gemm_dgrad", "mx_gemm_wgrad"):
        res[k]["frac_mfma_fp4"] = round(res[k]["TFLOP/s"] / MFMA_FP4_PEAK_TFLOPS, 4)
        del res[k]["frac_mfma_f16"]
    res["bits_per_element"] = 4.25
    return res


def bench_moe(nv, workloads, torch, dev, stream, flush, args):
    """The expert layer (128 experts, top-6 of 16384 tokens, hidden 2688, expert FFN 1856).
    Forward: per-expert quantize of the expert-sorted activations and stacked weights, then the
    grouped fprop GEMM. Backward, on the layout with each expert's tokens padded to a multiple
    of 64 with zero rows: the weights in 16x16 tiles with every expert's transpose, dY per
    expert in 1x16 SR, the grouped activation-gradient GEMM; dY and X transformed along tokens
    and quantized per expert, the weight-gradient GEMM grouped along K. GEMM rates count the
    real tokens only (2 * tokens * ffn * hidden per GEMM)."""
    fsum = torch.empty((1,), dtype=torch.int64, device=dev)
    x_bits, w_bits, off = workloads.moe()
    G, n, k = workloads.MOE_EXPERTS, workloads.MOE_FFN, workloads.MOE_HIDDEN
    total = int(off[-1])
    X = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    Wt = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    offd = torch.from_numpy(off).to(dev)
    wseg = torch.arange(G + 1, dtype=torch.int64, device=dev) * n
    Xq, Wq = nv.NVFP4Tensor.empty(total, k, G), nv.NVFP4Tensor.empty(G * n, k, G)
    D = torch.empty((total, n), dtype=torch.float32, device=dev)
    ws = torch.empty((4096,), dtype=torch.uint8, device=dev)
    flops = 2.0 * total * n * k
    calls = {
        "quantize_x_experts_1x16_rn": (lambda: nv.quantize(X, "1x16", "rn", segments=offd, out=Xq, workspace=ws),
                                       "GB/s", q_bytes(total, k)),
        "quantize_w_experts_16x16_rn": (lambda: nv.quantize(Wt, "16x16", "rn", segments=wseg, out=Wq, workspace=ws),
                                        "GB/s", q_bytes(G * n, k)),
        "grouped_gemm": (lambda: nv.grouped_gemm(offd, Xq, Wq, n, out=D), "TFLOP/s", flops),
    }
    # the two passes of each per-expert call timed apart: the amax pass (per-expert maxima) and
    # the encode pass with those maxima supplied (the pass the HBM roofline applies to)
    ax = nv.amax(X, segments=offd)
    aw = nv.amax(Wt, segments=wseg)
    calls.update({
        "amax_x_experts": (lambda: nv.amax(X, segments=offd, out=ax), "GB/s", 2.0 * total * k),
        "quantize_x_experts_1x16_rn_encode_pass": (
            lambda: nv.quantize(X, "1x16", "rn", segments=offd, amax=ax, out=Xq, workspace=ws), "GB/s", q_bytes(total, k)),
        "amax_w_experts": (lambda: nv.amax(Wt, segments=wseg, out=aw), "GB/s", 2.0 * G * n * k),
        "quantize_w_experts_16x16_rn_encode_pass": (
            lambda: nv.quantize(Wt, "16x16", "rn", segments=wseg, amax=aw, out=Wq, workspace=ws), "GB/s", q_bytes(G * n, k)),
    })
    res = _time_calls(calls, torch, stream, flush, fsum, args)
    del D, Xq

    # backward on the padded token layout
    x_pad, dy_pad, off_pad = workloads.moe_backward(x_bits, off)
    tp = int(off_pad[-1])
    Xp = torch.from_numpy(x_pad.view(np.int16)).view(torch.bfloat16).to(dev)
    dY = torch.from_numpy(dy_pad.view(np.int16)).view(torch.bfloat16).to(dev)
    del x_pad, dy_pad
    offp = torch.from_numpy(off_pad).to(dev)
    mask = workloads.wgrad_sign_mask()
    WqT = nv.NVFP4Tensor.empty(G * k, n, G)
    dYq = nv.NVFP4Tensor.empty(tp, n, G)
    dYt, Xt = nv.NVFP4Tensor.empty(n, tp, G), nv.NVFP4Tensor.empty(k, tp, G)
    dX = torch.empty((tp, k), dtype=torch.float32, device=dev)
    dW = torch.empty((G * n, k), dtype=torch.float32, device=dev)
    ws_r = torch.empty((nv.workspace_size(nv.OP_RHT_QUANTIZE, tp, n, G),), dtype=torch.uint8, device=dev)
    calls = {
        "quantize_w_experts_16x16_rn_transposed": (
            lambda: nv.quantize(Wt, "16x16", "rn", emit_transposed=True, segments=wseg, out=Wq, out_t=WqT,
                                workspace=ws), "GB/s", q_bytes(G * n, k, transposed=True)),
        "quantize_dy_experts_1x16_sr": (
            lambda: nv.quantize(dY, "1x16", "sr", seed=11, segments=offp, out=dYq, workspace=ws),
            "GB/s", q_bytes(tp, n)),
        "grouped_gemm_dgrad": (lambda: nv.grouped_gemm(offp, dYq, WqT, k, out=dX), "TFLOP/s", flops),
        "rht_quantize_dy_experts_sr": (
            lambda: nv.rht_quantize(dY, mask, "sr", seed=12, segments=offp, out=dYt, workspace=ws_r),
            "GB/s", q_bytes(tp, n)),
        "rht_quantize_x_experts_rn": (
            lambda: nv.rht_quantize(Xp, mask, "rn", segments=offp, out=Xt, workspace=ws_r),
            "GB/s", q_bytes(tp, k)),
        "grouped_gemm_k_wgrad": (lambda: nv.grouped_gemm_k(offp, dYt, Xt, out=dW), "TFLOP/s", flops),
    }
    ady = nv.amax(dY, segments=offp)
    ahdy = nv.amax(dY, segments=offp, rht=True, sign_mask=mask)
    ahx = nv.amax(Xp, segments=offp, rht=True, sign_mask=mask)
    calls.update({
        "quantize_w_experts_16x16_rn_transposed_encode_pass": (
            lambda: nv.quantize(Wt, "16x16", "rn", emit_transposed=True, segments=wseg, amax=aw, out=Wq, out_t=WqT,
                                workspace=ws), "GB/s", q_bytes(G * n, k, transposed=True)),
        "amax_dy_experts": (lambda: nv.amax(dY, segments=offp, out=ady), "GB/s", 2.0 * tp * n),
        "quantize_dy_experts_1x16_sr_encode_pass": (
            lambda: nv.quantize(dY, "1x16", "sr", seed=11, segments=offp, amax=ady, out=dYq, workspace=ws),
            "GB/s", q_bytes(tp, n)),
        "amax_rht_dy_experts": (lambda: nv.amax(dY, segments=offp, rht=True, sign_mask=mask, out=ahdy), "GB/s", 2.0 * tp * n),
        "rht_quantize_dy_experts_sr_encode_pass": (
            lambda: nv.rht_quantize(dY, mask, "sr", seed=12, segments=offp, amax=ahdy, out=dYt, workspace=ws_r),
            "GB/s", q_bytes(tp, n)),
        "amax_rht_x_experts": (lambda: nv.amax(Xp, segments=offp, rht=True, sign_mask=mask, out=ahx), "GB/s", 2.0 * tp * k),
        "rht_quantize_x_experts_rn_encode_pass": (
            lambda: nv.rht_quantize(Xp, mask, "rn", segments=offp, amax=ahx, out=Xt, workspace=ws_r),
            "GB/s", q_bytes(tp, k)),
    })
    res.update(_time_calls(calls, torch, stream, flush, fsum, args))
    res["config"] = {"experts": G, "tokens": workloads.MOE_TOKENS, "topk": workloads.MOE_TOPK,
                     "hidden": k, "ffn": n, "rows_total": total, "rows_total_padded_64": tp,
                     "rows_per_expert_max": int(np.diff(off).max()),
                     "rows_per_expert_min": int(np.diff(off).min())}
    return res


def _time_calls(calls, torch, stream, flush, fsum, args):
    """Median cold (L2 and MALL flushed) time of each call and its rate."""
    res = {}
    for name, (fn, unit, amount) in calls.items():
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(max(args.kernel_reps, 3)):
            torch.sum(flush.view(torch.int64), dim=0, out=fsum[0])
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        ms = float(np.median(times))
        if unit == "GB/s":
            v = amount / (ms * 1e-3) / 1e9
            res[name] = {"us": round(ms * 1e3, 2), "GB/s": round(v, 1), "frac_hbm": round(v / HBM_PEAK_GBS, 4)}
        else:
            v = amount / (ms * 1e-3) / 1e12
            res[name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(v, 1),
                         "frac_mfma_f16": round(v / MFMA_F16_PEAK_TFLOPS, 4)}
    return res


def reference_gemm(torch, dev, stream):
    """The vendor library's dense FP16 and BF16 GEMMs (torch.matmul -> hipBLASLt) on the three
    GEMM shapes of the step, same box and clock regime: context for the NVFP4 GEMM, which
    also decodes its operands and writes FP32. Random normal operands, output in the input
    dtype, mean of 5 warm launches."""
    res = {}
    shapes = {"fprop": (M, N_OUT, K_IN), "dgrad": (M, K_IN, N_OUT), "wgrad": (N_OUT, K_IN, M)}
    for name, (m, n, k) in shapes.items():
        row = {}
        for dt, tag in ((torch.float16, "fp16"), (torch.bfloat16, "bf16")):
            a = torch.randn((m, k), device=dev, dtype=dt)
            b = torch.randn((n, k), device=dev, dtype=dt)
            d = torch.empty((m, n), device=dev, dtype=dt)
            for _ in range(2):
                torch.matmul(a, b.t(), out=d)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            ev0.record(stream)
            for _ in range(5):
                torch.matmul(a, b.t(), out=d)
            ev1.record(stream)
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1) / 5
            row[f"{tag}_TFLOP/s"] = round(2.0 * m * n * k / (ms * 1e-3) / 1e12, 1)
            del a, b, d
        res[name] = row
    res["library"] = "torch.matmul (hipBLASLt), dense, operands already in FP16/BF16"
    return res


def _oracle_tiny_step():
    """The whole step of the tiny 256 x 256 x 256 layer through the oracle, timed in full (no
    sampling): tensor maxima, X 1x16 RN, W 16x16 RN and W^T, dY 1x16 SR, both Hadamard
    operands, and the three FP64 GEMMs of the dequantized operands."""
    import oracle
    import workloads
    f32 = workloads.bf16_bits_to_f32
    a_bits, w_bits = workloads.tiny()
    x, w = f32(a_bits), f32(w_bits)
    dy = f32(workloads.normal_bf16((256, 256), workloads.SEEDS["dgrad_dy"], std=1e-3))
    mask = workloads.wgrad_sign_mask()
    t0 = time.perf_counter()
    deq = oracle.dequantize
    xq = oracle.quantize_1x16(x)
    wq = oracle.quantize_16x16(w)
    wtq = oracle.quantize_16x16(np.ascontiguousarray(w.T))
    dyq = oracle.quantize_1x16(dy, "sr", seed=workloads.SR_SEED_DGRAD, offset=0)
    hdy = oracle.rht_quantize(dy, mask, "sr", seed=workloads.SR_SEED_WGRAD, offset=workloads.SR_OFFSET_WGRAD)
    hx = oracle.rht_quantize(x, mask, "rn")
    oracle.gemm_fp64(deq(*xq), deq(*wq))
    oracle.gemm_fp64(deq(*dyq), deq(*wtq))
    oracle.gemm_fp64(deq(*hdy), deq(*hx))
    return time.perf_counter() - t0


def cpu_baseline(x_bits, w_bits, dy_bits, mask, step_flops):
    """The oracle (numpy; BLAS dgemm for the FP64 reference GEMM) on the machine's host: timed on a
    bounded sample of the same step and scaled to the whole step (value), and timed in full on
    the tiny 256^3 layer (tiny_full, no extrapolation)."""
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    tiny_s = min(_oracle_tiny_step() for _ in range(3))
    tiny_flops = 3 * 2 * 256 ** 3
    f32 = workloads.bf16_bits_to_f32
    rng = np.random.default_rng(0)
    parts = []

    sample_times = []

    def timed(fn):
        t = time.perf_counter()
        r = fn()
        sample_times.append(time.perf_counter() - t)
        return sample_times[-1], r

    rows = 2048
    xs = f32(x_bits[:rows])
    A = oracle.amax(xs)
    t, _ = timed(lambda: oracle.quantize_1x16(xs, amax_vals=A))
    parts.append(t * M / rows)
    ws_ = f32(w_bits[:rows])
    t, _ = timed(lambda: (oracle.quantize_16x16(ws_, amax_vals=A),
                          oracle.quantize_16x16(np.ascontiguousarray(ws_.T), amax_vals=A)))
    parts.append(t * N_OUT / rows)
    dy_rows = 768
    dys = f32(dy_bits[:dy_rows])
    t, _ = timed(lambda: oracle.quantize_1x16(dys, "sr", seed=1, offset=0, amax_vals=A))
    parts.append(t * M / dy_rows)
    cols = 1024
    t, _ = timed(lambda: oracle.rht_quantize(f32(dy_bits[:, :cols]), mask, "sr", seed=1,
                                             amax_vals=A, col_ids=np.arange(cols)))
    parts.append(t * N_OUT / cols)
    t, _ = timed(lambda: oracle.rht_quantize(f32(x_bits[:, :cols]), mask, "rn",
                                             amax_vals=A, col_ids=np.arange(cols)))
    parts.append(t * K_IN / cols)
    # reference GEMM: a block of output rows of each GEMM against the full other operand
    g_rows = 1536
    a_hat = rng.standard_normal((g_rows, K_IN))
    b_hat = rng.standard_normal((N_OUT, K_IN))
    t, _ = timed(lambda: oracle.gemm_fp64(a_hat, b_hat))
    parts.append(3 * t * M / g_rows)
    sampled_s = float(sum(t for t in sample_times))
    total_s = float(sum(parts))
    return {"value": round(step_flops / total_s / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(os.cpu_count() or 1), "blas_threads": blas_threads, "kind": "oracle",
            "sample": f"oracle on {rows} rows of X and of W, {dy_rows} rows of dY, {cols} columns of "
                      f"each Hadamard operand and {g_rows} output rows of each FP64 GEMM "
                      f"({sampled_s:.1f} s measured), scaled to the full step: an estimate "
                      f"({total_s:.1f} s per step; numpy elementwise on 1 core, BLAS on "
                      f"{blas_threads} threads)",
            "tiny_full": {"seconds": round(tiny_s, 4),
                          "value": round(tiny_flops / tiny_s / 1e12, 9), "unit": "TFLOP/s",
                          "what": "the whole oracle step of the 256x256x256 layer (maxima, X 1x16, "
                                  "W 16x16 and W^T, dY SR, both Hadamard operands, three FP64 "
                                  "GEMMs), measured in full, best of 3"}}


if __name__ == "__main__":
    main()
