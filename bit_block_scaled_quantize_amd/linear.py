"""A linear layer whose three GEMMs run in NVFP4 on the library's kernels (autograd wrapper).

artiverse.ca "NVIDIA's 4-bit floating point pushes AI training limits" (paragraph on which
parts run in 4-bit) and the "Nemotron NVFP4" explainer ("Why 4-bit training normally falls
apart - and the three fixes") give the recipe this wrapper strings together; every step is a
call into libnvfp4, the wrapper only orders the calls and holds the buffers:

  forward   X [T, in] (BF16)  -> 1x16, nearest           -> Xq
            W [out, in]       -> 16x16, nearest, + W^T   -> Wq, WqT
            Y = Xq Wq^T, stored in BF16, with max|Y| from the GEMM epilogue (so the next
            layer's input quantization is a single pass: pass it as ``x_amax``)
  backward  dY [T, out]       -> max|dY| and max|H dY| from one read (amax pair); BF16 or
            FP32 gradients are quantized as they are
            dY -> 1x16, stochastic rounding                   -> dYq
            dX = dYq WqT^T, stored in BF16
            dY, X -> 16-point random-sign Hadamard transform along tokens, then 1x16 along
            tokens (dY stochastic, X nearest)                 -> (H dY)^T, (H X)^T
            dW = (H dY)^T (H X)^T^T in FP32, added into ``main_grad`` (or returned in the
            weight's dtype when the layer keeps no FP32 main gradient)

Stochastic rounding draws from Philox4x32-10 keyed by the layer's seed; call n of the layer's
backward uses counter offsets 2n (activation gradient) and 2n + 1 (weight gradient), so every
call draws fresh bits and a run is reproducible. Tokens (T) must be a multiple of 16 (the
Hadamard block), and in/out features multiples of 16 (the quantization block).
"""
from __future__ import annotations

import torch

from . import NVFP4Error, amax, amax_pair, gemm_ex, quantize, rht_quantize


class _LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, layer, x_amax):
        t = x.reshape(-1, x.shape[-1])
        if t.dtype != torch.bfloat16:
            raise NVFP4Error("the NVFP4 linear layer takes BF16 activations")
        t = t.contiguous()
        if t.shape[0] % 16:
            raise NVFP4Error(f"tokens ({t.shape[0]}) must be a multiple of 16")
        if x_amax is None:
            pair = amax_pair(t, layer.sign_mask)             # max|X|, max|H X| from one read
            x_amax, hx_amax = pair[0:1], pair[1:2]
        else:
            hx_amax = None                                   # taken in backward
        qx, _ = quantize(t, "1x16", "rn", amax=x_amax)
        qw, qwt = quantize(weight, "16x16", "rn", emit_transposed=True)
        y_amax = torch.empty((1,), dtype=torch.float32, device=t.device)
        y = gemm_ex(qx, qw, out_dtype=torch.bfloat16, amax_out=y_amax)
        layer.last_output_amax = y_amax
        ctx.layer = layer
        ctx.call = layer._calls
        layer._calls += 1
        ctx.hx_amax = hx_amax
        ctx.x_shape = x.shape
        ctx.weight_dtype = weight.dtype
        ctx.save_for_backward(t)
        ctx.qwt = qwt
        return y.view(*x.shape[:-1], weight.shape[0])

    @staticmethod
    def backward(ctx, dy):
        layer = ctx.layer
        (t,) = ctx.saved_tensors
        g = dy.reshape(-1, dy.shape[-1])
        if g.dtype not in (torch.bfloat16, torch.float32):
            g = g.float()                                    # exact widening; FP32 goes in as is
        g = g.contiguous()
        pair = amax_pair(g, layer.sign_mask)                 # max|dY|, max|H dY| from one read
        qdy, _ = quantize(g, "1x16", "sr", seed=layer.seed, offset=2 * ctx.call, amax=pair[0:1])
        dx = gemm_ex(qdy, ctx.qwt, out_dtype=torch.bfloat16)
        hx_amax = ctx.hx_amax
        if hx_amax is None:
            hx_amax = amax(t, rht=True, sign_mask=layer.sign_mask)
        qhdy = rht_quantize(g, layer.sign_mask, "sr", seed=layer.seed, offset=2 * ctx.call + 1,
                            amax=pair[1:2])
        qhx = rht_quantize(t, layer.sign_mask, "rn", amax=hx_amax)
        dw = None
        if layer.main_grad is not None:
            gemm_ex(qhdy, qhx, out=layer.main_grad, accumulate=True)
        else:
            out_dtype = ctx.weight_dtype if ctx.weight_dtype in (torch.bfloat16, torch.float32) else torch.float32
            dw = gemm_ex(qhdy, qhx, out_dtype=out_dtype).to(ctx.weight_dtype)   # rounded in the epilogue
        return dx.view(ctx.x_shape), dw, None, None


class NVFP4Linear(torch.nn.Module):
    """y = x W^T (no bias) with NVFP4 GEMMs; W is a BF16 parameter [out, in].

    main_grad: with ``fp32_main_grad`` (default) the weight gradient is accumulated into the
    FP32 tensor ``self.main_grad`` (zero it between optimizer steps) and ``weight.grad`` stays
    None; otherwise ``weight.grad`` receives it in BF16.
    last_output_amax: max|y| of the latest forward (a device float [1]), the ``x_amax`` of a
    following NVFP4Linear.
    """

    def __init__(self, in_features: int, out_features: int, device=None, sign_mask: int = 0x6E04,
                 seed: int = 0, fp32_main_grad: bool = True):
        super().__init__()
        if in_features % 16 or out_features % 16:
            raise NVFP4Error("in_features and out_features must be multiples of 16")
        self.weight = torch.nn.Parameter(torch.empty((out_features, in_features), dtype=torch.bfloat16,
                                                     device=device))
        self.main_grad = (torch.zeros((out_features, in_features), dtype=torch.float32, device=device)
                          if fp32_main_grad else None)
        self.sign_mask = sign_mask & 0xFFFF
        self.seed = seed
        self._calls = 0
        self.last_output_amax = None

    def forward(self, x: torch.Tensor, x_amax: torch.Tensor | None = None) -> torch.Tensor:
        return _LinearFn.apply(x, self.weight, self, x_amax)
