"""CPU oracle for NVFP4 block quantization, the random Hadamard transform and the
block-scaled GEMM.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this
package: only the tests, the smoke check and the bench's CPU-baseline leg use it. It shares
no code with the HIP library (no kernels, headers, helpers, tables or constant generators);
the only module both sides consume is ``workloads`` (seeded random inputs, no NVFP4 math).

The oracle is plain numpy, written from the format description on the pages:
  * "Nemotron NVFP4" explainer (ai.thesatyajit.com), section "What NVFP4 actually is":
    4-bit E2M1 elements (1 sign, 2 exponent, 1 mantissa bit), one FP8 E4M3 scale per 16
    elements, one FP32 scale per tensor (4.5 bits per element).
  * same page, section "Why 4-bit training normally falls apart - and the three fixes":
    2D (16x16) weight blocks, a random Hadamard transform on the wgrad inputs that is undone
    analytically, stochastic rounding for gradients only.
  * same page, the MXFP4 comparison: E2M1 elements with one power-of-two (E8M0) scale per
    32 elements, 4.25 bits per element (mx.py).
  * artiverse.ca "NVIDIA's 4-bit floating point pushes AI training limits" (stabilizer
    paragraph): 16x16 weight blocks instead of 1x16; stochastic rounding on gradients, not on
    activations; the Hadamard transform on the weight-gradient path.

Where the pages are silent (bit-level conventions, rounding order) the oracle follows the
readings stated in formats.py / quantize.py / hadamard.py / gemm.py / mx.py, each where it is used.

Parity status: every function here is pinned by tests under tests/test_oracle_*.py against
closed forms, library routines (numpy float16, torch float8_e4m3fn), published Philox
known-answer vectors, exact rational arithmetic or invariants. No function is unpinned.
"""
from .formats import (E2M1_MAX, E4M3_MAX, e2m1_decode, e2m1_encode_rn, e2m1_encode_sr,
                      e4m3_decode, e4m3_encode)
from .philox import philox4x32_10, block_random_bytes
from .quantize import (amax, global_scales, quantize_1x16, quantize_1x16_colsegments, quantize_16x16,
                       pack_nibbles,
                       unpack_nibbles, dequantize)
from .hadamard import (rht_columnwise, rht_columnwise_f64, hadamard_matrix_from_butterfly, rht_quantize,
                       rht_quantize_segments, rht_rowwise, rht_rowwise_quantize)
from .mx import (MX_BLOCK, e8m0_decode, mx_shared_exponent, quantize_mxfp4, dequantize_mxfp4)
from .gemm import (gemm_fp64, gemm_bound, grouped_gemm_fp64, grouped_gemm_bound, grouped_gemm_k_fp64,
                   grouped_gemm_k_bound, round_bf16, gemm_bf16_bound, gemm_accumulate_fp64,
                   gemm_accumulate_bound)

__all__ = [
    "E2M1_MAX", "E4M3_MAX", "e2m1_decode", "e2m1_encode_rn", "e2m1_encode_sr",
    "e4m3_decode", "e4m3_encode", "philox4x32_10", "block_random_bytes",
    "amax", "global_scales", "quantize_1x16", "quantize_1x16_colsegments", "quantize_16x16",
    "pack_nibbles",
    "unpack_nibbles", "dequantize", "rht_columnwise", "rht_columnwise_f64",
    "hadamard_matrix_from_butterfly", "rht_quantize", "rht_quantize_segments", "rht_rowwise",
    "rht_rowwise_quantize",
    "gemm_fp64", "gemm_bound", "grouped_gemm_fp64", "grouped_gemm_bound",
    "grouped_gemm_k_fp64", "grouped_gemm_k_bound", "round_bf16", "gemm_bf16_bound",
    "gemm_accumulate_fp64", "gemm_accumulate_bound",
    "MX_BLOCK", "e8m0_decode", "mx_shared_exponent", "quantize_mxfp4", "dequantize_mxfp4",
]
