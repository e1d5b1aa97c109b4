// Internal host-side launchers (not part of the C ABI). Shapes are validated by the caller
// (api.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

struct QuantOut {
  uint8_t* codes;
  uint8_t* scales;
  float* global_scale;
};

// Tensor amax of x[rows, cols]. With segments: amax_out[0..nseg) gets max|x| per segment
// (*parts = 1). Without: amax_out[0..*parts) gets partial maxima (at most 1024) whose max is
// the tensor amax; the encode launchers take (amax, parts) and fold the partials themselves.
hipError_t launch_amax_parts(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                             const int64_t* segments, int64_t nseg, float* amax_out, int* parts,
                             hipStream_t stream);

// out[i] = max of partial[i*parts .. (i+1)*parts) for i < count.
hipError_t launch_reduce_partials(const float* partial, int parts, float* out, hipStream_t stream,
                                  int count = 1);

hipError_t launch_encode_1x16(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                              bool sr, uint64_t seed, uint64_t offset,
                              const int64_t* segments, int64_t nseg, const float* amax, int parts,
                              QuantOut out, hipStream_t stream);

hipError_t launch_encode_16x16(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                               const int64_t* segments, int64_t nseg, const float* amax, int parts,
                               QuantOut out, const QuantOut* out_t, hipStream_t stream);

// Hadamard transform along tokens: partial maxima of the transformed tensor (at most 1024;
// with `plain`, *parts partial maxima of |x| itself come first, then those of the transformed
// tensor), and the transposed encode.
// With token segments (device int64[nseg + 1], multiples of 16): partial[0..nseg) receives the
// per-segment maxima of the transformed tensor (*parts = 1), and the encode takes one tensor
// scale per segment from amax[segment].
hipError_t launch_rht_amax_parts(const void* x, bool fp32, int64_t tokens, int64_t cols, int64_t ld,
                                 uint16_t sign_mask, bool plain, const int64_t* segments,
                                 int64_t nseg, float* partial, int* parts, hipStream_t stream);

hipError_t launch_rht_encode(const void* x, bool fp32, int64_t tokens, int64_t cols, int64_t ld,
                             uint16_t sign_mask, bool sr, uint64_t seed, uint64_t offset,
                             const int64_t* segments, int64_t nseg, const float* amax, int parts,
                             QuantOut out, hipStream_t stream);

// Rowwise rotation (each row's 16-blocks through the random-sign Hadamard transform) then
// 1x16 encode: partial maxima of the rotated tensor (*parts of them), and the encode.
hipError_t launch_rot_amax_parts(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                                 uint16_t mask, float* partial, int* parts, hipStream_t stream);
hipError_t launch_encode_rot(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld, uint16_t mask,
                             bool sr, uint64_t seed, uint64_t offset, const float* amax, int parts,
                             QuantOut out, hipStream_t stream);

// MXFP4 (E8M0 scale per 32 elements, no tensor scale): codes [rows, cols/2], scales
// [rows, cols/32]; cols % 32 == 0.
hipError_t launch_encode_mx(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                            bool sr, uint64_t seed, uint64_t offset, uint8_t* codes,
                            uint8_t* scales, hipStream_t stream);

// MXFP4 of x^T: x[rows, cols] -> codes [cols, rows/2], scales [cols, rows/32]; rows % 32 == 0.
hipError_t launch_encode_mx_cols(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld, bool sr,
                                 uint64_t seed, uint64_t offset, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream);

// p[0..n) = v
hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t stream);

constexpr int kMaxAmaxPartials = 1024;

struct GemmOperand {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global_scale;
};

hipError_t launch_gemm(GemmOperand a, GemmOperand b, int64_t M, int64_t N, int64_t K,
                       float* D, int64_t ldd, hipStream_t stream);

// MXFP4 GEMM (E8M0 scale per 32 along K, no tensor scale): D[M, N] FP32 = A B^T; K % 128 == 0.
hipError_t launch_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, float* D,
                          int64_t ldd, hipStream_t stream);

// The linear-layer form: kind 0 = FP32, 1 = FP32 added to D, 2 = BF16; amax (optional) gets
// max|stored D|. A partial last round is split along K with the parts' sums in ws
// (gemm_ex_workspace_bytes(M, N) bytes) and finished by a fixup kernel.
size_t gemm_ex_workspace_bytes(int64_t M, int64_t N);
hipError_t launch_gemm_ex(GemmOperand a, GemmOperand b, int64_t M, int64_t N, int64_t K, int kind,
                          void* D, int64_t ldd, float* amax, float* ws, hipStream_t stream);

hipError_t launch_grouped_gemm(int64_t G, const int64_t* m_offsets, GemmOperand a, GemmOperand b,
                               int64_t total_m, int64_t N, int64_t K, float* D, int64_t ldd,
                               hipStream_t stream);

// Groups along K (k_offsets: G + 1 multiples of 64), D [G*M, N]; K % 64 == 0.
hipError_t launch_grouped_gemm_k(int64_t G, const int64_t* k_offsets, GemmOperand a, GemmOperand b,
                                 int64_t M, int64_t N, int64_t K, float* D, int64_t ldd,
                                 hipStream_t stream);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* gscale,
                             const int64_t* segments, int64_t nseg, int64_t rows, int64_t cols,
                             float* y, hipStream_t stream);

}  // namespace nvfp4
