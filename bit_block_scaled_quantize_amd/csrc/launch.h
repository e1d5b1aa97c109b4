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

// amax: zero amax_out[0..nseg) and accumulate max|x| per row segment.
hipError_t launch_amax(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                       const int64_t* segments, int64_t nseg, float* amax_out,
                       hipStream_t stream);

hipError_t launch_encode_1x16(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                              bool sr, uint64_t seed, uint64_t offset,
                              const int64_t* segments, int64_t nseg, const float* amax,
                              QuantOut out, hipStream_t stream);

hipError_t launch_encode_16x16(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                               const int64_t* segments, int64_t nseg, const float* amax,
                               QuantOut out, const QuantOut* out_t, hipStream_t stream);

// Hadamard transform along tokens: amax of the transformed tensor, and the transposed encode.
hipError_t launch_rht_amax(const void* x, bool fp32, int64_t tokens, int64_t cols, int64_t ld,
                           uint16_t sign_mask, float* amax_out, hipStream_t stream);

hipError_t launch_rht_encode(const void* x, bool fp32, int64_t tokens, int64_t cols, int64_t ld,
                             uint16_t sign_mask, bool sr, uint64_t seed, uint64_t offset,
                             const float* amax, QuantOut out, hipStream_t stream);

struct GemmOperand {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global_scale;
};

hipError_t launch_gemm(GemmOperand a, GemmOperand b, int64_t M, int64_t N, int64_t K,
                       float* D, int64_t ldd, hipStream_t stream);

hipError_t launch_grouped_gemm(int64_t G, const int64_t* m_offsets, GemmOperand a, GemmOperand b,
                               int64_t total_m, int64_t N, int64_t K, float* D, int64_t ldd,
                               hipStream_t stream);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* gscale,
                             const int64_t* segments, int64_t nseg, int64_t rows, int64_t cols,
                             float* y, hipStream_t stream);

}  // namespace nvfp4
