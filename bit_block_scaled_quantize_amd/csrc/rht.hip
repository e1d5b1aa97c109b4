// Random Hadamard transform + transposed 1x16 quantization of the weight-gradient operands.
//
// "Nemotron NVFP4" explainer, "Why 4-bit training normally falls apart - and the three
// fixes": the wgrad GEMM's inputs are multiplied by a random Hadamard matrix before
// quantization, which spreads an outlier over its block, and the rotation cancels inside the
// GEMM. The rotation acts along the contraction (token) dimension in blocks of 16 tokens:
// for column c and token block t, y = 1/4 * H16 * diag(s) * x[16t..16t+15, c], with
// H16[i][j] = (-1)^popcount(i & j) and signs s from a 16-bit mask. The butterfly runs in
// binary64 (stages h = 1, 2, 4, 8), so for BF16 inputs every step is exact, and the result is
// rounded once to FP32. The 16 outputs of one (column, token block) are exactly one 1x16
// quantization block of the transposed output [cols, tokens].
//
// Layout: a lane owns two adjacent columns and walks a run of token blocks, so each 16-token
// load is one 4-byte (BF16 pair) or 8-byte (FP32 pair) vector per lane and a wave-wide load
// covers 128 contiguous columns of one token row.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kColsPerLane = 2;
constexpr int kColsPerBlock = kThreads * kColsPerLane;
constexpr int kTokenBlocksPerTask = 8;

// Columns c and c+1 of one token row. `both` says whether c+1 exists; `paired` whether the
// pair is aligned for one vector load (even row stride), else two scalar loads are used.
template <typename TIn>
__device__ __forceinline__ void load_pair(const TIn* p, bool both, bool paired, float& a, float& b);

template <>
__device__ __forceinline__ void load_pair<uint16_t>(const uint16_t* p, bool both, bool paired,
                                                    float& a, float& b) {
  if (both && paired) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    a = bf16_lo(w);
    b = bf16_hi(w);
  } else {
    a = __uint_as_float((uint32_t)p[0] << 16);
    b = both ? __uint_as_float((uint32_t)p[1] << 16) : 0.0f;
  }
}

template <>
__device__ __forceinline__ void load_pair<float>(const float* p, bool both, bool paired, float& a,
                                                 float& b) {
  if (both && paired) {
    const v2f32 w = *reinterpret_cast<const v2f32*>(p);
    a = w.x;
    b = w.y;
  } else {
    a = p[0];
    b = both ? p[1] : 0.0f;
  }
}

// y[i] = rn32(0.25 * sum_j H[i][j] * s_j * v[j]) via the binary64 butterfly.
__device__ __forceinline__ void rht16(const float (&v)[16], uint32_t mask, float (&y)[16]) {
  double u[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const double d = (double)v[j];
    u[j] = ((mask >> j) & 1u) ? -d : d;
  }
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if ((j & h) == 0) {
        const double a = u[j], b = u[j + h];
        u[j] = a + b;
        u[j + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = (float)(u[i] * 0.25);
}

template <typename TIn, bool ENCODE, bool SR>
__global__ __launch_bounds__(kThreads) void k_rht(
    const TIn* __restrict__ x, int64_t tokens, int64_t cols, int64_t ld, uint32_t mask,
    const float* __restrict__ amax, float* __restrict__ amax_out, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ gscale, uint64_t seed, uint64_t offset) {
  const int64_t c = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kColsPerLane;
  const int64_t nbt = tokens >> 4;                          // token blocks = output blocks per row
  const int64_t tb0 = (int64_t)blockIdx.y * kTokenBlocksPerTask;
  const int64_t tb1 = tb0 + kTokenBlocksPerTask < nbt ? tb0 + kTokenBlocksPerTask : nbt;
  const bool valid0 = c < cols;
  const bool valid1 = c + 1 < cols;
  const int64_t cl = valid0 ? c : 0;                         // clamped column for loads
  const bool paired = (ld & 1) == 0;

  float s_enc = 1.0f;
  if constexpr (ENCODE) {
    s_enc = tensor_encode_scale(amax[0]);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) gscale[0] = tensor_decode_scale(amax[0]);
  }
  float m = 0.0f;
  for (int64_t tb = tb0; tb < tb1; ++tb) {
    float v0[16], v1[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      load_pair<TIn>(x + (tb * 16 + j) * ld + cl, valid1, paired, v0[j], v1[j]);
#pragma unroll
    for (int k = 0; k < kColsPerLane; ++k) {
      const bool valid = k == 0 ? valid0 : valid1;
      float y[16];
      rht16(k == 0 ? v0 : v1, mask, y);
      float bm = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) bm = fmaxf(bm, fabsf(y[i]));
      if constexpr (!ENCODE) {
        if (valid) m = fmaxf(m, bm);
      } else {
        if (valid) {
          const int64_t row = c + k;                          // output row = input column
          const BlockScale bs = block_scale(bm, s_enc);
          u32x4 rnd{0, 0, 0, 0};
          if constexpr (SR) rnd = block_random((uint64_t)(row * nbt + tb), seed, offset);
          uint32_t lo, hi;
          encode16<SR>(y, bs.mult, rnd, lo, hi);
          *reinterpret_cast<uint2*>(codes + row * (tokens >> 1) + tb * 8) = make_uint2(lo, hi);
          scales[row * nbt + tb] = (uint8_t)bs.code;
        }
      }
    }
  }
  if constexpr (!ENCODE) {
    const float wm = wave_max(m);
    if ((threadIdx.x & 63) == 0) atomic_max_nonneg(amax_out, wm);
  }
}

__global__ void k_zero1(float* p) { *p = 0.0f; }

template <typename TIn, bool ENCODE, bool SR>
void launch_rht_t(const void* x, int64_t tokens, int64_t cols, int64_t ld, uint16_t mask,
                  const float* amax, float* amax_out, QuantOut out, uint64_t seed,
                  uint64_t offset, hipStream_t stream) {
  if (tokens == 0 || cols == 0) return;
  const dim3 grid((unsigned)((cols + kColsPerBlock - 1) / kColsPerBlock),
                  (unsigned)(((tokens >> 4) + kTokenBlocksPerTask - 1) / kTokenBlocksPerTask));
  hipLaunchKernelGGL((k_rht<TIn, ENCODE, SR>), grid, dim3(kThreads), 0, stream, (const TIn*)x,
                     tokens, cols, ld, (uint32_t)mask, amax, amax_out, out.codes, out.scales,
                     out.global_scale, seed, offset);
}

}  // namespace

hipError_t launch_rht_amax(const void* x, bool fp32, int64_t tokens, int64_t cols, int64_t ld,
                           uint16_t sign_mask, float* amax_out, hipStream_t stream) {
  hipLaunchKernelGGL(k_zero1, dim3(1), dim3(1), 0, stream, amax_out);
  const QuantOut none{nullptr, nullptr, nullptr};
  if (fp32)
    launch_rht_t<float, false, false>(x, tokens, cols, ld, sign_mask, nullptr, amax_out, none, 0, 0, stream);
  else
    launch_rht_t<uint16_t, false, false>(x, tokens, cols, ld, sign_mask, nullptr, amax_out, none, 0, 0, stream);
  return hipGetLastError();
}

hipError_t launch_rht_encode(const void* x, bool fp32, int64_t tokens, int64_t cols, int64_t ld,
                             uint16_t sign_mask, bool sr, uint64_t seed, uint64_t offset,
                             const float* amax, QuantOut out, hipStream_t stream) {
  if (fp32) {
    if (sr) launch_rht_t<float, true, true>(x, tokens, cols, ld, sign_mask, amax, nullptr, out, seed, offset, stream);
    else    launch_rht_t<float, true, false>(x, tokens, cols, ld, sign_mask, amax, nullptr, out, seed, offset, stream);
  } else {
    if (sr) launch_rht_t<uint16_t, true, true>(x, tokens, cols, ld, sign_mask, amax, nullptr, out, seed, offset, stream);
    else    launch_rht_t<uint16_t, true, false>(x, tokens, cols, ld, sign_mask, amax, nullptr, out, seed, offset, stream);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
