// NVFP4 block quantization kernels for gfx950: tensor amax, 1x16 encode (nearest or
// stochastic rounding) and 16x16 encode with optional transposed emission.
//
// Format and recipe: "Nemotron NVFP4" explainer, "What NVFP4 actually is" (E2M1 elements,
// one E4M3 scale per 16 elements, one FP32 tensor scale) and "Why 4-bit training normally
// falls apart - and the three fixes" (2D weight blocks, stochastic rounding of gradients);
// artiverse.ca "NVIDIA's 4-bit floating point pushes AI training limits" (16x16 weight
// blocks instead of 1x16, stochastic rounding on gradients only).
//
// All kernels are HBM-streaming: one wave owns whole rows (or a 16-row strip for 16x16
// tiles), every lane loads 16-byte vectors so that a wave-wide load covers a contiguous
// span of a row, and results are written as packed nibble words plus one scale byte per
// block. The encode pass walks the tensor in the reverse order of the amax pass so that
// its first reads hit the lines the amax pass touched last (still in the 256 MB
// Infinity Cache for tensors of that order of size).
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;

// 16 consecutive inputs starting at p (16-byte aligned) as floats.
template <typename TIn>
__device__ __forceinline__ void load16(const TIn* p, float (&v)[16]);

template <>
__device__ __forceinline__ void load16<uint16_t>(const uint16_t* p, float (&v)[16]) {
  const v4u32 a = ld_u32x4(p);
  const v4u32 b = ld_u32x4(p + 8);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}

template <>
__device__ __forceinline__ void load16<float>(const float* p, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v4f32 a = ld_f32x4(p + 4 * i);
    v[4 * i] = a.x;
    v[4 * i + 1] = a.y;
    v[4 * i + 2] = a.z;
    v[4 * i + 3] = a.w;
  }
}

__device__ __forceinline__ float abs_max16(const float (&v)[16]) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(v[j]));
  return m;
}

// ---------------------------------------------------------------------------------------
// amax: each wave owns rows r = wave, wave + nwaves, ...; lanes stride over 16-element
// groups of the row. Per-segment maxima are flushed with one atomic per (wave, segment run).
template <typename TIn, bool SEG>
__global__ __launch_bounds__(kThreads) void k_amax(const TIn* __restrict__ x, int64_t rows,
                                                   int64_t cols, int64_t ld,
                                                   const int64_t* __restrict__ seg, int64_t nseg,
                                                   float* __restrict__ amax_out) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t groups = cols >> 4;
  // contiguous row range per wave keeps segment runs long
  const int64_t per = (rows + nwaves - 1) / nwaves;
  const int64_t r0 = wave * per;
  const int64_t r1 = r0 + per < rows ? r0 + per : rows;
  float m = 0.0f;
  int64_t cur = -1;
  for (int64_t r = r0; r < r1; ++r) {
    if constexpr (SEG) {
      const int64_t s = find_segment(seg, nseg, r);
      if (s != cur) {
        if (cur >= 0) {
          const float wm = wave_max(m);
          if (lane == 0) atomic_max_nonneg(amax_out + cur, wm);
        }
        cur = s;
        m = 0.0f;
      }
    }
    const TIn* xr = x + r * ld;
    int64_t gidx = lane;
    for (; gidx + 64 < groups; gidx += 128) {
      float v[16], u[16];
      load16<TIn>(xr + gidx * 16, v);
      load16<TIn>(xr + (gidx + 64) * 16, u);
      m = fmaxf(m, fmaxf(abs_max16(v), abs_max16(u)));
    }
    if (gidx < groups) {
      float v[16];
      load16<TIn>(xr + gidx * 16, v);
      m = fmaxf(m, abs_max16(v));
    }
  }
  const float wm = wave_max(m);
  if (lane == 0 && r0 < r1) atomic_max_nonneg(amax_out + (SEG ? (cur < 0 ? 0 : cur) : 0), wm);
}

__global__ void k_fill_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

// ---------------------------------------------------------------------------------------
// 1x16 encode: lane = one 16-element block; wave = up to 64 consecutive blocks of a row.
template <typename TIn, bool SR, bool SEG>
__global__ __launch_bounds__(kThreads) void k_encode_1x16(
    const TIn* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ amax, const int64_t* __restrict__ seg, int64_t nseg,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gscale,
    uint64_t seed, uint64_t offset) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t nb = cols >> 4;
  if (blockIdx.x == 0)
    for (int64_t i = threadIdx.x; i < nseg; i += kThreads) gscale[i] = tensor_decode_scale(amax[i]);

  float s_enc = tensor_encode_scale(amax[0]);
  int64_t cur = 0;
  for (int64_t it = wave; it < rows; it += nwaves) {
    const int64_t r = rows - 1 - it;                 // reverse of the amax pass
    if constexpr (SEG) {
      const int64_t s = find_segment(seg, nseg, r);
      if (s != cur) {
        cur = s;
        s_enc = tensor_encode_scale(amax[s]);
      }
    }
    const TIn* xr = x + r * ld;
    uint2* cr = reinterpret_cast<uint2*>(codes + r * (cols >> 1));
    uint8_t* sr = scales + r * nb;
    for (int64_t b = lane; b < nb; b += 64) {
      float v[16];
      load16<TIn>(xr + b * 16, v);
      const BlockScale bs = block_scale(abs_max16(v), s_enc);
      u32x4 rnd{0, 0, 0, 0};
      if constexpr (SR) rnd = block_random((uint64_t)(r * nb + b), seed, offset);
      uint32_t lo, hi;
      encode16<SR>(v, bs.mult, rnd, lo, hi);
      cr[b] = make_uint2(lo, hi);
      sr[b] = (uint8_t)bs.code;
    }
  }
}

// ---------------------------------------------------------------------------------------
// 16x16 encode: a lane pair owns one 16x16 tile (each lane 16 rows x 8 columns); a wave
// covers 32 tiles (512 columns) of one 16-row strip. The tile amax is combined across the
// pair with one cross-lane max.
template <typename TIn>
__device__ __forceinline__ void load8(const TIn* p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const v4u32 a = ld_u32x4(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const v4f32 a = ld_f32x4(p);
  const v4f32 b = ld_f32x4(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename TIn, bool SEG, bool TRANS>
__global__ __launch_bounds__(kThreads) void k_encode_16x16(
    const TIn* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ amax, const int64_t* __restrict__ seg, int64_t nseg,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gscale,
    uint8_t* __restrict__ tcodes, uint8_t* __restrict__ tscales, float* __restrict__ tgscale) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t strips = rows >> 4;
  const int64_t half_tiles = cols >> 3;                 // 8-column pieces per row
  const int64_t chunks = (half_tiles + 63) >> 6;
  const int64_t tasks = strips * chunks;
  const int64_t nb = cols >> 4;
  if (blockIdx.x == 0) {
    for (int64_t i = threadIdx.x; i < nseg; i += kThreads) {
      const float d = tensor_decode_scale(amax[i]);
      gscale[i] = d;
      if constexpr (TRANS) tgscale[i] = d;
    }
  }
  float s_enc = tensor_encode_scale(amax[0]);
  int64_t cur = 0;
  for (int64_t it = wave; it < tasks; it += nwaves) {
    const int64_t task = tasks - 1 - it;
    const int64_t strip = task / chunks;
    const int64_t ht = (task - strip * chunks) * 64 + lane;   // this lane's 8-column piece
    const int64_t r0 = strip << 4;
    if constexpr (SEG) {
      const int64_t s = find_segment(seg, nseg, r0);
      if (s != cur) {
        cur = s;
        s_enc = tensor_encode_scale(amax[s]);
      }
    }
    const bool active = ht < half_tiles;
    const int64_t c0 = (active ? ht : 0) << 3;
    float v[16][8];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      load8<TIn>(x + (r0 + j) * ld + c0, v[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j][i]));
    }
    m = fmaxf(m, __shfl_xor(m, 1, 64));                 // partner lane holds the other half
    const BlockScale bs = block_scale(m, s_enc);
    uint32_t w[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      uint32_t c = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) c |= e2m1_rn(v[j][i] * bs.mult) << (4 * i);
      w[j] = c;
    }
    if (active) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        *reinterpret_cast<uint32_t*>(codes + (r0 + j) * (cols >> 1) + (c0 >> 1)) = w[j];
        if ((ht & 1) == 0) scales[(r0 + j) * nb + (c0 >> 4)] = (uint8_t)bs.code;
      }
      if constexpr (TRANS) {
        // x^T row (c0 + i) gets the 16 codes of column i, rows r0..r0+15 along its row.
        const int64_t tnb = rows >> 4;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t lo = 0, hi = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            lo |= ((w[j] >> (4 * i)) & 0xFu) << (4 * j);
            hi |= ((w[j + 8] >> (4 * i)) & 0xFu) << (4 * j);
          }
          const int64_t tr = c0 + i;
          *reinterpret_cast<uint2*>(tcodes + tr * (rows >> 1) + (r0 >> 1)) = make_uint2(lo, hi);
          tscales[tr * tnb + (r0 >> 4)] = (uint8_t)bs.code;
        }
      }
    }
  }
}

__global__ void k_dequantize(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                             const float* __restrict__ gscale, const int64_t* __restrict__ seg,
                             int64_t nseg, int64_t rows, int64_t cols, float* __restrict__ y) {
  const int64_t words = rows * (cols >> 3);            // 8 codes per 32-bit word
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < words;
       w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = w / (cols >> 3);
    const int64_t c = (w - r * (cols >> 3)) << 3;
    const int64_t s = seg ? find_segment(seg, nseg, r) : 0;
    const float gs = gscale[s];
    const float bs = e4m3_decode(scales[r * (cols >> 4) + (c >> 4)]);
    const uint32_t q = *reinterpret_cast<const uint32_t*>(codes + r * (cols >> 1) + (c >> 1));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t code = (q >> (4 * i)) & 0xFu;
      const uint32_t mag = code & 7u;
      const float e = mag < 2 ? 0.5f * (float)mag
                              : __uint_as_float(((126u + (mag >> 1)) << 23) | ((mag & 1u) << 22));
      const float v = (e * bs) * gs;                   // e * bs is exact in FP32
      y[r * cols + c + i] = (code & 8u) ? -v : v;
    }
  }
}

int grid_for(int64_t work_items, int64_t items_per_block, int64_t cap) {
  int64_t g = (work_items + items_per_block - 1) / items_per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

constexpr int64_t kMaxBlocks = 256 * 16;   // 16 workgroups per CU is plenty for streaming

}  // namespace

hipError_t launch_amax(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                       const int64_t* segments, int64_t nseg, float* amax_out,
                       hipStream_t stream) {
  hipLaunchKernelGGL(k_fill_zero, dim3(1), dim3(256), 0, stream, amax_out, nseg);
  const int grid = grid_for(rows, kWavesPerBlock, kMaxBlocks);
  if (fp32) {
    if (segments)
      hipLaunchKernelGGL((k_amax<float, true>), dim3(grid), dim3(kThreads), 0, stream,
                         (const float*)x, rows, cols, ld, segments, nseg, amax_out);
    else
      hipLaunchKernelGGL((k_amax<float, false>), dim3(grid), dim3(kThreads), 0, stream,
                         (const float*)x, rows, cols, ld, segments, nseg, amax_out);
  } else {
    if (segments)
      hipLaunchKernelGGL((k_amax<uint16_t, true>), dim3(grid), dim3(kThreads), 0, stream,
                         (const uint16_t*)x, rows, cols, ld, segments, nseg, amax_out);
    else
      hipLaunchKernelGGL((k_amax<uint16_t, false>), dim3(grid), dim3(kThreads), 0, stream,
                         (const uint16_t*)x, rows, cols, ld, segments, nseg, amax_out);
  }
  return hipGetLastError();
}

template <typename TIn, bool SR, bool SEG>
static void encode_1x16_t(const void* x, int64_t rows, int64_t cols, int64_t ld, uint64_t seed,
                          uint64_t offset, const int64_t* segments, int64_t nseg,
                          const float* amax, QuantOut out, hipStream_t stream) {
  const int grid = grid_for(rows, kWavesPerBlock, kMaxBlocks);
  hipLaunchKernelGGL((k_encode_1x16<TIn, SR, SEG>), dim3(grid), dim3(kThreads), 0, stream,
                     (const TIn*)x, rows, cols, ld, amax, segments, nseg, out.codes, out.scales,
                     out.global_scale, seed, offset);
}

hipError_t launch_encode_1x16(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                              bool sr, uint64_t seed, uint64_t offset,
                              const int64_t* segments, int64_t nseg, const float* amax,
                              QuantOut out, hipStream_t stream) {
  const bool seg = segments != nullptr;
#define NVFP4_E1(T, S, G) encode_1x16_t<T, S, G>(x, rows, cols, ld, seed, offset, segments, nseg, amax, out, stream)
  if (fp32) {
    if (sr) { if (seg) NVFP4_E1(float, true, true); else NVFP4_E1(float, true, false); }
    else    { if (seg) NVFP4_E1(float, false, true); else NVFP4_E1(float, false, false); }
  } else {
    if (sr) { if (seg) NVFP4_E1(uint16_t, true, true); else NVFP4_E1(uint16_t, true, false); }
    else    { if (seg) NVFP4_E1(uint16_t, false, true); else NVFP4_E1(uint16_t, false, false); }
  }
#undef NVFP4_E1
  return hipGetLastError();
}

template <typename TIn, bool SEG, bool TRANS>
static void encode_16x16_t(const void* x, int64_t rows, int64_t cols, int64_t ld,
                           const int64_t* segments, int64_t nseg, const float* amax,
                           QuantOut out, const QuantOut* out_t, hipStream_t stream) {
  const int64_t tasks = (rows >> 4) * (((cols >> 3) + 63) >> 6);
  const int grid = grid_for(tasks, kWavesPerBlock, kMaxBlocks);
  hipLaunchKernelGGL((k_encode_16x16<TIn, SEG, TRANS>), dim3(grid), dim3(kThreads), 0, stream,
                     (const TIn*)x, rows, cols, ld, amax, segments, nseg, out.codes, out.scales,
                     out.global_scale, TRANS ? out_t->codes : nullptr,
                     TRANS ? out_t->scales : nullptr, TRANS ? out_t->global_scale : nullptr);
}

hipError_t launch_encode_16x16(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                               const int64_t* segments, int64_t nseg, const float* amax,
                               QuantOut out, const QuantOut* out_t, hipStream_t stream) {
  const bool seg = segments != nullptr;
  const bool tr = out_t != nullptr;
#define NVFP4_E2(T, G, R) encode_16x16_t<T, G, R>(x, rows, cols, ld, segments, nseg, amax, out, out_t, stream)
  if (fp32) {
    if (seg) { if (tr) NVFP4_E2(float, true, true); else NVFP4_E2(float, true, false); }
    else     { if (tr) NVFP4_E2(float, false, true); else NVFP4_E2(float, false, false); }
  } else {
    if (seg) { if (tr) NVFP4_E2(uint16_t, true, true); else NVFP4_E2(uint16_t, true, false); }
    else     { if (tr) NVFP4_E2(uint16_t, false, true); else NVFP4_E2(uint16_t, false, false); }
  }
#undef NVFP4_E2
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* gscale,
                             const int64_t* segments, int64_t nseg, int64_t rows, int64_t cols,
                             float* y, hipStream_t stream) {
  const int grid = grid_for(rows * (cols >> 3), 256, kMaxBlocks);
  hipLaunchKernelGGL(k_dequantize, dim3(grid), dim3(256), 0, stream, codes, scales, gscale,
                     segments, nseg, rows, cols, y);
  return hipGetLastError();
}

}  // namespace nvfp4
