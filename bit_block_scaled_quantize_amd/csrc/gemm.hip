// Block-scaled NVFP4 GEMM on gfx950 matrix cores: D[M,N] = sA*sB * sum_k a[m,k] b[n,k].
//
// The pages run the forward, activation-gradient and weight-gradient GEMMs of linear layers
// (artiverse.ca "NVIDIA's 4-bit floating point pushes AI training limits") and the expert
// GEMMs of MoE layers ("Nemotron NVFP4" explainer, "The model underneath") in NVFP4 with
// FP32 accumulation; Blackwell consumes the format natively, which is prior art here.
//
// gfx950 path: an E2M1 element times its E4M3 block scale has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in FP16. Each lane decodes 8 packed codes with one
// v_cvt_scalef32_pk_f16_fp4 per code byte (scale operand 2^8, exponent-only) and multiplies
// by the block scale held as FP16 bits (code << 7) = S * 2^-8, giving exactly e2m1 * S, then
// feeds v_mfma_f32_16x16x32_f16 (FP32 accumulate). The per-tensor scales multiply the
// accumulator in the epilogue. gfx950's native FP4 MFMA takes power-of-two scales per 32
// elements, which cannot express an E4M3 scale per 16 elements without leaving most of each
// instruction idle, so the FP16 path is the one used.
//
// Operand layout inside a 16x16x32 MFMA: lane l supplies row (l % 16) of A (column of B)
// and 8 K-values. Since the K order inside a dot product is free as long as A and B agree,
// each lane loads one contiguous 16-byte run (32 codes) of its row per 128-K step and feeds
// its 4 octets to 4 consecutive MFMAs; the 4 lane groups cover 4 different 32-element runs.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;             // 4 waves, 2 x 2
constexpr int kFragsM = 4;                // wave tile 64 x 64 = 4 x 4 MFMA tiles of 16 x 16
constexpr int kFragsN = 4;
constexpr int kWaveM = 16 * kFragsM;
constexpr int kWaveN = 16 * kFragsN;
constexpr int kBlockM = 2 * kWaveM;       // 128
constexpr int kBlockN = 2 * kWaveN;       // 128
constexpr int kStepK = 128;

// FP16 pair (S * 2^-8, S * 2^-8) from an E4M3 code: the code shifted into the FP16 exponent
// and mantissa fields reads as S * 2^-8 for every code, subnormal ones included.
__device__ __forceinline__ half2v scale_pair(uint32_t s) {
  const uint32_t b = (s << 7) | (s << 23);
  return __builtin_bit_cast(half2v, b);
}

__device__ __forceinline__ half8 decode8(uint32_t codes, half2v s2) {
  const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0) * s2;
  const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1) * s2;
  const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2) * s2;
  const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3) * s2;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

struct FragLoad { uint4 codes; uint32_t scales; };

// 32 codes of row `row` starting at element k (multiple of 32) and their two scale bytes;
// elements at or beyond K read as zero codes.
__device__ __forceinline__ FragLoad load_frag(const uint8_t* __restrict__ codes,
                                              const uint8_t* __restrict__ scales, int64_t row,
                                              int64_t K, int64_t k) {
  FragLoad f{make_uint4(0, 0, 0, 0), 0};
  const int64_t left = K - k;
  if (left <= 0) return f;
  const uint8_t* cp = codes + row * (K >> 1) + (k >> 1);
  const uint8_t* sp = scales + row * (K >> 4) + (k >> 4);
  if (left >= 32) {
    if ((K & 31) == 0) {
      f.codes = *reinterpret_cast<const uint4*>(cp);
    } else {
      const uint2 a = *reinterpret_cast<const uint2*>(cp);
      const uint2 b = *reinterpret_cast<const uint2*>(cp + 8);
      f.codes = make_uint4(a.x, a.y, b.x, b.y);
    }
    f.scales = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
  } else {                                  // exactly 16 elements remain (K % 16 == 0)
    const uint2 a = *reinterpret_cast<const uint2*>(cp);
    f.codes = make_uint4(a.x, a.y, 0, 0);
    f.scales = (uint32_t)sp[0];
  }
  return f;
}

__device__ __forceinline__ uint32_t word(const uint4& v, int t) {
  return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w;
}

// Tile (tm, tn) of a grid of tiles_m x tiles_n tiles for workgroup `bid`. Workgroups are
// dealt round-robin to the 8 XCDs, so consecutive ids are first regrouped per XCD; tiles are
// then walked in column-major bands of 8 tile-rows so neighbours share A and B panels in L2.
__device__ __forceinline__ void tile_of(int64_t bid, int64_t tiles_m, int64_t tiles_n,
                                        int64_t& tm, int64_t& tn) {
  const int64_t n = tiles_m * tiles_n;
  const int64_t per = (n + 7) / 8;
  const int64_t xcd = bid % 8, local = bid / 8;
  const int64_t tall = (n % 8) == 0 ? 8 : (n % 8);
  const int64_t id = xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
  constexpr int64_t kGroupM = 8;
  const int64_t band = kGroupM * tiles_n;
  const int64_t first_m = (id / band) * kGroupM;
  const int64_t gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int64_t in_band = id % band;
  tm = first_m + in_band % gm;
  tn = in_band / gm;
}

// One 128 x 128 output tile: rows [m0, m1) of A against rows [n0, n0 + 128) of B.
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
                                          const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs,
                                          int64_t m0, int64_t m1, int64_t n0, int64_t n1, int64_t K,
                                          float alpha, float* __restrict__ D, int64_t ldd) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t wm0 = m0 + (wave >> 1) * kWaveM;
  const int64_t wn0 = n0 + (wave & 1) * kWaveN;

  int64_t arow[kFragsM], brow[kFragsN];
#pragma unroll
  for (int i = 0; i < kFragsM; ++i) {
    const int64_t rr = wm0 + 16 * i + r;
    arow[i] = rr < m1 ? rr : m0;                 // clamp: rows past the end load row m0
  }
#pragma unroll
  for (int j = 0; j < kFragsN; ++j) {
    const int64_t rr = wn0 + 16 * j + r;
    brow[j] = rr < n1 ? rr : n0;
  }

  float4v acc[kFragsM][kFragsN];
#pragma unroll
  for (int i = 0; i < kFragsM; ++i)
#pragma unroll
    for (int j = 0; j < kFragsN; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

  FragLoad fa[kFragsM], fb[kFragsN];
  int64_t k = (int64_t)g * 32;
#pragma unroll
  for (int i = 0; i < kFragsM; ++i) fa[i] = load_frag(ac, as, arow[i], K, k);
#pragma unroll
  for (int j = 0; j < kFragsN; ++j) fb[j] = load_frag(bc, bs, brow[j], K, k);

  for (int64_t k0 = 0; k0 < K; k0 += kStepK) {
    FragLoad na[kFragsM], nb[kFragsN];
    const int64_t kn = k0 + kStepK + (int64_t)g * 32;
#pragma unroll
    for (int i = 0; i < kFragsM; ++i) na[i] = load_frag(ac, as, arow[i], K, kn);
#pragma unroll
    for (int j = 0; j < kFragsN; ++j) nb[j] = load_frag(bc, bs, brow[j], K, kn);

#pragma unroll
    for (int t = 0; t < 4; ++t) {
      half8 av[kFragsM], bv[kFragsN];
#pragma unroll
      for (int i = 0; i < kFragsM; ++i)
        av[i] = decode8(word(fa[i].codes, t), scale_pair((fa[i].scales >> (8 * (t >> 1))) & 0xFFu));
#pragma unroll
      for (int j = 0; j < kFragsN; ++j)
        bv[j] = decode8(word(fb[j].codes, t), scale_pair((fb[j].scales >> (8 * (t >> 1))) & 0xFFu));
#pragma unroll
      for (int i = 0; i < kFragsM; ++i)
#pragma unroll
        for (int j = 0; j < kFragsN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kFragsM; ++i) fa[i] = na[i];
#pragma unroll
    for (int j = 0; j < kFragsN; ++j) fb[j] = nb[j];
  }

  // D fragment layout: lane l holds rows 4*(l/16) + 0..3 of column l % 16.
#pragma unroll
  for (int i = 0; i < kFragsM; ++i) {
#pragma unroll
    for (int j = 0; j < kFragsN; ++j) {
      const int64_t col = wn0 + 16 * j + r;
      if (col >= n1) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = wm0 + 16 * i + 4 * g + q;
        if (row < m1) D[row * ldd + col] = acc[i][j][q] * alpha;
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_gemm(const uint8_t* __restrict__ ac,
                                                   const uint8_t* __restrict__ as,
                                                   const float* __restrict__ ag,
                                                   const uint8_t* __restrict__ bc,
                                                   const uint8_t* __restrict__ bs,
                                                   const float* __restrict__ bg, int64_t M,
                                                   int64_t N, int64_t K, float* __restrict__ D,
                                                   int64_t ldd) {
  const int64_t tiles_m = (M + kBlockM - 1) / kBlockM;
  const int64_t tiles_n = (N + kBlockN - 1) / kBlockN;
  int64_t tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * kBlockM, n0 = tn * kBlockN;
  const int64_t m1 = m0 + kBlockM < M ? m0 + kBlockM : M;
  const int64_t n1 = n0 + kBlockN < N ? n0 + kBlockN : N;
  const float alpha = ag[0] * bg[0];
  gemm_tile(ac, as, bc, bs, m0, m1, n0, n1, K, alpha, D, ldd);
}

// Grouped GEMM: workgroup slot s enumerates (m-tile of some group, n-tile); groups are found
// by walking the device offset table. Slots past the last tile exit at once.
__global__ __launch_bounds__(kThreads) void k_grouped_gemm(
    int64_t G, const int64_t* __restrict__ off, const uint8_t* __restrict__ ac,
    const uint8_t* __restrict__ as, const float* __restrict__ ag, const uint8_t* __restrict__ bc,
    const uint8_t* __restrict__ bs, const float* __restrict__ bg, int64_t total_m, int64_t N,
    int64_t K, float* __restrict__ D, int64_t ldd) {
  const int64_t tiles_n = (N + kBlockN - 1) / kBlockN;
  const int64_t slot_m = blockIdx.x / tiles_n;
  const int64_t tn = blockIdx.x - slot_m * tiles_n;
  int64_t base = 0, g = -1, m0 = 0, m1 = 0;
  int64_t prev = off[0] < 0 ? 0 : off[0];
  for (int64_t q = 0; q < G; ++q) {
    int64_t hi = off[q + 1];
    hi = hi < prev ? prev : (hi > total_m ? total_m : hi);   // clamp a malformed table
    const int64_t t = (hi - prev + kBlockM - 1) / kBlockM;
    if (slot_m < base + t) {
      g = q;
      m0 = prev + (slot_m - base) * kBlockM;
      m1 = m0 + kBlockM < hi ? m0 + kBlockM : hi;
      break;
    }
    base += t;
    prev = hi;
  }
  if (g < 0) return;
  const int64_t n0 = tn * kBlockN;
  const int64_t n1 = n0 + kBlockN < N ? n0 + kBlockN : N;
  const float alpha = ag[g] * bg[g];
  gemm_tile(ac, as, bc + g * N * (K >> 1), bs + g * N * (K >> 4), m0, m1, n0, n1, K, alpha, D,
            ldd);
}

}  // namespace

hipError_t launch_gemm(GemmOperand a, GemmOperand b, int64_t M, int64_t N, int64_t K, float* D,
                       int64_t ldd, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles = ((M + kBlockM - 1) / kBlockM) * ((N + kBlockN - 1) / kBlockN);
  hipLaunchKernelGGL(k_gemm, dim3((unsigned)tiles), dim3(kThreads), 0, stream, a.codes, a.scales,
                     a.global_scale, b.codes, b.scales, b.global_scale, M, N, K, D, ldd);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(int64_t G, const int64_t* m_offsets, GemmOperand a, GemmOperand b,
                               int64_t total_m, int64_t N, int64_t K, float* D, int64_t ldd,
                               hipStream_t stream) {
  if (total_m == 0 || N == 0) return hipSuccess;
  const int64_t tiles_n = (N + kBlockN - 1) / kBlockN;
  const int64_t slots_m = total_m / kBlockM + G;          // >= sum_g ceil(M_g / 128)
  hipLaunchKernelGGL(k_grouped_gemm, dim3((unsigned)(slots_m * tiles_n)), dim3(kThreads), 0,
                     stream, G, m_offsets, a.codes, a.scales, a.global_scale, b.codes, b.scales,
                     b.global_scale, total_m, N, K, D, ldd);
  return hipGetLastError();
}

}  // namespace nvfp4
