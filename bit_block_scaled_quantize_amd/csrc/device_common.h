// Device-side building blocks shared by the quantize, Hadamard and GEMM kernels (gfx950).
//
// Element format ("Nemotron NVFP4" explainer, "What NVFP4 actually is"): E2M1 elements, one
// E4M3 scale per 16 elements, one FP32 tensor scale. The bit-level conventions (E2M1 bias 1,
// OCP E4M3 "FN", nearest-even rounding, the 8-bit stochastic-rounding rule, the
// Philox4x32-10 counter layout) are the ones documented in include/nvfp4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rht_exact.h"

#pragma clang fp contract(off)

namespace nvfp4 {

constexpr float kScaleNumerator = 2688.0f;   // largest element (6) x largest E4M3 (448)
constexpr float kFltMax = 3.40282346638528859812e+38f;

// ---- vector loads -------------------------------------------------------------------------
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));
typedef float v4f32 __attribute__((ext_vector_type(4)));
typedef float v2f32 __attribute__((ext_vector_type(2)));

template <typename T>
__device__ __forceinline__ v4u32 ld_u32x4(const T* p) { return *reinterpret_cast<const v4u32*>(p); }
template <typename T>
__device__ __forceinline__ v4f32 ld_f32x4(const T* p) { return *reinterpret_cast<const v4f32*>(p); }

// ---- BF16 / FP32 inputs --------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---- tensor scales ---------------------------------------------------------------------
// Encode multiplier s_enc = rn32(2688 / amax) (FLT_MAX if that overflows), 1 for amax == 0.
__device__ __forceinline__ float tensor_encode_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  return fminf(kScaleNumerator / amax, kFltMax);
}
// Stored decode scale s_dec = rn32(amax / 2688), 1 for amax == 0.
__device__ __forceinline__ float tensor_decode_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  return amax / kScaleNumerator;
}

// ---- E4M3 block scale ------------------------------------------------------------------
// Nearest-even E4M3 code of a non-negative value, saturating at 448 (code 0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
  if (!(t < 448.0f)) return 0x7Eu;
  if (t < 0.015625f) {                           // below 2^-6: subnormal steps of 2^-9
    return (uint32_t)__builtin_rintf(t * 512.0f);  // exact scaling, ties to even; 8 -> 0x08
  }
  const uint32_t b = __float_as_uint(t);
  // keep 3 mantissa bits with round-half-even, then rebias the exponent 127 -> 7
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  return (r >> 20) - (120u << 3);
}

// Exact value of a non-negative E4M3 code (0x00..0x7E).
__device__ __forceinline__ float e4m3_decode(uint32_t s) {
  const uint32_t e = s >> 3, m = s & 7u;
  const float sub = (float)m * 0.001953125f;     // m * 2^-9
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}

// ---- E2M1 elements ---------------------------------------------------------------------
// gfx950 converts FP32 to E2M1 in hardware. With its scale operand at 1 the pair conversion
// rounds to nearest even and saturates at 6, with the sign taken from the input (zero included):
// exactly the element rounding fixed above, so the element multiply rn32(x * r_b) is done in
// FP32 first and the result is handed to the converter. The pair (y0, y1) lands in byte `sel`
// of the result, y0 in the low nibble; the other bytes keep `old`.
template <int sel>
__device__ __forceinline__ uint32_t e2m1_rn_pair(uint32_t old, float y0, float y1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y0, y1, 1.0f, sel);
}

// Eight codes (y[0] in the low nibble) rounded to nearest even.
__device__ __forceinline__ uint32_t e2m1_rn8(const float* y) {
  uint32_t w = e2m1_rn_pair<0>(0u, y[0], y[1]);
  w = e2m1_rn_pair<1>(w, y[2], y[3]);
  w = e2m1_rn_pair<2>(w, y[4], y[5]);
  return e2m1_rn_pair<3>(w, y[6], y[7]);
}

// Stochastic rounding with the random byte r of the element: round up iff frac + r/256 >= 1.
// The hardware stochastic converter adds part of its seed operand to the FP32 mantissa, aligned
// just below the kept E2M1 bit (in fixed point for the subnormal range), and truncates: bits
// 31..10 of the seed for the first value of the pair, bits 30..9 for the second. A seed holding
// r in bits 31..24 (first value) or 30..23 (second value) with zeros below therefore is the
// 8-bit rule above. One seed cannot serve both values with independent bytes, so each pair is
// converted twice, once per seed, and each conversion contributes the nibble whose seed fits.
template <int byte0, int byte1>
__device__ __forceinline__ uint32_t e2m1_sr_pair(float y0, float y1, uint32_t word) {
  // byte k of word moved to bits 31..24 (zeros below) by a byte permute
  const uint32_t s0 = __builtin_amdgcn_perm(0u, word, 0x000C0C0Cu | ((uint32_t)byte0 << 24));
  const uint32_t s1 = __builtin_amdgcn_perm(0u, word, 0x000C0C0Cu | ((uint32_t)byte1 << 24)) >> 1;
  const uint32_t c0 = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, v2f32{y0, y1}, s0, 1.0f, 0);
  const uint32_t c1 = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, v2f32{y0, y1}, s1, 1.0f, 0);
  return __builtin_amdgcn_ubfe(c0, 0, 4) | (c1 & 0xF0u);   // bits 8..31 of c0, c1 undefined
}

// Eight stochastically rounded codes; element i takes byte i%4 of words w0 (i < 4), w1.
__device__ __forceinline__ uint32_t e2m1_sr8(const float* y, uint32_t w0, uint32_t w1) {
  const uint32_t p0 = e2m1_sr_pair<0, 1>(y[0], y[1], w0);
  const uint32_t p1 = e2m1_sr_pair<2, 3>(y[2], y[3], w0);
  const uint32_t p2 = e2m1_sr_pair<0, 1>(y[4], y[5], w1);
  const uint32_t p3 = e2m1_sr_pair<2, 3>(y[6], y[7], w1);
  return p0 | (p1 << 8) | (p2 << 16) | (p3 << 24);
}

// ---- Philox4x32-10 (Salmon et al., SC'11) ----------------------------------------------
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = u32x4{(uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1,
              (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// The 16 random bytes of quantization block `b`.
__device__ __forceinline__ u32x4 block_random(uint64_t b, uint64_t seed, uint64_t offset) {
  return philox4x32_10(u32x4{(uint32_t)b, (uint32_t)(b >> 32), (uint32_t)offset,
                             (uint32_t)(offset >> 32)},
                       (uint32_t)seed, (uint32_t)(seed >> 32));
}

// ---- one 16-element block ----------------------------------------------------------------
// Block scale code and element multiplier from the block amax and the tensor encode scale:
// t = rn32(rn32(a_b / 6) * s_enc), S = E4M3(t), r = min(rn32(s_enc / dec(S)), FLT_MAX),
// r = 0 when S decodes to zero (every element then encodes as a signed zero).
struct BlockScale { uint32_t code; float mult; };

// rn32(a / 6) for a >= 0. From 2^-125 up, the product with rn32(1/6) corrected by one fused
// remainder step (Markstein's division method, "IA-64 and Elementary Functions", 2000) is the
// correctly rounded quotient; an exhaustive device check against the IEEE division over every
// non-negative binary32 found mismatches only below 2^-125 (subnormal quotients), which take
// the IEEE division.
__device__ __forceinline__ float div6(float a) {
  constexpr float kSixth = 1.0f / 6.0f;
  const float q0 = a * kSixth;
  const float r = __builtin_fmaf(-q0, 6.0f, a);
  float q = __builtin_fmaf(r, kSixth, q0);
  if (a < 0x1p-125f) q = a / 6.0f;
  return q;
}

// Element multiplier of a block with scale code s: min(rn32(s_enc / dec(s)), FLT_MAX), 0 for a
// zero scale.
__device__ __forceinline__ float block_recip(uint32_t s, float s_enc) {
  const float d = e4m3_decode(s);
  return d > 0.0f ? fminf(s_enc / d, kFltMax) : 0.0f;
}

__device__ __forceinline__ BlockScale block_scale(float block_amax, float s_enc) {
  const uint32_t s = e4m3_encode(div6(block_amax) * s_enc);
  return BlockScale{s, block_recip(s, s_enc)};
}

// The same with the multipliers of all 127 scale codes precomputed for one tensor scale
// (build_recip_table: once per workgroup, then a barrier), so a block costs a table read
// instead of a division.
__device__ __forceinline__ void build_recip_table(float s_enc, float* table) {
  for (uint32_t c = threadIdx.x; c < 128u; c += blockDim.x) table[c] = block_recip(c, s_enc);
}

__device__ __forceinline__ BlockScale block_scale_table(float block_amax, float s_enc,
                                                        const float* table) {
  const uint32_t s = e4m3_encode(div6(block_amax) * s_enc);   // <= 0x7E
  return BlockScale{s, table[s]};
}

// Encode 16 values v[0..15] (already in float) into two code words (element j -> nibble j).
template <bool SR>
__device__ __forceinline__ void encode16(const float (&v)[16], float mult, u32x4 rnd,
                                         uint32_t& lo, uint32_t& hi) {
  float y[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) y[j] = v[j] * mult;
  if constexpr (SR) {
    lo = e2m1_sr8(y, rnd.x, rnd.y);
    hi = e2m1_sr8(y + 8, rnd.z, rnd.w);
  } else {
    lo = e2m1_rn8(y);
    hi = e2m1_rn8(y + 8);
  }
}

// ---- reductions ----------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// atomic max of a non-negative float through its bit pattern (monotone for v >= 0)
__device__ __forceinline__ void atomic_max_nonneg(float* p, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(p), __float_as_uint(v));
}

// The 16-point random-sign Hadamard transform of one block ("Nemotron NVFP4" explainer, "Why
// 4-bit training normally falls apart - and the three fixes"); the Hadamard kernels apply it
// along tokens, the rowwise quantization along each row.
// y[i] = rn32(1/4 * sum_j H[i][j] * s_j * v[j]), the exact value rounded once (+0 for an exact
// zero), in two steps:
//  * rht16_f64: the butterfly in binary64 on the terms fma(v_j, +-1/4, +0) (exact, and -0
//    becomes +0, so no step yields -0 and a zero output is +0), rounded once at the end, plus
//    a range test that proves every step exact;
//  * rht16_exact, for the blocks the test rejects (values spread over very many binades):
//    exact integer sums (exact_quarter_sum_at), one output at a time.
// Range test: every partial sum of the butterfly is a +- sum of a subset of the terms u_j, so it
// is at most sum |u_j| in magnitude and a multiple of the smallest nonzero term's last-bit
// weight 2^q; all are binary64 numbers when sum |u_j| < 2^(q + 53). Since v = 1/4 D H y, each
// |v_j| <= 4 max|y| and sum |u_j| <= 16 max|y|, so max|y| < 2^(q + 49) suffices. With the
// smallest nonzero exponent field f (1 for subnormals), q = f - 136 for BF16 inputs (8
// significant bits) and f - 152 for FP32 ones, so the test is max|y| < 2^(f - 87) or 2^(f - 103).
// max|y| is the maximum of the binary64 results rounded to binary32, within a relative
// 2^-40 of the exact one even when a step rounded; the factor 1 - 2^-16 on the bound covers it.
// Bounds past the binary32 range are taken as FLT_MAX (conservative), and an infinite max|y|
// (a sum beyond the binary32 range) fails the test, so the exact path produces the infinity.
__device__ __forceinline__ float pow2_or_max(uint32_t biased) {
  return biased >= 255u ? kFltMax : __uint_as_float(biased << 23);
}

// Returns true when the range test proves the result exact; bm = max_i |y_i|. `fmin`: the
// block's smallest nonzero exponent field, 255 for an all-zero block.
template <typename TIn>
__device__ __forceinline__ bool rht16_f64(const float (&v)[16], uint32_t mask, uint32_t fmin,
                                          float (&y)[16], float& bm) {
  constexpr bool kBf16 = sizeof(TIn) == 2;
  double u[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if constexpr (kBf16) u[j] = (double)__builtin_fmaf(v[j], ((mask >> j) & 1u) ? -0.25f : 0.25f, 0.0f);
    else u[j] = __builtin_fma((double)v[j], ((mask >> j) & 1u) ? -0.25 : 0.25, 0.0);
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
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    y[i] = (float)u[i];
    m = fmaxf(m, fabsf(y[i]));
  }
  bm = m;
  return m <= pow2_or_max(kBf16 ? fmin + 40u : fmin + 24u) * 0.9999847412109375f;   // 1 - 2^-16
}

// Exact outputs of one block (rarely taken; divergent). The block's 16 inputs are parked in this
// lane's slots of `lds` (the wave's kRhtExactLds floats: slot j of lane l at [j * 64 + l]) and read
// back one term at a time, so the path holds few registers beyond the outputs; the kernels that
// contain it keep their register count. Returns max_i |y_i|.
// WANT_Y = false computes only the maximum (the amax kernels), leaving y untouched.
constexpr int kRhtExactLds = 16 * 64;

template <bool WANT_Y = true>
__device__ __forceinline__ float rht16_exact(const float (&v)[16], uint32_t mask, float (&y)[16], float* lds) {
  const int lane = threadIdx.x & 63;
  uint32_t signs = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    lds[j * 64 + lane] = v[j];
    signs |= (__float_as_uint(v[j]) >> 31) << j;
  }
  float out[16];
  if constexpr (WANT_Y) {
#pragma unroll
    for (int k = 0; k < 16; ++k) out[k] = 0.0f;          // the binary64 values are not needed here
  }
  float m = 0.0f;
#pragma unroll 1
  for (uint32_t i = 0; i < 16; ++i) {
    const float r = exact_quarter_sum_at(lds + lane, 64, signs ^ mask ^ hadamard_row_negatives(i));
    if constexpr (WANT_Y) {
#pragma unroll
      for (uint32_t k = 0; k < 16; ++k) out[k] = (k == i) ? r : out[k];
    }
    m = fmaxf(m, fabsf(r));
  }
  if constexpr (WANT_Y) {
#pragma unroll
    for (int k = 0; k < 16; ++k) y[k] = out[k];
  }
  return m;
}

// Smallest nonzero exponent field (1 for subnormals; 255 if all are zero) from a running
// minimum of (magnitude << 1) - 1, where zero wraps to all ones. BF16: two values per word,
// packed 16-bit arithmetic (both halves at once): h * 2 + 0xFFFF drops the sign bit and
// subtracts one in a single packed multiply-add when the 2 comes from a register the compiler
// cannot see through (opaque_two; a literal 2 becomes a shift and a separate add). FP32: one
// value per word.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 opaque_two() {
  u16x2 two = {2, 2};
  asm volatile("" : "+v"(two));
  return two;
}
__device__ __forceinline__ u16x2 min_mag_bf16x2(u16x2 acc, uint32_t w, u16x2 two) {
  const u16x2 h = __builtin_bit_cast(u16x2, w);
  return __builtin_elementwise_min(acc, (u16x2)(h * two + (unsigned short)0xFFFF));
}
__device__ __forceinline__ uint32_t field_from_min_bf16(uint32_t mn) {
  if (mn == 0xFFFFu) return 255u;
  const uint32_t f = ((mn + 1u) & 0xFFFFu) >> 8;
  return f > 1u ? f : 1u;
}
__device__ __forceinline__ uint32_t min_field_f32(const float (&v)[16]) {
  uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < 16; ++j) mn = min(mn, (__float_as_uint(v[j]) << 1) - 1u);
  if (mn == 0xFFFFFFFFu) return 255u;
  const uint32_t f = (mn + 1u) >> 24;
  return f > 1u ? f : 1u;
}

// Segment containing `row` for a non-decreasing offset table off[0..nseg] (clamped).
__device__ __forceinline__ int64_t find_segment(const int64_t* off, int64_t nseg, int64_t row) {
  int64_t lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace nvfp4
