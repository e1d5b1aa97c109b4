// Exact evaluation of one output of the 16-point random-sign Hadamard transform ("Nemotron
// NVFP4" explainer, "Why 4-bit training normally falls apart - and the three fixes": the
// weight-gradient GEMM's inputs are multiplied by a random Hadamard matrix).
//
// y = rn32(1/4 * sum_j s_j * v_j) for 16 binary32 values v_j and signs s_j = +-1, rounded once
// to binary32 (nearest, ties to even; +0 for an exactly zero sum, the sign kept when a nonzero
// sum rounds to zero, infinity beyond the largest finite value). Used for blocks whose values
// span too many binades for a binary64 butterfly to be exact; plain C++ (no device builtins),
// so the same code is compiled for the host and checked there against the oracle.
//
// Method: every binary32 value quartered is an integer multiple of 2^-151, so the sum is an
// integer in units of 2^-151 of at most 283 bits. Each term m * 2^p (m < 2^24, p <= 253 its
// position in those units) is added into one of eight 64-bit limb sums at weight 2^(32 k)
// (k = p / 32, value m << (p % 32) < 2^55, so 16 terms cannot overflow), the limbs are
// normalised to 32-bit digits with a signed top digit, the magnitude is taken, and its leading
// 53 bits are rounded to odd (truncated, the last bit set when anything nonzero was dropped).
// Converting that binary64 value to binary32 gives the correctly rounded result: rounding to
// odd with at least two extra bits followed by round-to-nearest equals a single
// round-to-nearest (Boldo and Melquiond, "Emulation of FMA and correctly rounded sums: proved
// algorithms using rounding to odd", IEEE Trans. Computers 57(4), 2008).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Bit j of the result: (-1)^popcount(i & j) = -1, i.e. row i of the Sylvester Hadamard matrix
// as a sign mask.
__host__ __device__ inline uint32_t hadamard_row_negatives(uint32_t i) {
  return ((i & 1u) ? 0xAAAAu : 0u) ^ ((i & 2u) ? 0xCCCCu : 0u) ^ ((i & 4u) ? 0xF0F0u : 0u) ^
         ((i & 8u) ? 0xFF00u : 0u);
}

// rn32(1/4 * sum_j (-1)^(bit j of neg) * |v_j|) for 16 binary32 values (their sign bits are
// ignored; the caller folds them into neg). Finite inputs.
// The 16 values are read from v[0], v[stride], ..., v[15 * stride] one at a time (the loop over
// terms is not unrolled), so only the limb sums stay live.
__host__ __device__ inline float exact_quarter_sum_at(const float* v, int stride, uint32_t neg) {
  int64_t L[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 1
  for (int j = 0; j < 16; ++j) {
    uint32_t bits;
    __builtin_memcpy(&bits, v + j * stride, 4);
    const uint32_t e = (bits >> 23) & 0xFFu;
    const uint64_t m = (uint64_t)((bits & 0x7FFFFFu) | (e ? 0x800000u : 0u));
    const uint32_t p = (e ? e : 1u) - 1u;                 // v/4 = m * 2^(p - 151)
    const uint32_t w = p >> 5;
    int64_t c = (int64_t)(m << (p & 31u));
    if ((neg >> j) & 1u) c = -c;
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) L[k] += (w == k) ? c : 0;
  }
  // digits d[0..7] in [0, 2^32) and a signed top digit
  uint32_t d[9];
  int64_t carry = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t t = L[k] + carry;
    d[k] = (uint32_t)t;
    carry = t >> 32;                                      // arithmetic: floor division
  }
  const bool negative = carry < 0;
  if (negative) {                                         // two's complement of all 9 digits
    uint64_t c1 = 1;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint64_t s = (uint64_t)(uint32_t)~d[k] + c1;
      d[k] = (uint32_t)s;
      c1 = s >> 32;
    }
    carry = ~carry + (int64_t)c1;
  }
  d[8] = (uint32_t)carry;                                 // |sum| < 2^283: fits one digit
  // leading nonzero digit t; the 96 bits d[t], d[t-1], d[t-2]; everything below is sticky
  int t = -1;
#pragma unroll
  for (int k = 0; k < 9; ++k) t = d[k] ? k : t;
  if (t < 0) return 0.0f;                                 // exact zero: +0
  uint32_t hi = 0, mid = 0, lo = 0, sticky = 0;
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    hi = (k == t) ? d[k] : hi;
    mid = (k == t - 1) ? d[k] : mid;
    lo = (k == t - 2) ? d[k] : lo;
    sticky |= (k < t - 2) ? d[k] : 0u;
  }
  const int n = __builtin_clz(hi);                        // hi != 0: normalise the window
  if (n) {
    hi = (hi << n) | (mid >> (32 - n));
    mid = (mid << n) | (lo >> (32 - n));
    lo <<= n;
  }
  // top 64 bits; lo now holds the bits below them
  const uint64_t W = ((uint64_t)hi << 32) | mid;
  uint64_t w53 = W >> 11;
  if ((W & 0x7FFu) | lo | sticky) w53 |= 1u;              // round to odd at 53 bits
  // the 96-bit window's lowest bit weighs 2^(32(t-2) - 151); after the shift by n and
  // dropping 32 + 11 bits, w53's unit weighs 2^(32 t - n - 172)
  const int k = 32 * t - n - 172;                         // in [-203, 84]
  union { uint64_t u; double f; } s;
  s.u = (uint64_t)(k + 1023) << 52;
  const double mag = (double)w53 * s.f;                   // exact: w53 < 2^53
  return (float)(negative ? -mag : mag);
}

}  // namespace nvfp4
