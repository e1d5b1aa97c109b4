// Host build of the exact Hadamard output (csrc/rht_exact.h) for a CPU test against the
// oracle. Reads blocks from stdin: a count n, then per block a 16-bit sign mask followed by
// 16 binary32 bit patterns (hex); writes the 16 transformed outputs of each block as binary32
// bit patterns, output i = rn32(1/4 * sum_j H[i][j] * s_j * v_j) through exact_quarter_sum_at.
#include <cstdio>

#include "../../bit_block_scaled_quantize_amd/csrc/rht_exact.h"

int main() {
  long n = 0;
  if (std::scanf("%ld", &n) != 1) return 1;
  for (long blk = 0; blk < n; ++blk) {
    unsigned mask = 0;
    float b[16];
    if (std::scanf("%x", &mask) != 1) return 1;
    uint32_t signs = 0;
    for (int j = 0; j < 16; ++j) {
      unsigned v = 0;
      if (std::scanf("%x", &v) != 1) return 1;
      __builtin_memcpy(&b[j], &v, 4);
      signs |= (v >> 31) << j;
    }
    for (uint32_t i = 0; i < 16; ++i) {
      const float y = nvfp4::exact_quarter_sum_at(b, 1, signs ^ mask ^ nvfp4::hadamard_row_negatives(i));
      union { float f; uint32_t u; } c;
      c.f = y;
      std::printf("%08x%c", c.u, i == 15 ? '\n' : ' ');
    }
  }
  return 0;
}
