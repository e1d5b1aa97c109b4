// MXFP4 quantization of a tensor's columns: x[rows, cols] -> out[cols, rows], each output row (an
// input column) quantized along the input rows in 32-element blocks. The format is the pages'
// comparison format ("Nemotron NVFP4" explainer, "What NVFP4 actually is": E2M1 elements, one
// power-of-two E8M0 scale per 32 elements, no tensor scale); the result is by definition the
// row-wise MXFP4 quantization of x^T (mxfp4_quantize of the transposed tensor): shared exponent
// e = floor(log2(block amax)) - 2 clamped to [-127, 127], elements E2M1(x * 2^-e) rounded to
// nearest or stochastically with the Philox bytes of the 16-element half block at its place in
// the output. The activation-gradient and weight-gradient GEMMs contract over the other
// dimension of W, dY and X than the forward one, so these operands need exactly this.
//
// Layout: a tile is 128 columns x 256 rows (8 blocks of 32). Lane l of a wave owns columns 2l
// and 2l+1, so a wave-wide load of one row is 256 contiguous bytes (BF16); wave w takes the
// 32-row blocks w and w + 4 of the tile. Workgroups walk tiles with a stride of the grid (the
// resident workgroup count); each wave requests its next block's 32 rows before encoding the
// current one. Codes and E8M0 bytes are staged in LDS as [column][row]; codes go out as
// 128-byte row segments of the transposed tensor, scales as two 4-byte pieces per output row
// (the scale layout is K step by K step, so consecutive output rows' pieces are consecutive).
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTileCols = 128;                  // 64 lanes x 2 columns
constexpr int kTileRows = 256;                  // 8 blocks of 32 rows
constexpr int kBlocksPerTile = kTileRows / 32;
constexpr int kItemsPerWave = kBlocksPerTile / kWaves;

// Columns c and c+1 of one row, kept packed until use (as the Hadamard kernel's loads).
template <typename TIn>
struct ColPair;

template <>
struct ColPair<uint16_t> {
  uint32_t w;
  __device__ __forceinline__ void load(const uint16_t* p, bool both, bool paired) {
    if (both && paired) w = *reinterpret_cast<const uint32_t*>(p);
    else w = (uint32_t)p[0] | (both ? (uint32_t)p[1] << 16 : 0u);
  }
  __device__ __forceinline__ void load_pair(const uint16_t* p) { w = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ float get(int q) const { return q == 0 ? bf16_lo(w) : bf16_hi(w); }
};

template <>
struct ColPair<float> {
  v2f32 w;
  __device__ __forceinline__ void load(const float* p, bool both, bool paired) {
    if (both && paired) w = *reinterpret_cast<const v2f32*>(p);
    else w = v2f32{p[0], both ? p[1] : 0.0f};
  }
  __device__ __forceinline__ void load_pair(const float* p) { w = *reinterpret_cast<const v2f32*>(p); }
  __device__ __forceinline__ float get(int q) const { return q == 0 ? w.x : w.y; }
};

template <typename TIn, bool SR>
__global__ __launch_bounds__(kThreads) void k_encode_mx_cols(
    const TIn* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, uint64_t seed, uint64_t offset) {
  __shared__ __attribute__((aligned(16))) uint8_t tc[kTileCols][kTileRows / 2];
  __shared__ __attribute__((aligned(16))) uint8_t ts[kTileCols][kBlocksPerTile];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar registers
  const int64_t nblk = rows >> 5;                               // 32-row blocks
  const int64_t tiles_c = (cols + kTileCols - 1) / kTileCols;
  const int64_t tiles = tiles_c * ((nblk + kBlocksPerTile - 1) / kBlocksPerTile);
  const bool paired = (ld & 1) == 0;
  const int64_t halves = rows >> 4;                             // 16-element halves per output row

  struct Geo { int64_t C0, B0; };
  auto geo = [&](int64_t it) {
    const int64_t tt = it / tiles_c;
    return Geo{(it - tt * tiles_c) * kTileCols, tt * kBlocksPerTile};
  };
  auto load_item = [&](ColPair<TIn> (&raw)[32], int64_t it, int k) {
    const Geo g = geo(it);
    const int64_t c = g.C0 + 2 * lane;
    const int64_t cl = c < cols ? c : 0;                          // clamped column for loads
    const int64_t b = g.B0 + wave + kWaves * k;
    const int64_t bl = b < nblk ? b : 0;                          // clamped block for loads
    const TIn* p = x + bl * 32 * ld + cl;
    if (paired && (g.C0 + kTileCols <= cols || (cols & 1) == 0)) {
      // uniform: every lane's pair is whole and aligned (a full tile, or even rows; lanes past
      // the row read columns 0 and 1, whose results are never written); branch-free loads keep
      // all 32 rows in flight at once, where the per-element form's branches would make each
      // load of a partial last tile wait for the one before. Odd strides or odd rows take the
      // per-element loads.
#pragma unroll
      for (int j = 0; j < 32; ++j) raw[j].load_pair(p + j * ld);
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) raw[j].load(p + j * ld, c + 1 < cols, paired);
    }
  };

  ColPair<TIn> cur[32], nxt[32];
  int64_t it = blockIdx.x;
  int k = 0;
  if (it < tiles) load_item(cur, it, 0);

  auto step = [&](ColPair<TIn> (&cur)[32], ColPair<TIn> (&nxt)[32]) {
    int64_t it_n = it;
    int k_n = k + 1;
    if (k_n == kItemsPerWave) {
      k_n = 0;
      it_n = it + gridDim.x;
    }
    if (it_n < tiles) load_item(nxt, it_n, k_n);

    const Geo g = geo(it);
    const int64_t c = g.C0 + 2 * lane;
    const int bl = wave + kWaves * k;                             // block within the tile
    const int64_t b = g.B0 + bl;
    if (b < nblk) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float v[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = cur[j].get(q);
        float am = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) am = fmaxf(am, fabsf(v[j]));
        int e = am > 0.0f ? __builtin_amdgcn_frexp_expf(am) - 3 : -127;   // floor(log2 am) - 2
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
        const float mult = __builtin_ldexpf(1.0f, -e);
        const int64_t orow = c + q;                               // output row = input column
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float h16[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) h16[j] = v[16 * hh + j];
          u32x4 rnd{0, 0, 0, 0};
          if constexpr (SR) rnd = block_random((uint64_t)(orow * halves + 2 * b + hh), seed, offset);
          uint32_t lo, hi;
          encode16<SR>(h16, mult, rnd, lo, hi);
          *reinterpret_cast<uint2*>(&tc[2 * lane + q][bl * 16 + hh * 8]) = make_uint2(lo, hi);
        }
        ts[2 * lane + q][bl] = (uint8_t)(e + 127);
      }
    }

    if (k == kItemsPerWave - 1) {                                 // tile complete: write x^T rows
      __syncthreads();
      const int64_t valid_cols = cols - g.C0 < kTileCols ? cols - g.C0 : kTileCols;
      const int64_t valid_b = nblk - g.B0 < kBlocksPerTile ? nblk - g.B0 : kBlocksPerTile;
      // codes: 128 columns x 8 blocks of 16 bytes, one 16-byte piece per thread and pass
#pragma unroll
      for (int pass = 0; pass < kTileCols * kBlocksPerTile / kThreads; ++pass) {
        const int idx = pass * kThreads + threadIdx.x;
        const int cr = idx >> 3, p = idx & 7;
        if (cr < valid_cols && p < valid_b)
          *reinterpret_cast<uint4*>(codes + (g.C0 + cr) * (rows >> 1) + (g.B0 + p) * 16) =
              *reinterpret_cast<const uint4*>(&tc[cr][p * 16]);
      }
      // scales K step by K step (block j of output row c at byte ((j / 4) * cols + c) * 4 +
      // j % 4): the tile's 8 blocks are two 4-byte pieces of each output row, and consecutive
      // output rows' pieces are consecutive dwords
      if (threadIdx.x < valid_cols) {
        const int64_t c = g.C0 + threadIdx.x;
        const int cr = threadIdx.x;
        if (valid_b == kBlocksPerTile) {
          *reinterpret_cast<uint32_t*>(scales + ((g.B0 >> 2) * cols + c) * 4) =
              *reinterpret_cast<const uint32_t*>(&ts[cr][0]);
          *reinterpret_cast<uint32_t*>(scales + (((g.B0 >> 2) + 1) * cols + c) * 4) =
              *reinterpret_cast<const uint32_t*>(&ts[cr][4]);
        } else {
          for (int p = 0; p < valid_b; ++p)
            scales[(((g.B0 + p) >> 2) * cols + c) * 4 + ((g.B0 + p) & 3)] = ts[cr][p];
        }
      }
      __syncthreads();                                            // LDS reused by the next tile
    }
    it = it_n;
    k = k_n;
  };
  while (it < tiles) {                                            // uniform across the workgroup
    step(cur, nxt);
    if (it >= tiles) break;
    step(nxt, cur);
  }
}

template <typename TIn, bool SR>
int64_t resident_groups_mx() {
  static const int64_t n = [] {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_encode_mx_cols<TIn, SR>, kThreads, 0) != hipSuccess)
      return (int64_t)1024;
    return (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
  }();
  return n;
}

template <typename TIn, bool SR>
void launch_mx_cols_t(const void* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes, uint8_t* scales,
                      uint64_t seed, uint64_t offset, hipStream_t stream) {
  const int64_t tiles = ((cols + kTileCols - 1) / kTileCols) * (((rows >> 5) + kBlocksPerTile - 1) / kBlocksPerTile);
  const int64_t cap = resident_groups_mx<TIn, SR>();
  const int grid = (int)(tiles < cap ? (tiles < 1 ? 1 : tiles) : cap);
  hipLaunchKernelGGL((k_encode_mx_cols<TIn, SR>), dim3(grid), dim3(kThreads), 0, stream, (const TIn*)x, rows, cols, ld,
                     codes, scales, seed, offset);
}

}  // namespace

hipError_t launch_encode_mx_cols(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld, bool sr,
                                 uint64_t seed, uint64_t offset, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (fp32) {
    if (sr) launch_mx_cols_t<float, true>(x, rows, cols, ld, codes, scales, seed, offset, stream);
    else launch_mx_cols_t<float, false>(x, rows, cols, ld, codes, scales, seed, offset, stream);
  } else {
    if (sr) launch_mx_cols_t<uint16_t, true>(x, rows, cols, ld, codes, scales, seed, offset, stream);
    else launch_mx_cols_t<uint16_t, false>(x, rows, cols, ld, codes, scales, seed, offset, stream);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
