// Random Hadamard transform + transposed 1x16 quantization of the weight-gradient operands.
//
// "Nemotron NVFP4" explainer, "Why 4-bit training normally falls apart - and the three
// fixes": the wgrad GEMM's inputs are multiplied by a random Hadamard matrix before
// quantization, which spreads an outlier over its block, and the rotation cancels inside the
// GEMM. The rotation acts along the contraction (token) dimension in blocks of 16 tokens:
// for column c and token block t, y = 1/4 * H16 * diag(s) * x[16t..16t+15, c], with
// H16[i][j] = (-1)^popcount(i & j) and signs s from a 16-bit mask, each output the exact
// value rounded once to FP32 (rht16_f64: a binary64 butterfly where a range test proves it
// exact; rht16_exact: exact integer sums otherwise). The 16 outputs of one (column, token block)
// are exactly one 1x16 quantization block of the transposed output [cols, tokens].
//
// Layout: a tile is 128 columns x 256 tokens (16 token blocks). Lane l of every wave owns
// columns 2l and 2l+1, so a wave-wide load of one token row is 64 x 4 bytes (BF16) of
// contiguous memory; wave w handles token blocks w, w+4, w+8, w+12 of a tile. Workgroups walk
// tiles with a stride of the grid (sized to what the device keeps resident), and each wave
// requests the 16 rows of its next token block before transforming the current one, across
// tile boundaries too. Codes and scales are staged in LDS as [column][token block] and written
// out as 128-byte row segments of the transposed tensor. The amax variant walks the same tiles
// and leaves one partial maximum per workgroup; its PLAIN form also keeps max|x| of the
// untransformed input (a second array of partials), so one read of a tensor gives the tensor
// scales of both its rowwise and its Hadamard quantization.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTileCols = 128;                  // 64 lanes x 2 columns
constexpr int kTileBlocks = 16;                 // 256 tokens
constexpr int kBlocksPerWave = kTileBlocks / kWaves;
constexpr int kMaxPartials = 1024;
constexpr int kLdsSeg = 512;                    // segment tables up to this size live in LDS
constexpr int kAccWin = 64;                     // SEG amax: per-workgroup window of segment maxima

// Columns c and c+1 of one token row, kept packed until use. `both` says whether c+1
// exists; `paired` whether the pair is aligned for one vector load (even row stride), else
// two scalar loads are used.
template <typename TIn>
struct Pair;

template <>
struct Pair<uint16_t> {
  uint32_t w;
  __device__ __forceinline__ void load(const uint16_t* p, bool both, bool paired) {
    if (both && paired) w = *reinterpret_cast<const uint32_t*>(p);
    else w = (uint32_t)p[0] | (both ? (uint32_t)p[1] << 16 : 0u);
  }
  __device__ __forceinline__ void load_pair(const uint16_t* p) { w = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ float get(int q) const { return q == 0 ? bf16_lo(w) : bf16_hi(w); }
};

template <>
struct Pair<float> {
  v2f32 w;
  __device__ __forceinline__ void load(const float* p, bool both, bool paired) {
    if (both && paired) w = *reinterpret_cast<const v2f32*>(p);
    else w = v2f32{p[0], both ? p[1] : 0.0f};
  }
  __device__ __forceinline__ void load_pair(const float* p) { w = *reinterpret_cast<const v2f32*>(p); }
  __device__ __forceinline__ float get(int q) const { return q == 0 ? w.x : w.y; }
};


__device__ __forceinline__ float block_max(float m, float* red) {
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// SEG: token segments (the tokens of each expert, multiples of 16) with one tensor scale each.
// Tables of up to kLdsSeg segments are copied into LDS (segment starts; for encode also each
// segment's encode scale), so finding an item's segment costs no global round trip, and each
// workgroup walks a contiguous range of tiles (instead of a grid stride; the encode form
// backwards), so consecutive tiles share their token rows and a wave's segment cursor rarely
// moves. The amax form folds each wave's runs of items in one segment into an LDS window of
// per-segment maxima, and the workgroup ends with one global atomic max per segment it
// touched (partial[segment], zeroed by the caller). The encode form takes the scale of the
// item's segment.
template <typename TIn, bool ENCODE, bool SR, bool PLAIN = false, bool SEG = false>
__global__ __launch_bounds__(kThreads, (ENCODE && SEG && sizeof(TIn) == 2) ? 3 : 1) void k_rht(
    const TIn* __restrict__ x, int64_t tokens, int64_t cols, int64_t ld, uint32_t mask,
    const float* __restrict__ amax, int amax_parts, float* __restrict__ partial,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gscale,
    const int64_t* __restrict__ seg, int64_t nseg, uint64_t seed, uint64_t offset) {
  static_assert(!(PLAIN && SEG), "the amax pair is unsegmented");
  __shared__ float red[kWaves];
  __shared__ __attribute__((aligned(16))) uint8_t tc[ENCODE ? kTileCols : 1][kTileBlocks * 8];
  __shared__ __attribute__((aligned(16))) uint8_t ts[ENCODE ? kTileCols : 1][kTileBlocks];
  __shared__ float rtab[ENCODE ? 128 : 1];       // block multipliers of the tensor scale
  __shared__ int64_t sseg[SEG ? kLdsSeg : 1];     // segment starts (nseg <= kLdsSeg)
  __shared__ float ssenc[SEG && ENCODE ? kLdsSeg : 1];
  __shared__ float sacc[SEG && !ENCODE ? kAccWin : 1];
  __shared__ float sexact[kWaves][kRhtExactLds];  // the exact transform's per-wave slots
  constexpr bool kBlocked = SEG;                 // contiguous tile range per workgroup

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar registers
  const int64_t nbt = tokens >> 4;
  const u16x2 two = opaque_two();                  // for the range test's packed minimum
  const int64_t tiles_c = (cols + kTileCols - 1) / kTileCols;
  const int64_t tiles = tiles_c * ((nbt + kTileBlocks - 1) / kTileBlocks);
  const bool paired = (ld & 1) == 0;

  // A workgroup walks tiles blockIdx.x, blockIdx.x + gridDim.x, ...; in each, wave w takes the
  // token blocks w, w+4, w+8, w+12 (item k = 0..3). The next item's 16 rows are requested
  // before the current item is transformed, also across tiles.
  struct Geo { int64_t C0, TB0; };
  const int64_t per = kBlocked ? (tiles + gridDim.x - 1) / gridDim.x : 0;
  const int64_t it_begin = kBlocked ? (int64_t)blockIdx.x * per : (int64_t)blockIdx.x;
  const int64_t it_end = kBlocked ? (it_begin + per < tiles ? it_begin + per : tiles) : tiles;
  const int64_t rbase = kBlocked ? it_begin + it_end - 1 : tiles - 1;
  auto geo = [&](int64_t it) {
    const int64_t tile = ENCODE ? rbase - it : it;       // encode walks back over the amax order
    const int64_t tt = tile / tiles_c;
    return Geo{(tile - tt * tiles_c) * kTileCols, tt * kTileBlocks};
  };
  auto load_item = [&](Pair<TIn> (&raw)[16], int64_t it, int k) {
    const Geo g = geo(it);
    const int64_t c = g.C0 + 2 * lane;
    const int64_t cl = c < cols ? c : 0;                    // clamped column for loads
    const int64_t tb = g.TB0 + wave + 4 * k;
    const int64_t tbl = tb < nbt ? tb : 0;                  // clamped token block for loads
    const TIn* p = x + tbl * 16 * ld + cl;
    // uniform: every lane's pair is whole and aligned: in a full tile, or in the last, partial
    // one when the rows are even (lanes past the row then read columns 0 and 1, whose results
    // are never used). Only odd strides or odd rows take the per-element loads, whose branches
    // make each load wait for the one before (a partial last tile read that way cost 2-3 full
    // tiles: [102656, 1856] at 2.7 TB/s against 4.1 TB/s at 1920 columns).
    if (paired && (g.C0 + kTileCols <= cols || (cols & 1) == 0)) {
#pragma unroll
      for (int j = 0; j < 16; ++j) raw[j].load_pair(p + j * ld);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) raw[j].load(p + j * ld, c + 1 < cols, paired);
    }
  };

  Pair<TIn> cur[16], nxt[16];
  int64_t it = it_begin;
  const int64_t it_stride = kBlocked ? 1 : gridDim.x;
  int k = 0;
  if (it < it_end) load_item(cur, it, 0);

  const bool lds_seg = SEG && nseg <= kLdsSeg;
  if constexpr (SEG) {
    if (lds_seg) {
      for (int64_t i = threadIdx.x; i < nseg; i += kThreads) {
        sseg[i] = seg[i];
        if constexpr (ENCODE) ssenc[i] = tensor_encode_scale(amax[i]);
      }
    }
    if constexpr (!ENCODE) {
      for (int i = threadIdx.x; i < kAccWin; i += kThreads) sacc[i] = 0.0f;
    }
    __syncthreads();
  }

  // Segment of a token block (the last segment whose first token is at or before the block's
  // first token, as find_segment): a per-wave cursor that moves from the previous item's
  // segment, so a walk in either direction costs O(1) table reads per item.
  int64_t sg = 0;
  auto seg_walk = [&](const int64_t* t, int64_t tok) {
    while (sg > 0 && t[sg] > tok) --sg;
    while (sg + 1 < nseg && t[sg + 1] <= tok) ++sg;
    return sg;
  };
  auto seg_of = [&](int64_t tb) { return lds_seg ? seg_walk(sseg, tb * 16) : seg_walk(seg, tb * 16); };
  // SEG amax: the window of segments [win_lo, win_lo + kAccWin) is kept in LDS; win_lo is the
  // segment of the workgroup's first token (segments only grow along the walk).
  int64_t win_lo = 0;
  if constexpr (SEG && !ENCODE) {
    if (it < it_end) win_lo = seg_of(geo(it).TB0);
  }
  auto flush = [&](int64_t sgi, float mv) {            // uniform: one wave's run maximum
    const float wm = wave_max(mv);
    if (lane == 0) {
      // (a malformed, decreasing table can put sgi below the window: the global path then)
      if ((uint64_t)(sgi - win_lo) < (uint64_t)kAccWin)
        atomicMax(reinterpret_cast<unsigned int*>(&sacc[sgi - win_lo]), __float_as_uint(wm));
      else
        atomic_max_nonneg(partial + sgi, wm);
    }
  };
  int64_t se_seg = -1;                                      // SEG encode: segment of se_cached
  float se_cached = 1.0f;

  float s_enc = 1.0f;
  if constexpr (ENCODE && SEG) {
    if (blockIdx.x == 0)
      for (int64_t i = threadIdx.x; i < nseg; i += kThreads) gscale[i] = tensor_decode_scale(amax[i]);
  } else if constexpr (ENCODE) {
    float a = 0.0f;
    if (amax_parts <= 1) {
      a = amax[0];
    } else {
      for (int i = threadIdx.x; i < amax_parts; i += kThreads) a = fmaxf(a, amax[i]);
      a = block_max(a, red);
    }
    s_enc = tensor_encode_scale(a);
    if (blockIdx.x == 0 && threadIdx.x == 0) gscale[0] = tensor_decode_scale(a);
    build_recip_table(s_enc, rtab);
    __syncthreads();
  }

  float m = 0.0f, mp = 0.0f;                                // max|Hx|, max|x| (PLAIN)
  int64_t m_seg = -1;                                       // SEG amax: segment of m
  // One token block: request the next one into `nxt`, transform `cur`. The loop alternates
  // the two register sets (no copies between blocks).
  auto step = [&](Pair<TIn> (&cur)[16], Pair<TIn> (&nxt)[16]) {
    int64_t it_n = it;
    int k_n = k + 1;
    if (k_n == kBlocksPerWave) {
      k_n = 0;
      it_n = it + it_stride;
    }
    if (it_n < it_end) load_item(nxt, it_n, k_n);

    const Geo g = geo(it);
    const int64_t c = g.C0 + 2 * lane;
    const int bl = wave + 4 * k;                            // token block within the tile
    const int64_t tb = g.TB0 + bl;
    if (tb < nbt) {
      float se = s_enc;
      if constexpr (SEG) {
        const int64_t sgi = seg_of(tb);
        if constexpr (ENCODE) {
          if (sgi != se_seg) {
            se_seg = sgi;
            se_cached = lds_seg ? ssenc[sgi] : tensor_encode_scale(amax[sgi]);
          }
          se = se_cached;
        } else if (sgi != m_seg) {                          // uniform: flush the previous run
          if (m_seg >= 0) flush(m_seg, m);
          m = 0.0f;
          m_seg = sgi;
        }
      }
      // smallest nonzero exponent field of each column's block (the transform's range test)
      // and, for the amax pair, each column's max|x|: packed 16-bit arithmetic on BF16 words
      uint32_t fmin[2] = {255u, 255u};
      float pmax[2] = {0.0f, 0.0f};
      if constexpr (sizeof(TIn) == 2) {
        u16x2 acc = {0xFFFF, 0xFFFF}, mag = {0, 0};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          acc = min_mag_bf16x2(acc, cur[j].w, two);
          if constexpr (PLAIN)
            mag = __builtin_elementwise_max(mag, __builtin_bit_cast(u16x2, cur[j].w & 0x7FFF7FFFu));
        }
        fmin[0] = field_from_min_bf16(acc.x);
        fmin[1] = field_from_min_bf16(acc.y);
        pmax[0] = __uint_as_float((uint32_t)mag.x << 16);
        pmax[1] = __uint_as_float((uint32_t)mag.y << 16);
      }
      // The block of column c + q: its maximum into the tensor maximum, or its scale and codes
      // into the tile's LDS staging.
      auto finish = [&](int q, const float (&y)[16], float bm) {
        if constexpr (!ENCODE) {
          if (c + q < cols) m = fmaxf(m, bm);
        } else {
          const int64_t row = c + q;                        // output row = input column
          BlockScale bs;
          if constexpr (SEG) bs = block_scale(bm, se);
          else bs = block_scale_table(bm, s_enc, rtab);
          u32x4 rnd{0, 0, 0, 0};
          if constexpr (SR) rnd = block_random((uint64_t)(row * nbt + tb), seed, offset);
          uint32_t lo, hi;
          encode16<SR>(y, bs.mult, rnd, lo, hi);
          *reinterpret_cast<uint2*>(&tc[2 * lane + q][bl * 8]) = make_uint2(lo, hi);
          ts[2 * lane + q][bl] = (uint8_t)bs.code;
        }
      };
      uint32_t pending = 0;                                 // bit q: block q needs exact sums
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float v[16], y[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = cur[j].get(q);
        if constexpr (PLAIN) {
          float pm = pmax[q];
          if constexpr (sizeof(TIn) != 2) {
#pragma unroll
            for (int j = 0; j < 16; ++j) pm = fmaxf(pm, fabsf(v[j]));
          }
          if (c + q < cols) mp = fmaxf(mp, pm);
        }
        float bm;
        if (rht16_f64<TIn>(v, mask, sizeof(TIn) == 2 ? fmin[q] : min_field_f32(v), y, bm)) finish(q, y, bm);
        else pending |= 1u << q;
      }
      if (pending) {
        // rare (divergent): exact sums for the blocks the range test rejected, once the item's
        // loaded words are no longer needed; their inputs are read again from memory, so
        // nothing is kept in registers across the butterflies above for this path.
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if ((pending >> q) & 1u) {
            Pair<TIn> again[16];
            load_item(again, it, k);
            float v[16], y[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = again[j].get(q);
            const float bm = rht16_exact<ENCODE>(v, mask, y, sexact[wave]);
            finish(q, y, bm);
          }
        }
      }
    }

    if constexpr (ENCODE) {
      if (k == kBlocksPerWave - 1) {                        // tile complete: write x^T rows
        __syncthreads();
        const int64_t valid_cols = cols - g.C0 < kTileCols ? cols - g.C0 : kTileCols;
        const int64_t valid_tb = nbt - g.TB0 < kTileBlocks ? nbt - g.TB0 : kTileBlocks;
#pragma unroll
        for (int pass = 0; pass < kTileCols * kTileBlocks / kThreads; ++pass) {
          const int idx = pass * kThreads + threadIdx.x;
          const int cr = idx >> 4, p = idx & 15;
          if (cr < valid_cols && p < valid_tb)
            *reinterpret_cast<uint2*>(codes + (g.C0 + cr) * (tokens >> 1) + (g.TB0 + p) * 8) =
                *reinterpret_cast<const uint2*>(&tc[cr][p * 8]);
        }
        if (threadIdx.x < valid_cols) {
          const int cr = threadIdx.x;
          uint8_t* dst = scales + (g.C0 + cr) * nbt + g.TB0;
          if (valid_tb == kTileBlocks && ((reinterpret_cast<uintptr_t>(dst) & 15) == 0)) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(&ts[cr][0]);
          } else {
            for (int p = 0; p < valid_tb; ++p) dst[p] = ts[cr][p];
          }
        }
        __syncthreads();                                    // LDS reused by the next tile
      }
    }
    it = it_n;
    k = k_n;
  };
  while (it < it_end) {                                     // uniform across the workgroup
    step(cur, nxt);
    if (it >= it_end) break;
    step(nxt, cur);
  }
  if constexpr (!ENCODE && SEG) {
    if (m_seg >= 0) flush(m_seg, m);
    __syncthreads();
    for (int i = threadIdx.x; i < kAccWin; i += kThreads) {
      const float v = sacc[i];
      if (__float_as_uint(v) != 0u && win_lo + i < nseg) atomic_max_nonneg(partial + win_lo + i, v);
    }
  } else if constexpr (!ENCODE) {
    m = block_max(m, red);
    if constexpr (PLAIN) {                                  // [max|x| partials][max|Hx| partials]
      mp = block_max(mp, red);
      if (threadIdx.x == 0) {
        partial[blockIdx.x] = mp;
        partial[gridDim.x + blockIdx.x] = m;
      }
    } else {
      if (threadIdx.x == 0) partial[blockIdx.x] = m;
    }
  }
}

int64_t rht_tiles(int64_t tokens, int64_t cols) {
  return ((cols + kTileCols - 1) / kTileCols) * (((tokens >> 4) + kTileBlocks - 1) / kTileBlocks);
}

// Workgroups of k_rht<...> that the device keeps resident at once (each walks tiles, so a
// grid of exactly this many has no second wave of late starters). Queried once per kernel.
template <typename TIn, bool ENCODE, bool SR, bool PLAIN, bool SEG>
int64_t resident_groups() {
  static const int64_t n = [] {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_rht<TIn, ENCODE, SR, PLAIN, SEG>, kThreads, 0) !=
            hipSuccess)
      return (int64_t)1024;
    return (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
  }();
  return n;
}

// Every form walks tiles with a stride of its grid, so a grid of more workgroups than stay
// resident would only add a tail of late starters: the grid is capped at the resident count
// (the amax forms then leave that many partial maxima, at most kMaxPartials).
template <typename TIn, bool ENCODE, bool SR, bool PLAIN = false, bool SEG = false>
void launch_rht_t(const void* x, int64_t tokens, int64_t cols, int64_t ld, uint16_t mask,
                  const float* amax, int parts, float* partial, QuantOut out,
                  const int64_t* segments, int64_t nseg, uint64_t seed, uint64_t offset, int& grid,
                  hipStream_t stream) {
  const int64_t cap = resident_groups<TIn, ENCODE, SR, PLAIN, SEG>();
  if (grid > cap) grid = (int)cap;
  hipLaunchKernelGGL((k_rht<TIn, ENCODE, SR, PLAIN, SEG>), dim3(grid), dim3(kThreads), 0, stream,
                     (const TIn*)x, tokens, cols, ld, (uint32_t)mask, amax, parts, partial,
                     out.codes, out.scales, out.global_scale, segments, nseg, seed, offset);
}

}  // namespace

hipError_t launch_rht_amax_parts(const void* x, bool fp32, int64_t tokens, int64_t cols, int64_t ld,
                                 uint16_t sign_mask, bool plain, const int64_t* segments,
                                 int64_t nseg, float* partial, int* parts, hipStream_t stream) {
  const int64_t tiles = rht_tiles(tokens, cols);
  int grid = (int)(tiles < 1 ? 1 : (tiles < kMaxPartials ? tiles : kMaxPartials));
  const QuantOut none{nullptr, nullptr, nullptr};
  if (segments) {                                 // per-segment maxima straight into partial[nseg]
    hipError_t e = launch_fill(partial, nseg, 0.0f, stream);
    if (e != hipSuccess) return e;
    if (fp32) launch_rht_t<float, false, false, false, true>(x, tokens, cols, ld, sign_mask, nullptr, 0, partial, none, segments, nseg, 0, 0, grid, stream);
    else      launch_rht_t<uint16_t, false, false, false, true>(x, tokens, cols, ld, sign_mask, nullptr, 0, partial, none, segments, nseg, 0, 0, grid, stream);
    *parts = 1;
    return hipGetLastError();
  }
#define NVFP4_RA(T, P) launch_rht_t<T, false, false, P>(x, tokens, cols, ld, sign_mask, nullptr, 0, partial, none, nullptr, 1, 0, 0, grid, stream)
  if (fp32) { if (plain) NVFP4_RA(float, true); else NVFP4_RA(float, false); }
  else      { if (plain) NVFP4_RA(uint16_t, true); else NVFP4_RA(uint16_t, false); }
#undef NVFP4_RA
  *parts = grid;
  return hipGetLastError();
}

hipError_t launch_rht_encode(const void* x, bool fp32, int64_t tokens, int64_t cols, int64_t ld,
                             uint16_t sign_mask, bool sr, uint64_t seed, uint64_t offset,
                             const int64_t* segments, int64_t nseg, const float* amax, int parts,
                             QuantOut out, hipStream_t stream) {
  const int64_t tiles = rht_tiles(tokens, cols);
  int grid = (int)(tiles < 1 ? 1 : (tiles < (1 << 30) ? tiles : (1 << 30)));   // capped at launch
#define NVFP4_RE(T, S, G) launch_rht_t<T, true, S, false, G>(x, tokens, cols, ld, sign_mask, amax, parts, nullptr, out, segments, nseg, seed, offset, grid, stream)
  const bool seg = segments != nullptr;
  if (fp32) {
    if (sr) { if (seg) NVFP4_RE(float, true, true); else NVFP4_RE(float, true, false); }
    else    { if (seg) NVFP4_RE(float, false, true); else NVFP4_RE(float, false, false); }
  } else {
    if (sr) { if (seg) NVFP4_RE(uint16_t, true, true); else NVFP4_RE(uint16_t, true, false); }
    else    { if (seg) NVFP4_RE(uint16_t, false, true); else NVFP4_RE(uint16_t, false, false); }
  }
#undef NVFP4_RE
  return hipGetLastError();
}

}  // namespace nvfp4
