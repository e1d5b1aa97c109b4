// NVFP4 block quantization kernels for gfx950: tensor amax, 1x16 encode (nearest or
// stochastic rounding) and 16x16 encode with optional transposed emission.
//
// Format and recipe: "Nemotron NVFP4" explainer, "What NVFP4 actually is" (E2M1 elements,
// one E4M3 scale per 16 elements, one FP32 tensor scale) and "Why 4-bit training normally
// falls apart - and the three fixes" (2D weight blocks, stochastic rounding of gradients);
// artiverse.ca "NVIDIA's 4-bit floating point pushes AI training limits" (16x16 weight
// blocks instead of 1x16, stochastic rounding on gradients only).
//
// All kernels stream from HBM with 16-byte vector loads that cover contiguous row spans.
// The tensor amax (needed before any block scale is final) is a separate pass: for an
// unsegmented tensor each workgroup writes one partial maximum and the encode kernel folds
// the partials itself (no same-address atomics, no extra launch); for per-expert segments
// one atomic max per (wave, segment run) lands on that segment's slot. The encode pass walks
// the tensor in the reverse order of the amax pass so that its first reads hit the lines
// the amax pass touched last (still in the 256 MB Infinity Cache).
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;
constexpr int kMaxPartials = 1024;
constexpr int kAmaxUnroll = 8;         // 16-byte loads in flight per thread in the amax pass

__device__ __forceinline__ float abs_max16(const float (&v)[16]) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(v[j]));
  return m;
}

// max |.| of one 16-byte vector of inputs (8 BF16 or 4 FP32)
template <typename TIn>
__device__ __forceinline__ float vec_absmax(const TIn* p);

template <>
__device__ __forceinline__ float vec_absmax<uint16_t>(const uint16_t* p) {
  const v4u32 a = ld_u32x4(p);
  return fmaxf(fmaxf(fmaxf(fabsf(bf16_lo(a.x)), fabsf(bf16_hi(a.x))),
                     fmaxf(fabsf(bf16_lo(a.y)), fabsf(bf16_hi(a.y)))),
               fmaxf(fmaxf(fabsf(bf16_lo(a.z)), fabsf(bf16_hi(a.z))),
                     fmaxf(fabsf(bf16_lo(a.w)), fabsf(bf16_hi(a.w)))));
}

template <>
__device__ __forceinline__ float vec_absmax<float>(const float* p) {
  const v4f32 a = ld_f32x4(p);
  return fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w)));
}

// Workgroup-wide max; every thread gets the result.
__device__ __forceinline__ float block_max(float m, float* red) {
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------------------
// amax, unsegmented: workgroup b reduces its share of the 16-byte vectors of x (rows of
// `vecs_per_row` vectors, row stride ld) into partial[b].
template <typename TIn>
__global__ __launch_bounds__(kThreads) void k_amax_partial(const TIn* __restrict__ x, int64_t rows,
                                                           int64_t vecs_per_row, int64_t ld,
                                                           float* __restrict__ partial) {
  __shared__ float red[kWavesPerBlock];
  constexpr int64_t kVec = 16 / sizeof(TIn);
  const int64_t total = rows * vecs_per_row;
  const int64_t per = (total + gridDim.x - 1) / gridDim.x;
  const int64_t q0 = (int64_t)blockIdx.x * per;
  const int64_t q1 = q0 + per < total ? q0 + per : total;
  const bool contiguous = ld == vecs_per_row * kVec;
  float m = 0.0f;
  int64_t q = q0 + threadIdx.x;
  for (; q + (kAmaxUnroll - 1) * kThreads < q1; q += kAmaxUnroll * kThreads) {
    float a[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int64_t qq = q + u * kThreads;
      const int64_t off = contiguous ? qq * kVec : (qq / vecs_per_row) * ld + (qq % vecs_per_row) * kVec;
      a[u] = vec_absmax<TIn>(x + off);
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) m = fmaxf(m, a[u]);
  }
  if (q < q1) {
    // the last (fewer than kAmaxUnroll) vectors of the thread, requested together: indices past
    // the range read the range's last vector again, which leaves the maximum unchanged (a loop
    // of single loads would pay one memory round trip per vector)
    float a[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int64_t qq = q + u * kThreads < q1 ? q + u * kThreads : q1 - 1;
      const int64_t off = contiguous ? qq * kVec : (qq / vecs_per_row) * ld + (qq % vecs_per_row) * kVec;
      a[u] = vec_absmax<TIn>(x + off);
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) m = fmaxf(m, a[u]);
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// One 16-byte vector of inputs, loaded now and reduced later (so a batch of loads is in
// flight before the first one is used).
template <typename TIn>
struct Vec16;

template <>
struct Vec16<uint16_t> {
  v4u32 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = ld_u32x4(p); }
  __device__ __forceinline__ float absmax() const {
    return fmaxf(fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))), fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y)))),
                 fmaxf(fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))), fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w)))));
  }
};

template <>
struct Vec16<float> {
  v4f32 v;
  __device__ __forceinline__ void load(const float* p) { v = ld_f32x4(p); }
  __device__ __forceinline__ float absmax() const {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  }
};

// amax per row segment (row r counts toward segment find_segment(seg, nseg, r)). Workgroup b
// reduces a contiguous range of the tensor's 16-byte vectors, walked as in the unsegmented
// pass (thread t takes vectors t, t + 256, ... of the range, eight requested at a time). A
// thread's rows only grow along its walk, so it keeps the maximum of its current segment and
// hands it to an LDS window of per-segment maxima (LDS atomics) when its row enters another
// segment; the workgroup ends with one global atomic max per segment of the window it touched
// (the slots start at zero). Offset tables of up to kSegTab entries are searched in LDS; the
// table's loads are requested before the first vectors, so the search waits on one round trip
// that the data loads share.
template <typename TIn>
__global__ __launch_bounds__(kThreads) void k_amax_seg(const TIn* __restrict__ x, int64_t rows,
                                                       int64_t vecs_per_row, int64_t ld,
                                                       const int64_t* __restrict__ seg, int64_t nseg,
                                                       float* __restrict__ amax_out) {
  constexpr int64_t kVec = 16 / sizeof(TIn);
  constexpr int kSegTab = 1024, kWin = 64;
  __shared__ int64_t stab[kSegTab];
  __shared__ unsigned int sacc[kWin];
  __shared__ int64_t swin_s;
  const int64_t total = rows * vecs_per_row;
  const int64_t per = (total + gridDim.x - 1) / gridDim.x;
  const int64_t q0 = (int64_t)blockIdx.x * per;
  const int64_t q1 = q0 + per < total ? q0 + per : total;
  if (q0 >= q1) return;                                     // uniform: an empty range
  const bool contiguous = ld == vecs_per_row * kVec;
  const bool in_lds = nseg < kSegTab;                        // nseg + 1 offsets
  const int64_t* off = in_lds ? stab : seg;

  // the table's entries for this thread (clamped indices: every load is valid)
  constexpr int kTabLoads = kSegTab / kThreads;
  int64_t tv[kTabLoads];
  if (in_lds) {
#pragma unroll
    for (int k = 0; k < kTabLoads; ++k) {
      const int64_t i = threadIdx.x + k * kThreads;
      tv[k] = seg[i <= nseg ? i : nseg];
    }
  }
  // position of the thread's first vector, advanced by 256 vectors per step
  const int64_t d_row = kThreads / vecs_per_row, d_col = kThreads % vecs_per_row;
  int64_t q = q0 + threadIdx.x;
  int64_t row = q / vecs_per_row, col = q - (q / vecs_per_row) * vecs_per_row;
  const int64_t last_el = contiguous ? (q1 - 1) * kVec
                                     : ((q1 - 1) / vecs_per_row) * ld + ((q1 - 1) % vecs_per_row) * kVec;
  Vec16<TIn> a[kAmaxUnroll];
  int64_t arow[kAmaxUnroll];
  bool avalid[kAmaxUnroll];
  // requests the next batch: vectors q, q + 256, ... (past the range: the range's last vector
  // again, not counted)
  auto issue = [&]() {
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int64_t qq = q + u * kThreads;
      avalid[u] = qq < q1;
      arow[u] = row;
      const int64_t off_el = !avalid[u] ? last_el : contiguous ? qq * kVec : row * ld + col * kVec;
      a[u].load(x + off_el);
      col += d_col;
      row += d_row;
      if (col >= vecs_per_row) {
        col -= vecs_per_row;
        ++row;
      }
    }
    q += kAmaxUnroll * kThreads;
  };
  const bool any = q < q1;
  if (any) issue();

  if (in_lds) {
#pragma unroll
    for (int k = 0; k < kTabLoads; ++k) {
      const int64_t i = threadIdx.x + k * kThreads;
      if (i <= nseg) stab[i] = tv[k];
    }
  }
  for (int i = threadIdx.x; i < kWin; i += kThreads) sacc[i] = 0u;
  __syncthreads();
  if (threadIdx.x == 0) swin_s = find_segment(off, nseg, q0 / vecs_per_row);
  __syncthreads();
  const int64_t swin = swin_s;

  // the thread's current segment [.., seg_end) and its running maximum
  int64_t cur = swin;
  auto seg_end_of = [&](int64_t c) { return c + 1 < nseg ? off[c + 1] : INT64_MAX; };
  int64_t seg_end = seg_end_of(cur);
  float m = 0.0f;
  auto flush = [&]() {
    if (m > 0.0f) {
      if (cur - swin < kWin) atomicMax(&sacc[cur - swin], __float_as_uint(m));
      else atomic_max_nonneg(amax_out + cur, m);
    }
    m = 0.0f;
  };
  auto consume = [&]() {
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      if (avalid[u]) {
        if (arow[u] >= seg_end) {                            // rare: the next segment
          flush();
          while (cur + 1 < nseg && off[cur + 1] <= arow[u]) ++cur;
          seg_end = seg_end_of(cur);
        }
        m = fmaxf(m, a[u].absmax());
      }
    }
  };
  bool pending = any;
  while (pending) {
    consume();
    pending = q < q1;
    if (pending) issue();
  }
  flush();
  __syncthreads();
  for (int i = threadIdx.x; i < kWin; i += kThreads) {
    const unsigned int v = sacc[i];
    if (v != 0u && swin + i < nseg) atomic_max_nonneg(amax_out + swin + i, __uint_as_float(v));
  }
}

__global__ void k_fill(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Workgroup i folds the i-th array of `parts` partial maxima into out[i].
__global__ __launch_bounds__(kThreads) void k_reduce_partials(const float* __restrict__ partial,
                                                              int parts, float* __restrict__ out) {
  __shared__ float red[kWavesPerBlock];
  const float* p = partial + (int64_t)blockIdx.x * parts;
  float m = 0.0f;
  for (int i = threadIdx.x; i < parts; i += kThreads) m = fmaxf(m, p[i]);
  m = block_max(m, red);
  if (threadIdx.x == 0) out[blockIdx.x] = m;
}

// Tensor amax seen by an encode workgroup: either amax[seg] directly (parts == 1) or the
// max of `parts` partial maxima of an unsegmented tensor.
__device__ __forceinline__ float fold_amax(const float* __restrict__ amax, int parts, float* red) {
  if (parts <= 1) return amax[0];
  float m = 0.0f;
  for (int i = threadIdx.x; i < parts; i += kThreads) m = fmaxf(m, amax[i]);
  return block_max(m, red);
}

// ---------------------------------------------------------------------------------------
// 1x16 encode: lane = one 16-element block. A wave walks its rows (rows wave, wave + nwaves, ...
// counted from the end of the tensor, the reverse of the amax pass) in chunks of U blocks per
// lane (64*U consecutive blocks of a row) and keeps the next chunk's loads in flight while it
// encodes the current one; the first chunk is requested before the tensor amax is folded, so
// the fold hides under the load latency.
// Lane-pair exchange (DPP quad permute [1,0,3,2]): every lane receives its partner's value.
__device__ __forceinline__ uint32_t pair_swap(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}

// Chunk of U groups of 64 consecutive blocks of one row. BF16: each load instruction covers
// 1 KiB of the row contiguously (lane l: bytes 16l..16l+15 of a group half), so lane l holds
// half l%2 of block l/2 (first 1 KiB) and of block 32 + l/2 (second 1 KiB); one lane-pair
// exchange then gives even lanes block l/2 and odd lanes block 32 + l/2 of the group whole.
// FP32: each lane loads its own 64-byte block.
template <typename TIn>
struct Chunk;

template <>
struct Chunk<uint16_t> {
  static constexpr int U = 4;
  v4u32 h0[U], h1[U];                                   // first / second KiB of group u
  __device__ __forceinline__ static int64_t block_of(int lane, int u) {
    return 64 * u + ((lane & 1) << 5) + (lane >> 1);
  }
  __device__ __forceinline__ void load_group(const uint16_t* xr, int64_t b0, int64_t nb, int lane, int u) {
    const int64_t g = b0 + 64 * u;
    if (g + (lane >> 1) < nb) h0[u] = ld_u32x4(xr + g * 16 + lane * 8);
    if (g + 32 + (lane >> 1) < nb) h1[u] = ld_u32x4(xr + g * 16 + 512 + lane * 8);
  }
  __device__ __forceinline__ void load(const uint16_t* xr, int64_t b0, int64_t nb, int lane) {
#pragma unroll
    for (int u = 0; u < U; ++u) load_group(xr, b0, nb, lane, u);
  }
  __device__ __forceinline__ void get(int u, int lane, float (&v)[16]) const {
    uint32_t w[8];
    get(u, lane, v, w);
  }
  // the same, also returning the block's 8 words (element 2i in the low half of word i)
  __device__ __forceinline__ void get(int u, int lane, float (&v)[16], uint32_t (&w)[8]) const {
    const bool odd = lane & 1;
    v4u32 send = odd ? h0[u] : h1[u], recv;
    recv.x = pair_swap(send.x);
    recv.y = pair_swap(send.y);
    recv.z = pair_swap(send.z);
    recv.w = pair_swap(send.w);
    const v4u32 lo = odd ? recv : h0[u];                 // elements 0..7 of the lane's block
    const v4u32 hi = odd ? h1[u] : recv;                 // elements 8..15
    w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
    w[4] = hi.x; w[5] = hi.y; w[6] = hi.z; w[7] = hi.w;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  }
};

template <>
struct Chunk<float> {
  static constexpr int U = 2;
  v4f32 q[U][4];
  __device__ __forceinline__ static int64_t block_of(int lane, int u) { return 64 * u + lane; }
  __device__ __forceinline__ void load_group(const float* xr, int64_t b0, int64_t nb, int lane, int u) {
    const int64_t b = b0 + block_of(lane, u);
    if (b < nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) q[u][i] = ld_f32x4(xr + b * 16 + 4 * i);
    }
  }
  __device__ __forceinline__ void load(const float* xr, int64_t b0, int64_t nb, int lane) {
#pragma unroll
    for (int u = 0; u < U; ++u) load_group(xr, b0, nb, lane, u);
  }
  __device__ __forceinline__ void get(int u, int, float (&v)[16]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[4 * i] = q[u][i].x;
      v[4 * i + 1] = q[u][i].y;
      v[4 * i + 2] = q[u][i].z;
      v[4 * i + 3] = q[u][i].w;
    }
  }
};

// The lane's block u of a chunk put through the Hadamard transform (rowwise rotation) by the
// binary64 butterfly; returns its range test (rht16_f64). The smallest nonzero exponent field
// comes from the BF16 words with packed 16-bit arithmetic, or from the FP32 values.
// bm = max_i |y_i|.
template <typename TIn>
__device__ __forceinline__ bool rot_block(const Chunk<TIn>& c, int u, int lane, uint32_t mask,
                                          float (&y)[16], float& bm) {
  float v[16];
  uint32_t fmin;
  if constexpr (sizeof(TIn) == 2) {
    uint32_t w[8];
    c.get(u, lane, v, w);
    u16x2 acc = {0xFFFF, 0xFFFF};
    const u16x2 two = opaque_two();
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = min_mag_bf16x2(acc, w[i], two);
    fmin = field_from_min_bf16(min((uint32_t)acc.x, (uint32_t)acc.y));
  } else {
    c.get(u, lane, v);
    fmin = min_field_f32(v);
  }
  return rht16_f64<TIn>(v, mask, fmin, y, bm);
}

// The blocks of a chunk whose range test failed (bit u of `pending`, per lane), once the chunk's
// registers are no longer needed: block group u is read again from memory (row pointer xr,
// first block b0; wave-wide, like the exchange inside get()), the failing lanes compute exact
// sums and hand them to finish(u, y, bm). Rarely taken; keeps the main path's registers.
template <bool WANT_Y, typename TIn, typename Finish>
__device__ __forceinline__ void rot_pending(uint32_t pending, const TIn* xr, int64_t b0, int64_t nb, int lane,
                                            uint32_t mask, float* lds, Finish finish) {
  if (!__any(pending != 0)) return;
#pragma unroll 1
  for (int u = 0; u < Chunk<TIn>::U; ++u) {
    if (!__any((pending >> u) & 1u)) continue;
    Chunk<TIn> c;                                 // group u of the chunk, held as group 0
    c.load_group(xr, b0 + 64 * u, nb, lane, 0);
    float v[16], y[16];
    c.get(0, lane, v);
    if ((pending >> u) & 1u) {
      const float bm = rht16_exact<WANT_Y>(v, mask, y, lds);
      finish(u, y, bm);
    }
  }
}

// ROT: each block is first put through the 16-point random-sign Hadamard transform (sign
// mask `mask`), the rowwise rotation of the activation gradient of the Mosaic variant's dgrad
// GEMM (thelatentdaily "What matters for NVFP4 training?": transforms on both backward GEMMs).
template <typename TIn, bool SR, bool SEG, bool ROT = false>
__global__ __launch_bounds__(kThreads) void k_encode_1x16(
    const TIn* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ amax, int amax_parts, const int64_t* __restrict__ seg, int64_t nseg,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gscale,
    uint64_t seed, uint64_t offset, uint32_t mask = 0) {
  static_assert(!(SEG && ROT), "the rotated encode is unsegmented");
  using C = Chunk<TIn>;
  constexpr int U = C::U;
  constexpr int64_t kSpan = 64 * U;            // blocks of a row covered by one chunk
  __shared__ float red[kWavesPerBlock];
  __shared__ float rexact[ROT ? kWavesPerBlock : 1][ROT ? kRhtExactLds : 1];   // exact transform slots
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t nb = cols >> 4;

  // Rows are walked downwards (the amax pass left the last rows in cache): without segments
  // with a stride of all waves; with segments, each workgroup takes a contiguous row range
  // whose rows its waves share out in turn (wave w: the range's last row - w, then every
  // fourth row), so a wave meets few segment changes and a workgroup's loads stay together.
  // Row r = base - it for it = it0, it0 + stride, ... < lim.
  int64_t base = rows - 1, it0 = wave, stride = nwaves, lim = rows;
  if constexpr (SEG) {
    const int64_t per = (rows + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per < rows ? (int64_t)blockIdx.x * per : rows;
    const int64_t hi = lo + per < rows ? lo + per : rows;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    base = hi - 1 - w;
    it0 = 0;
    stride = kWavesPerBlock;
    lim = hi - lo - w;
  }
  C cur, nxt;
  int64_t it = it0, b0 = 0;
  if (it < lim) cur.load(x + (base - it) * ld, b0, nb, lane);
  // SEG: offset tables of up to kSegLds entries are searched in LDS (one round trip for the
  // workgroup, requested behind the first chunk's loads, instead of a binary search through
  // global memory per wave)
  constexpr int kSegLds = SEG ? 1024 : 1;
  __shared__ int64_t sseg[kSegLds];
  const bool seg_in_lds = SEG && nseg < kSegLds;
  if constexpr (SEG) {
    if (seg_in_lds)
      for (int64_t i = threadIdx.x; i <= nseg; i += kThreads) sseg[i] = seg[i];
    __syncthreads();
  }
  const int64_t* off = seg_in_lds ? sseg : seg;

  const float a0 = fold_amax(amax, SEG ? 1 : amax_parts, red);
  if (blockIdx.x == 0) {
    if constexpr (SEG) {
      for (int64_t i = threadIdx.x; i < nseg; i += kThreads) gscale[i] = tensor_decode_scale(amax[i]);
    } else if (threadIdx.x == 0) {
      gscale[0] = tensor_decode_scale(a0);
    }
  }
  float s_enc = tensor_encode_scale(a0);
  // Block multipliers of the tensor scale: one table per workgroup, or with segments one per
  // wave, rebuilt when the wave enters another segment. seg_lo/seg_hi: the current segment's
  // row range (empty before the first row).
  __shared__ float rtab[SEG ? kWavesPerBlock : 1][128];
  float* tab = rtab[SEG ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0];
  int64_t seg_lo = 0, seg_hi = 0;
  if constexpr (!SEG) {
    build_recip_table(s_enc, tab);
    __syncthreads();
  }

  // One chunk: request the next chunk into `nxt`, encode `cur`. The loop alternates the two
  // buffers (no register copies between chunks).
  auto step = [&](C& cur, C& nxt) {
    int64_t it_n = it, b0_n = b0 + kSpan;
    if (b0_n >= nb) {
      b0_n = 0;
      it_n = it + stride;
    }
    if (it_n < lim) nxt.load(x + (base - it_n) * ld, b0_n, nb, lane);

    const int64_t r = base - it;
    if constexpr (SEG) {
      if (r < seg_lo || r >= seg_hi) {                       // uniform: another segment
        const int64_t sg = find_segment(off, nseg, r);
        seg_lo = off[sg];
        seg_hi = off[sg + 1];
        s_enc = tensor_encode_scale(amax[sg]);
        __builtin_amdgcn_wave_barrier();                     // the wave's reads of the old table
        tab[lane] = block_recip(lane, s_enc);
        tab[lane + 64] = block_recip(lane + 64, s_enc);
        __builtin_amdgcn_wave_barrier();
      }
    }
    uint2* cr = reinterpret_cast<uint2*>(codes + r * (cols >> 1));
    uint8_t* sr = scales + r * nb;
    auto finish = [&](int u, const float (&v)[16], float bm) {
      const int64_t b = b0 + C::block_of(lane, u);
      if (b < nb) {
        const BlockScale bs = block_scale_table(bm, s_enc, tab);
        u32x4 rnd{0, 0, 0, 0};
        if constexpr (SR) rnd = block_random((uint64_t)(r * nb + b), seed, offset);
        uint32_t lo, hi;
        encode16<SR>(v, bs.mult, rnd, lo, hi);
        cr[b] = make_uint2(lo, hi);
        sr[b] = (uint8_t)bs.code;
      }
    };
    uint32_t pending = 0;                        // ROT: bit u: block u needs exact sums
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float v[16], bm = 0.0f;
      if constexpr (ROT) {
        if (!rot_block(cur, u, lane, mask, v, bm)) {
          pending |= 1u << u;                    // encoded below, after the exact sums
          continue;
        }
      } else {
        cur.get(u, lane, v);                     // all lanes: the exchange is wave-wide
        bm = abs_max16(v);
      }
      finish(u, v, bm);
    }
    if constexpr (ROT) rot_pending<true>(pending, x + r * ld, b0, nb, lane, mask, rexact[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)], finish);
    it = it_n;
    b0 = b0_n;
  };
  while (it < lim) {
    step(cur, nxt);
    if (it >= lim) break;
    step(nxt, cur);
  }
}

// Partial maxima of the rowwise-rotated tensor (the amax of k_encode_1x16<.., ROT>): waves walk
// rows as the encode does, one partial per workgroup.
template <typename TIn>
__global__ __launch_bounds__(kThreads) void k_amax_rot(const TIn* __restrict__ x, int64_t rows, int64_t cols,
                                                       int64_t ld, uint32_t mask, float* __restrict__ partial) {
  using C = Chunk<TIn>;
  constexpr int U = C::U;
  constexpr int64_t kSpan = 64 * U;
  __shared__ float red[kWavesPerBlock];
  __shared__ float rexact[kWavesPerBlock][kRhtExactLds];                   // exact transform slots
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t nb = cols >> 4;
  C cur, nxt;
  int64_t r = wave, b0 = 0;
  float m = 0.0f;
  if (r < rows) cur.load(x + r * ld, b0, nb, lane);
  auto step = [&](C& cur, C& nxt) {
    int64_t r_n = r, b0_n = b0 + kSpan;
    if (b0_n >= nb) {
      b0_n = 0;
      r_n = r + nwaves;
    }
    if (r_n < rows) nxt.load(x + r_n * ld, b0_n, nb, lane);
    auto finish = [&](int u, const float (&)[16], float bm) {
      if (b0 + C::block_of(lane, u) < nb) m = fmaxf(m, bm);
    };
    uint32_t pending = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float y[16], bm;
      if (rot_block(cur, u, lane, mask, y, bm)) finish(u, y, bm);
      else pending |= 1u << u;
    }
    rot_pending<false>(pending, x + r * ld, b0, nb, lane, mask, rexact[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)], finish);
    r = r_n;
    b0 = b0_n;
  };
  while (r < rows) {
    step(cur, nxt);
    if (r >= rows) break;
    step(nxt, cur);
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// ---------------------------------------------------------------------------------------
// MXFP4 encode, the format the pages compare NVFP4 with ("Nemotron NVFP4" explainer, "What
// NVFP4 actually is"): 32-element blocks with one power-of-two (E8M0) scale and no tensor
// scale, so one pass over the input. The shared exponent is floor(log2(block amax)) - 2,
// clamped to [-127, 127] (the block's largest element lands in [4, 8)); elements are
// x * 2^-e (exact) rounded to E2M1 as in the 1x16 encode, stochastically with the same
// Philox bytes per 16-element half. Lane = one 16-element half, walked as k_encode_1x16
// walks blocks; the halves of a 32-block sit in lanes l and l^2 (BF16 chunks) or l and l^1
// (FP32 chunks) and swap their maxima.
template <typename TIn>
__device__ __forceinline__ uint32_t mx_partner(uint32_t v) {
  constexpr int kCtrl = sizeof(TIn) == 2 ? 0x4E : 0xB1;        // quad_perm [2,3,0,1] / [1,0,3,2]
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, false);
}

template <typename TIn, bool SR>
__global__ __launch_bounds__(kThreads) void k_encode_mx(const TIn* __restrict__ x, int64_t rows,
                                                        int64_t cols, int64_t ld,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, uint64_t seed,
                                                        uint64_t offset) {
  using C = Chunk<TIn>;
  constexpr int U = C::U;
  constexpr int64_t kSpan = 64 * U;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t nb = cols >> 4;                        // 16-element halves per row (even)

  C cur, nxt;
  int64_t r = wave, b0 = 0;
  if (r < rows) cur.load(x + r * ld, b0, nb, lane);
  auto step = [&](C& cur, C& nxt) {
    int64_t r_n = r, b0_n = b0 + kSpan;
    if (b0_n >= nb) {
      b0_n = 0;
      r_n = r + nwaves;
    }
    if (r_n < rows) nxt.load(x + r_n * ld, b0_n, nb, lane);
    uint2* cr = reinterpret_cast<uint2*>(codes + r * (cols >> 1));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float v[16];
      cur.get(u, lane, v);
      const float m16 = abs_max16(v);
      const float am = fmaxf(m16, __uint_as_float(mx_partner<TIn>(__float_as_uint(m16))));
      int e = am > 0.0f ? __builtin_amdgcn_frexp_expf(am) - 3 : -127;   // floor(log2 am) - 2
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
      const int64_t b = b0 + C::block_of(lane, u);
      if (b < nb) {
        u32x4 rnd{0, 0, 0, 0};
        if constexpr (SR) rnd = block_random((uint64_t)(r * nb + b), seed, offset);
        uint32_t lo, hi;
        encode16<SR>(v, __builtin_ldexpf(1.0f, -e), rnd, lo, hi);
        cr[b] = make_uint2(lo, hi);
        // scales K step by K step: block j of row r at byte ((j / 4) * rows + r) * 4 + j % 4
        if ((b & 1) == 0) scales[((b >> 3) * rows + r) * 4 + ((b >> 1) & 3)] = (uint8_t)(e + 127);
      }
    }
    r = r_n;
    b0 = b0_n;
  };
  while (r < rows) {
    step(cur, nxt);
    if (r >= rows) break;
    step(nxt, cur);
  }
}

// ---------------------------------------------------------------------------------------
// 16x16 encode. A workgroup owns a 256-row x 128-column tile: 16 strips of 16 rows x 8 tiles
// of 16 columns. Lane pairs own one 16x16 tile (each lane 16 rows x 8 columns; the tile amax
// is combined across the pair with one cross-lane max). Codes of x are written row by row
// (4 bytes per lane); the transposed copy (x^T: row c holds column c) is assembled in LDS
// and written as 128-byte row segments (256 rows of x = 128 bytes of x^T codes).
constexpr int kTileRows = 256, kTileCols = 128;

template <typename TIn>
struct Raw8;                                   // 8 consecutive inputs of one row

template <>
struct Raw8<uint16_t> {
  v4u32 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = ld_u32x4(p); }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t word = (i >> 1) == 0 ? w.x : (i >> 1) == 1 ? w.y : (i >> 1) == 2 ? w.z : w.w;
    return (i & 1) ? bf16_hi(word) : bf16_lo(word);
  }
};

template <>
struct Raw8<float> {
  v4f32 a, b;
  __device__ __forceinline__ void load(const float* p) { a = ld_f32x4(p); b = ld_f32x4(p + 4); }
  __device__ __forceinline__ float get(int i) const {
    const v4f32& v = i < 4 ? a : b;
    const int k = i & 3;
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
  }
};

// In-place transpose of an 8x8 matrix of nibbles held as 8 words (word j, nibble i =
// element (j, i)): swap the off-diagonal 4x4 blocks (16-bit halves), then the 2x2 blocks
// (bytes), then single nibbles; afterwards word i, nibble j = the former element (j, i).
__device__ __forceinline__ void nibble_transpose8(uint32_t (&w)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t a = w[j], b = w[j + 4];
    w[j] = __builtin_amdgcn_perm(b, a, 0x05040100u);      // a.h0 | b.h0 << 16
    w[j + 4] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // a.h1 | b.h1 << 16
  }
#pragma unroll
  for (int j : {0, 1, 4, 5}) {
    const uint32_t a = w[j], b = w[j + 2];
    w[j] = __builtin_amdgcn_perm(b, a, 0x06020400u);      // a.b0 b.b0 a.b2 b.b2
    w[j + 2] = __builtin_amdgcn_perm(b, a, 0x07030501u);  // a.b1 b.b1 a.b3 b.b3
  }
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const uint32_t a = w[j], b = w[j + 1];
    w[j] = (a & 0x0F0F0F0Fu) | ((b & 0x0F0F0F0Fu) << 4);
    w[j + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  }
}

// With SEG and TRANS (an expert weight stack of nseg equal segments of seg_rows rows, a
// multiple of 16), segment g's transpose goes to rows g*cols .. of x^T [nseg*cols, seg_rows].
template <typename TIn, bool SEG, bool TRANS>
__global__ __launch_bounds__(kThreads) void k_encode_16x16(
    const TIn* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ amax, int amax_parts, const int64_t* __restrict__ seg, int64_t nseg,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gscale,
    uint8_t* __restrict__ tcodes, uint8_t* __restrict__ tscales, float* __restrict__ tgscale,
    int64_t seg_rows) {
  __shared__ float red[kWavesPerBlock];
  __shared__ __attribute__((aligned(16))) uint8_t tc[TRANS ? kTileCols : 1][kTileRows / 2];
  __shared__ __attribute__((aligned(16))) uint8_t ts[TRANS ? kTileCols : 1][kTileRows / 16];

  const int64_t tiles_c = (cols + kTileCols - 1) / kTileCols;
  const int64_t tiles_r = (rows + kTileRows - 1) / kTileRows;
  // Workgroups are dealt to the 8 XCDs round robin; XCD x takes a contiguous eighth of the
  // walk, so the tiles that share a 128-byte line of codes or scales write it through one L2,
  // which merges the pieces before the line goes to HBM (tiles on different XCDs wrote partial
  // lines). The walk runs in the reverse order of the amax pass, by rows of tiles (side-by-side
  // tiles share lines of x's codes and scales); with the transpose of one whole tensor, in
  // bands of 8 rows of tiles, column by column, so that the up to 8 tiles stacked one above
  // the other that share a line of x^T's scales also run back to back (measured 5% faster on
  // a [20480, 5120] weight; on an expert stack the band walk measured 3% slower).
  const int64_t n_tiles = tiles_r * tiles_c;
  const int64_t per = (n_tiles + 7) / 8;
  const int64_t xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const int64_t tall = (n_tiles % 8) == 0 ? 8 : (n_tiles % 8);
  const int64_t id = xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
  const int64_t t = n_tiles - 1 - id;
  int64_t tile_r, tile_c;
  if constexpr (TRANS && !SEG) {
    constexpr int64_t kBand = 8;
    const int64_t first_r = (t / (kBand * tiles_c)) * kBand;
    const int64_t gr = tiles_r - first_r < kBand ? tiles_r - first_r : kBand;
    const int64_t in_band = t - first_r * tiles_c;
    tile_r = first_r + in_band % gr;
    tile_c = in_band / gr;
  } else {
    tile_r = t / tiles_c;
    tile_c = t - tile_r * tiles_c;
  }
  const int64_t R0 = tile_r * kTileRows, C0 = tile_c * kTileCols;

  const float a0 = fold_amax(amax, SEG ? 1 : amax_parts, red);
  if (blockIdx.x == 0) {
    if constexpr (SEG) {
      for (int64_t i = threadIdx.x; i < nseg; i += kThreads) {
        gscale[i] = tensor_decode_scale(amax[i]);
        if constexpr (TRANS) tgscale[i] = gscale[i];
      }
    } else if (threadIdx.x == 0) {
      gscale[0] = tensor_decode_scale(a0);
      if constexpr (TRANS) tgscale[0] = gscale[0];
    }
  }

  const int lane = threadIdx.x & 63;
  const int strip = (threadIdx.x >> 6) * 4 + (lane >> 4);   // 0..15
  const int ht = lane & 15;                                 // 8-column piece within the tile
  const int64_t r0 = R0 + strip * 16;
  const int64_t c0 = C0 + ht * 8;
  const bool active = r0 < rows && c0 < cols;
  const int64_t nb = cols >> 4;

  Raw8<TIn> v[16];
  float m = 0.0f;
  const TIn* xp = x + (active ? r0 : 0) * ld + (active ? c0 : 0);
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j].load(xp + j * ld);

  float s_enc;
  if constexpr (SEG) {
    // the segment starts and each segment's encode scale go to LDS in the round trip of the
    // tile's loads (requested first) and the strip's segment is searched there (a binary
    // search through global memory per thread cost several round trips per workgroup)
    constexpr int kSegLds = 1024;
    __shared__ int64_t sseg[kSegLds];
    __shared__ float ssenc[kSegLds];
    if (nseg < kSegLds) {
      for (int64_t i = threadIdx.x; i <= nseg; i += kThreads) {
        sseg[i] = seg[i];
        if (i < nseg) ssenc[i] = tensor_encode_scale(amax[i]);
      }
      __syncthreads();
      s_enc = ssenc[find_segment(sseg, nseg, active ? r0 : 0)];
    } else {
      s_enc = tensor_encode_scale(amax[find_segment(seg, nseg, active ? r0 : 0)]);
    }
  } else {
    s_enc = tensor_encode_scale(a0);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j].get(i)));
  m = fmaxf(m, __shfl_xor(m, 1, 64));                       // partner lane: other 8 columns
  const BlockScale bs = block_scale(m, s_enc);

  uint32_t w[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = v[j].get(i) * bs.mult;
    w[j] = e2m1_rn8(y);
  }
  // The strip's 8 tile scales are the same on each of its 16 rows: gather them from the lane
  // pairs of the 16-lane group (all lanes take part in the exchange) and let lane ht write
  // row r0 + ht's 8-byte segment in one store when the segment is whole and aligned.
  const int grp = lane & ~15;
  uint32_t srow[2] = {0, 0};
#pragma unroll
  for (int t = 0; t < 8; ++t)
    srow[t >> 2] |= ((uint32_t)__shfl((int)bs.code, grp + 2 * t, 64) & 0xFFu) << (8 * (t & 3));
  const bool whole_row = (nb & 7) == 0 && C0 + kTileCols <= cols;
  if (active) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      *reinterpret_cast<uint32_t*>(codes + (r0 + j) * (cols >> 1) + (c0 >> 1)) = w[j];
    if (whole_row) {
      *reinterpret_cast<uint2*>(scales + (r0 + ht) * nb + (C0 >> 4)) = make_uint2(srow[0], srow[1]);
    } else if ((ht & 1) == 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) scales[(r0 + j) * nb + (c0 >> 4)] = (uint8_t)bs.code;
    }
  }
  if constexpr (TRANS) {
    // column i of this lane's piece -> row (ht*8 + i) of the transposed tile, 16 codes:
    // two 8x8 nibble transposes (rows 0-7 and 8-15 of the strip)
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo[j] = w[j];
      hi[j] = w[j + 8];
    }
    nibble_transpose8(lo);
    nibble_transpose8(hi);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<uint2*>(&tc[ht * 8 + i][strip * 8]) = make_uint2(lo[i], hi[i]);
      ts[ht * 8 + i][strip] = (uint8_t)bs.code;
    }
    __syncthreads();
    // write-out: x^T row C0 + cr, bytes [R0/2, R0/2 + 128), in 8-byte pieces (one strip each)
    const int64_t valid_strips = (rows - R0) / 16 < 16 ? (rows - R0) / 16 : 16;
    const int64_t valid_cols = cols - C0 < kTileCols ? cols - C0 : kTileCols;
    if constexpr (SEG) {
      // the rows R0 + 16 sp .. of a strip lie in one segment g: they go to x^T row
      // g*cols + C0 + cr at the strip's offset within its segment
      if ((seg_rows & 63) == 0) {
        // Segments then start on 4-strip boundaries (rows, and so R0 and valid_strips, are
        // multiples of 64): the codes of strips 2i, 2i+1 and the scales of strips 4i .. 4i+3
        // lie in one segment, 16- and 4-byte aligned in x^T (an expert's 928-byte x^T rows
        // for 1856 rows put a tile's 128-byte pieces off line boundaries; whole 16-byte and
        // 4-byte stores in place of 8-byte and single-byte ones).
#pragma unroll
        for (int pass = 0; pass < kTileCols * 8 / kThreads; ++pass) {
          const int idx = pass * kThreads + threadIdx.x;
          const int cr = idx >> 3, sp = (idx & 7) * 2;
          if (cr < valid_cols && sp < valid_strips) {
            const int64_t r = R0 + 16 * sp;
            const int64_t g = r / seg_rows, lr = r - g * seg_rows;
            const int64_t trow = g * cols + C0 + cr;
            *reinterpret_cast<uint4*>(tcodes + trow * (seg_rows >> 1) + (lr >> 1)) =
                *reinterpret_cast<const uint4*>(&tc[cr][sp * 8]);
          }
        }
#pragma unroll
        for (int pass = 0; pass < kTileCols * 4 / kThreads; ++pass) {
          const int idx = pass * kThreads + threadIdx.x;
          const int cr = idx >> 2, sp = (idx & 3) * 4;
          if (cr < valid_cols && sp < valid_strips) {
            const int64_t r = R0 + 16 * sp;
            const int64_t g = r / seg_rows, lr = r - g * seg_rows;
            const int64_t trow = g * cols + C0 + cr;
            *reinterpret_cast<uint32_t*>(tscales + trow * (seg_rows >> 4) + (lr >> 4)) =
                *reinterpret_cast<const uint32_t*>(&ts[cr][sp]);
          }
        }
        return;
      }
#pragma unroll
      for (int pass = 0; pass < kTileCols * 16 / kThreads; ++pass) {
        const int idx = pass * kThreads + threadIdx.x;
        const int cr = idx >> 4, sp = idx & 15;
        if (cr < valid_cols && sp < valid_strips) {
          const int64_t r = R0 + 16 * sp;
          const int64_t g = r / seg_rows, lr = r - g * seg_rows;
          const int64_t trow = g * cols + C0 + cr;
          *reinterpret_cast<uint2*>(tcodes + trow * (seg_rows >> 1) + (lr >> 1)) =
              *reinterpret_cast<const uint2*>(&tc[cr][sp * 8]);
          tscales[trow * (seg_rows >> 4) + (lr >> 4)] = ts[cr][sp];
        }
      }
      return;
    }
#pragma unroll
    for (int pass = 0; pass < kTileCols * 16 / kThreads; ++pass) {
      const int idx = pass * kThreads + threadIdx.x;
      const int cr = idx >> 4, sp = idx & 15;
      if (cr < valid_cols && sp < valid_strips)
        *reinterpret_cast<uint2*>(tcodes + (C0 + cr) * (rows >> 1) + (R0 >> 1) + sp * 8) =
            *reinterpret_cast<const uint2*>(&tc[cr][sp * 8]);
    }
    if (threadIdx.x < kTileCols && threadIdx.x < valid_cols) {
      const int cr = threadIdx.x;
      uint8_t* dst = tscales + (C0 + cr) * (rows >> 4) + (R0 >> 4);
      if (valid_strips == 16 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(&ts[cr][0]);
      } else {
        for (int sp = 0; sp < valid_strips; ++sp) dst[sp] = ts[cr][sp];
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
constexpr int64_t kEncodeBlocks = 256 * 4;   // 1x16 encode: 4 workgroups per CU, waves loop over rows

template <typename TIn>
void amax_t(const void* x, int64_t rows, int64_t cols, int64_t ld, const int64_t* segments,
            int64_t nseg, float* out, int* parts, hipStream_t stream) {
  const int64_t vpr = cols * (int64_t)sizeof(TIn) / 16;
  if (segments) {
    hipLaunchKernelGGL(k_fill, dim3(1), dim3(256), 0, stream, out, nseg, 0.0f);
    const int grid = grid_for(rows * vpr, kThreads * 8, kMaxPartials);
    hipLaunchKernelGGL((k_amax_seg<TIn>), dim3(grid), dim3(kThreads), 0, stream, (const TIn*)x,
                       rows, vpr, ld, segments, nseg, out);
    *parts = 1;
  } else {
    const int grid = grid_for(rows * vpr, kThreads * 8, kMaxPartials);
    hipLaunchKernelGGL((k_amax_partial<TIn>), dim3(grid), dim3(kThreads), 0, stream,
                       (const TIn*)x, rows, vpr, ld, out);
    *parts = grid;
  }
}

}  // namespace

hipError_t launch_amax_parts(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                             const int64_t* segments, int64_t nseg, float* ws, int* parts,
                             hipStream_t stream) {
  if (fp32) amax_t<float>(x, rows, cols, ld, segments, nseg, ws, parts, stream);
  else amax_t<uint16_t>(x, rows, cols, ld, segments, nseg, ws, parts, stream);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t stream) {
  hipLaunchKernelGGL(k_fill, dim3(1), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

hipError_t launch_reduce_partials(const float* partials, int parts, float* out, hipStream_t stream,
                                  int count) {
  hipLaunchKernelGGL(k_reduce_partials, dim3(count), dim3(kThreads), 0, stream, partials, parts, out);
  return hipGetLastError();
}

template <typename TIn, bool SR, bool SEG>
static void encode_1x16_t(const void* x, int64_t rows, int64_t cols, int64_t ld, uint64_t seed,
                          uint64_t offset, const int64_t* segments, int64_t nseg,
                          const float* amax, int parts, QuantOut out, hipStream_t stream) {
  const int grid = grid_for(rows, kWavesPerBlock, kEncodeBlocks);
  hipLaunchKernelGGL((k_encode_1x16<TIn, SR, SEG>), dim3(grid), dim3(kThreads), 0, stream,
                     (const TIn*)x, rows, cols, ld, amax, parts, segments, nseg, out.codes,
                     out.scales, out.global_scale, seed, offset);
}

hipError_t launch_rot_amax_parts(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                                 uint16_t mask, float* partial, int* parts, hipStream_t stream) {
  const int grid = grid_for(rows, kWavesPerBlock, kMaxPartials);
  if (fp32) hipLaunchKernelGGL((k_amax_rot<float>), dim3(grid), dim3(kThreads), 0, stream, (const float*)x, rows, cols, ld, (uint32_t)mask, partial);
  else hipLaunchKernelGGL((k_amax_rot<uint16_t>), dim3(grid), dim3(kThreads), 0, stream, (const uint16_t*)x, rows, cols, ld, (uint32_t)mask, partial);
  *parts = grid;
  return hipGetLastError();
}

hipError_t launch_encode_rot(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld, uint16_t mask,
                             bool sr, uint64_t seed, uint64_t offset, const float* amax, int parts,
                             QuantOut out, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int grid = grid_for(rows, kWavesPerBlock, kEncodeBlocks);
#define NVFP4_ER(T, S) hipLaunchKernelGGL((k_encode_1x16<T, S, false, true>), dim3(grid), dim3(kThreads), 0, stream, \
                                          (const T*)x, rows, cols, ld, amax, parts, nullptr, 1, out.codes,        \
                                          out.scales, out.global_scale, seed, offset, (uint32_t)mask)
  if (fp32) { if (sr) NVFP4_ER(float, true); else NVFP4_ER(float, false); }
  else      { if (sr) NVFP4_ER(uint16_t, true); else NVFP4_ER(uint16_t, false); }
#undef NVFP4_ER
  return hipGetLastError();
}

// A contiguous tensor (ld == cols) is a flat run of blocks: codes, scales and the blocks'
// stochastic-rounding counters (row * cols/16 + col/16) all follow the flat order. The encode
// kernels give each wave one row per chunk of 64 * U blocks, so rows shorter than a chunk, or
// not a multiple of it, leave lanes idle; such a tensor is encoded as rows of exactly one chunk
// (4096 BF16 or 2048 FP32 elements) when its size allows, with identical output.
static void flatten_rows(bool fp32, int64_t& rows, int64_t& cols, int64_t& ld) {
  const int64_t L = fp32 ? 2048 : 4096;
  if (ld == cols && cols % L != 0 && (rows * cols) % L == 0) {
    rows = rows * cols / L;
    cols = ld = L;
  }
}

hipError_t launch_encode_mx(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                            bool sr, uint64_t seed, uint64_t offset, uint8_t* codes,
                            uint8_t* scales, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  // No flattening into chunk-wide rows (as the NVFP4 encode does): a scale's place in the
  // K-step layout depends on its true row and block (laying the rows end to end and mapping
  // each half back to its row measured no faster on [8192, 5120] and [8192, 20480] BF16).
  const int grid = grid_for(rows, kWavesPerBlock, kEncodeBlocks);
#define NVFP4_MX(T, S) hipLaunchKernelGGL((k_encode_mx<T, S>), dim3(grid), dim3(kThreads), 0, stream, \
                                          (const T*)x, rows, cols, ld, codes, scales, seed, offset)
  if (fp32) { if (sr) NVFP4_MX(float, true); else NVFP4_MX(float, false); }
  else      { if (sr) NVFP4_MX(uint16_t, true); else NVFP4_MX(uint16_t, false); }
#undef NVFP4_MX
  return hipGetLastError();
}

hipError_t launch_encode_1x16(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                              bool sr, uint64_t seed, uint64_t offset,
                              const int64_t* segments, int64_t nseg, const float* amax, int parts,
                              QuantOut out, hipStream_t stream) {
  const bool seg = segments != nullptr;
  if (!seg) flatten_rows(fp32, rows, cols, ld);
#define NVFP4_E1(T, S, G) encode_1x16_t<T, S, G>(x, rows, cols, ld, seed, offset, segments, nseg, amax, parts, out, stream)
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
                           const int64_t* segments, int64_t nseg, const float* amax, int parts,
                           QuantOut out, const QuantOut* out_t, hipStream_t stream) {
  const int64_t tiles = ((rows + kTileRows - 1) / kTileRows) * ((cols + kTileCols - 1) / kTileCols);
  if (tiles == 0) return;
  hipLaunchKernelGGL((k_encode_16x16<TIn, SEG, TRANS>), dim3((unsigned)tiles), dim3(kThreads), 0,
                     stream, (const TIn*)x, rows, cols, ld, amax, parts, segments, nseg,
                     out.codes, out.scales, out.global_scale, TRANS ? out_t->codes : nullptr,
                     TRANS ? out_t->scales : nullptr, TRANS ? out_t->global_scale : nullptr,
                     rows / (nseg > 0 ? nseg : 1));
}

hipError_t launch_encode_16x16(const void* x, bool fp32, int64_t rows, int64_t cols, int64_t ld,
                               const int64_t* segments, int64_t nseg, const float* amax, int parts,
                               QuantOut out, const QuantOut* out_t, hipStream_t stream) {
  const bool seg = segments != nullptr;
  const bool tr = out_t != nullptr;
  if (rows == 0) {
    // nothing to encode; the tensor scales of an empty tensor are 1
    hipLaunchKernelGGL(k_fill, dim3(1), dim3(256), 0, stream, out.global_scale, nseg, 1.0f);
    if (tr) hipLaunchKernelGGL(k_fill, dim3(1), dim3(256), 0, stream, out_t->global_scale, nseg, 1.0f);
    return hipGetLastError();
  }
#define NVFP4_E2(T, G, R) encode_16x16_t<T, G, R>(x, rows, cols, ld, segments, nseg, amax, parts, out, out_t, stream)
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
