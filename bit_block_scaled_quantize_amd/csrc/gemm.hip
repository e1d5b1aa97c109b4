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
// feeds the FP16 matrix cores (FP32 accumulate). The per-tensor scales multiply the
// accumulator in the epilogue. gfx950's native FP4 MFMA takes power-of-two scales per 32
// elements, which cannot express an E4M3 scale per 16 elements, so the FP16 path is the one
// used.
//
// Since the K order inside a dot product is free as long as A and B agree, every lane holds
// one contiguous run of codes of its row per K step and feeds consecutive octets of it to
// consecutive MFMAs.
//
// Two kernels:
//  * main (K % 64 == 0, every shape of the workloads): v_mfma_f32_32x32x16_f16; a workgroup of
//    4 waves (2 x 2) owns a 256 x 256 output tile, each wave 128 x 128 (4 x 4 MFMA tiles, 256
//    FP32 accumulators per lane in AGPRs). Per 128-wide K step the workgroup's FP4 panels
//    (2 x 16 KB) and scale bytes (2 x 2 KB) go straight from global memory into LDS with
//    buffer-to-LDS DMA, three stages deep, so no registers are spent on staging. Buffer bounds
//    make rows past the end of an operand read as zero. The grouped (MoE) GEMM uses the same
//    tile code with two narrower shapes for ragged edges: 256 x 64 (waves stacked 4 x 1) for a
//    last column at most 64 wide, 128 x 256 (1 x 4) for a group's last slot of at most 128
//    rows.
//  * general (any K % 16 == 0): v_mfma_f32_16x16x32_f16, 128 x 128 tiles, each wave 64 x 64,
//    operands loaded straight into registers one K step ahead.
// In both, scale bytes at or past K are forced to 0, which zeroes whatever codes sit in a
// partial last step.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kThreads = 256;
constexpr int kStepK = 128;

// FP16 pair (S * 2^-8, S * 2^-8) from an E4M3 code: the code shifted into the FP16 exponent
// and mantissa fields reads as S * 2^-8 for every code, subnormal ones included.
__device__ __forceinline__ half2v scale_pair(uint32_t s) {
  return __builtin_bit_cast(half2v, (s << 7) | (s << 23));
}

// 8 codes (one 32-bit word) -> 8 FP16 values e2m1 * S.
__device__ __forceinline__ half8 decode8(uint32_t codes, half2v s2) {
  const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0) * s2;
  const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1) * s2;
  const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2) * s2;
  const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3) * s2;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ uint32_t word(const v4u32& v, int t) {
  return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w;
}

// Scale-byte mask for the 32-element run starting at element k: bytes at or past K -> 0.
__device__ __forceinline__ uint32_t k_mask(int64_t K, int64_t k) {
  return (k < K ? 0xFFu : 0u) | (k + 16 < K ? 0xFF00u : 0u);
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

// Group g and rows [m0, m1) of m-tile slot `slot_m` for tiles of height bm; false past the
// last slot. The whole workgroup (256 threads, all of which must call it) searches: thread q
// counts the slots of group c + q, a workgroup prefix sum over those counts brackets slot_m.
// Offsets are clamped to [0, total_m] (a malformed table gives unspecified rows, never an
// access outside A or D).
__device__ __forceinline__ bool group_of(int64_t G, const int64_t* __restrict__ off, int64_t total_m,
                                         int64_t bm, int64_t slot_m, int64_t& g, int64_t& m0,
                                         int64_t& m1) {
  __shared__ int wsum[4];
  __shared__ int64_t found[3];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) found[0] = -1;
  int base = 0;                                   // slots of the groups before this chunk
  for (int64_t c = 0; c < G; c += 256) {
    const int64_t q = c + threadIdx.x;
    int64_t lo = 0, hi = 0;
    int t = 0;
    if (q < G) {
      lo = off[q];
      lo = lo < 0 ? 0 : (lo > total_m ? total_m : lo);
      hi = off[q + 1];
      hi = hi < lo ? lo : (hi > total_m ? total_m : hi);
      t = (int)((hi - lo + bm - 1) / bm);
    }
    int x = t;                                    // inclusive scan within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = base;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int incl = before + x, excl = incl - t;
    if (t > 0 && slot_m >= excl && slot_m < incl) {
      found[0] = q;
      found[1] = lo + (slot_m - excl) * bm;
      found[2] = found[1] + bm < hi ? found[1] + bm : hi;
    }
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    if (found[0] >= 0) break;                     // the same for every thread after the barrier
  }
  g = found[0];
  m0 = found[1];
  m1 = found[2];
  return g >= 0;
}

// Rows [lo, hi) of group g (offsets clamped as group_of clamps them) in 256-row slots: `full`
// slots of 256 rows (the last of them cut at hi when more than 128 rows remain for it) and, when
// 1..128 rows remain, one short slot, which the 128 x 256 tiles compute.
__device__ __forceinline__ void group_slots(const int64_t* __restrict__ off, int64_t g, int64_t total_m,
                                            int64_t& lo, int64_t& hi, int& full, int& shrt) {
  lo = off[g];
  lo = lo < 0 ? 0 : (lo > total_m ? total_m : lo);
  hi = off[g + 1];
  hi = hi < lo ? lo : (hi > total_m ? total_m : hi);
  const int64_t m = hi - lo, rem = m % 256;
  full = (int)(m / 256) + (rem > 128 ? 1 : 0);
  shrt = rem > 0 && rem <= 128 ? 1 : 0;
}

// Tile j of XCD xcd in the grouped GEMM with 256-row slots: group g, rows [m0, m1) and column
// tile tn; false past the XCD's tiles. Full-height slots are numbered over all groups in group
// order, short slots likewise (F and Sh of them), and the two numberings are merged into one
// slot order with the short slots spread evenly: position r (of T = F + Sh) is short iff
// floor((r + 1) Sh / T) > floor(r Sh / T), and is then short slot floor(r Sh / T), else full
// slot r - floor(r Sh / T). A short slot costs about 0.6 of a full one and short slots cluster
// where the groups are small, so giving each XCD equal shares of one slot numbering left one XCD
// with 15% more work than another on a Zipf-routed expert layer, and whole slots per XCD one
// with a slot more than the rest. XCD x instead takes an equal run of the tiles before column
// cols_main in merged slot order ([L x / 8, L (x + 1) / 8) of L = T cols_main, slot by slot, the
// same mix of both kinds everywhere), then, when cols_main < tiles_n, the last column tiles of
// the merged slots [T x / 8, T (x + 1) / 8) (narrowest last, to fill the gaps at the end; by
// then a slot's A panel has long left the XCD's L2 wherever it ran). The whole workgroup (all
// 256 threads) calls it: thread q walks groups [q p, q p + p), p = ceil(G / 256), twice (the
// offsets come from the cache the second time), with one workgroup scan between.
__device__ __forceinline__ bool grouped_slot(int64_t G, const int64_t* __restrict__ off, int64_t total_m,
                                             int64_t xcd, int64_t j, int64_t cols_main, int64_t tiles_n,
                                             int64_t& g, int64_t& m0, int64_t& m1, int64_t& tn) {
  __shared__ int wsum[2][4];
  __shared__ int64_t found[3];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t per = (G + 255) / 256;
  const int64_t g0 = (int64_t)threadIdx.x * per < G ? (int64_t)threadIdx.x * per : G;
  const int64_t g1 = g0 + per < G ? g0 + per : G;
  int nf = 0, ns = 0;
  for (int64_t q = g0; q < g1; ++q) {
    int64_t lo, hi;
    int f, sh;
    group_slots(off, q, total_m, lo, hi, f, sh);
    nf += f;
    ns += sh;
  }
  int cf = nf, cs = ns;                           // inclusive scans within the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int yf = __shfl_up(cf, d), ys = __shfl_up(cs, d);
    if (lane >= d) {
      cf += yf;
      cs += ys;
    }
  }
  if (lane == 63) {
    wsum[0][wave] = cf;
    wsum[1][wave] = cs;
  }
  __syncthreads();
  int64_t bf = cf - nf, bs = cs - ns, F = 0, Sh = 0;
  for (int w = 0; w < 4; ++w) {
    if (w < wave) {
      bf += wsum[0][w];
      bs += wsum[1][w];
    }
    F += wsum[0][w];
    Sh += wsum[1][w];
  }
  const int64_t T = F + Sh, L = T * cols_main;
  const int64_t la = L * xcd / 8, nl = L * (xcd + 1) / 8 - la;
  const int64_t ta = T * xcd / 8, nt = cols_main < tiles_n ? T * (xcd + 1) / 8 - ta : 0;
  int64_t r;                                      // merged slot position
  if (j < nl) {
    r = (la + j) / cols_main;
    tn = (la + j) % cols_main;
  } else if (j < nl + nt) {
    r = ta + (j - nl);
    tn = tiles_n - 1;
  } else {
    return false;                                 // uniform over the workgroup
  }
  const int64_t before = r * Sh / T;              // short slots at merged positions < r
  const bool is_short = (r + 1) * Sh / T > before;
  const int64_t idx = is_short ? before : r - before;
  // the one thread whose groups hold slot idx of its kind finds the group and its rows
  const int64_t base = is_short ? bs : bf, cnt = is_short ? ns : nf;
  if (idx >= base && idx < base + cnt) {
    int64_t run = base;
    for (int64_t q = g0; q < g1; ++q) {
      int64_t lo, hi;
      int f, sh;
      group_slots(off, q, total_m, lo, hi, f, sh);
      const int c = is_short ? sh : f;
      if (idx < run + c) {
        const int64_t r0 = lo + 256 * (is_short ? (int64_t)f : idx - run);
        found[0] = q;
        found[1] = r0;
        found[2] = r0 + 256 < hi ? r0 + 256 : hi;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  g = found[0];
  m0 = found[1];
  m1 = found[2];
  return true;
}

struct Operand {
  const uint8_t* codes;   // [rows, K/2]
  const uint8_t* scales;  // [rows, K/16]
  int64_t rows;           // rows addressable through this operand
};

// =========================================================================================
// main kernel: 256 x 256 tiles, 32x32x16 MFMA, LDS DMA staging (K % 64 == 0)
// =========================================================================================
// In v_mfma_f32_32x32x16_f16 lane l supplies row (l % 32) of A (column of B) and 8 K-values;
// lane half h = l / 32 picks which 8. Per 128-wide K step each lane therefore owns one
// contiguous 64-code run (32 bytes, 4 scale blocks = one aligned scale dword) of its row,
// bytes [32h, 32h + 32) of the step, and feeds its 8 octets to 8 consecutive MFMAs.
// Output of the linear-layer entry point (nvfp4_gemm_ex): FP32, FP32 added to what D holds
// (the weight gradient accumulating into an FP32 main gradient), or BF16 (the activations and
// activation gradients passed on in 16-bit), with the maximum |stored value| folded into
// `amax` (the tensor amax the next quantization of D needs, so that quantization is one pass).
// artiverse.ca "NVIDIA's 4-bit floating point pushes AI training limits": only the GEMMs run
// in 4-bit, the layer's other tensors in higher precision.
enum OutKind : int { kOutF32 = 0, kOutF32Add = 1, kOutBF16 = 2 };

struct ExtOut {
  void* d;          // output, row stride ldd elements
  int64_t ldd;
  float* part;      // a K-split tile's partial sums (tile-local, FP32), else null
  float* amax;      // device float or null
};

// The tile a persistent workgroup computes next (same operands and tile shape): its first
// DMA stages are issued before this tile's epilogue, so their latency passes under the stores.
struct TileNext {
  bool valid;
  int64_t m0, n0, k_begin, k_end;
};

// BF16 bits of v and w rounded to nearest, ties to even (low and high half; one
// v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_rn_pair(float v, float w) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f32{v, w}, bf16x2));
}
__device__ __forceinline__ uint32_t bf16_rn_bits(float v) { return bf16_rn_pair(v, 0.0f) & 0xFFFFu; }

// Stores v as output element (row, col); returns |stored value|.
template <int KIND>
__device__ __forceinline__ float put_out(void* d, int64_t ldd, int64_t row, int64_t col, float v) {
  if constexpr (KIND == kOutBF16) {
    const uint32_t b = bf16_rn_bits(v);
    __builtin_nontemporal_store((uint16_t)b, static_cast<uint16_t*>(d) + row * ldd + col);
    return fabsf(__uint_as_float(b << 16));
  } else if constexpr (KIND == kOutF32Add) {
    float* p = static_cast<float*>(d) + row * ldd + col;
    const float sum = *p + v;
    *p = sum;
    return fabsf(sum);
  } else {
    __builtin_nontemporal_store(v, static_cast<float*>(d) + row * ldd + col);
    return fabsf(v);
  }
}

// Workgroup maximum of every thread's mx into *amax (one atomic; all threads must call).
__device__ __forceinline__ void group_amax(float mx, float* amax) {
  __shared__ float red[kThreads / 64];
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, red[w]);
    atomic_max_nonneg(amax, m);
  }
}

namespace big {
constexpr int kFragBytes = 32 * 64;                           // 32 rows x 128 codes
constexpr int kFragScaleBytes = 32 * 8;                       // 32 rows x 8 scale bytes
constexpr int kStages = 3;                                    // DMA runs two K steps ahead

// Tile shape: 4 waves in a WM x WN grid, each wave FM x FN MFMA tiles of 32 x 32. A
// "fragment" is 32 rows of A or B for one K step; wave w moves fragments w, w + 4, w + 8, ...
// of the step (three DMA operations each: two 1 KB code halves and the scale dwords), every
// wave the same number of operations (padded with out-of-range ones).
template <int FM, int FN, int WM, int WN>
struct Cfg {
  static_assert(WM * WN == 4, "four waves");
  static constexpr int kFragsM = FM, kFragsN = FN, kWavesM = WM, kWavesN = WN;
  static constexpr int kWaveM = 32 * FM, kWaveN = 32 * FN;
  static constexpr int kBlockM = WM * kWaveM, kBlockN = WN * kWaveN;
  static constexpr int kFragsA = kBlockM / 32;
  static constexpr int kPanelFrags = kFragsA + kBlockN / 32;
  static_assert(kFragsA % 4 == 0, "A fragments of a wave's i-th DMA slot are A for every wave");
  static constexpr int kCodeBytes = kPanelFrags * kFragBytes;
  static constexpr int kStageBytes = kCodeBytes + kPanelFrags * kFragScaleBytes;
  static constexpr int kFragsPerWave = (kPanelFrags + 3) / 4;
  static constexpr int kLdsBytes = kStages * kStageBytes + (kPanelFrags % 4 ? 1024 : 0);   // + pad
  static constexpr int kDmaPerWaveStep = 3 * kFragsPerWave;
};
using Full = Cfg<4, 4, 2, 2>;     // 256 x 256: 16 fragments, 12 DMA operations per wave, 108 KB
using NTail = Cfg<2, 2, 4, 1>;    // 256 x 64 (a last column tile at most 64 wide)
using MTail = Cfg<4, 2, 1, 4>;    // 128 x 256 (a group's last row slot at most 128 high)
using NHalf = Cfg<4, 2, 2, 2>;    // 256 x 128 (a last column tile at most 128 wide)
constexpr int kBlockM = Full::kBlockM, kBlockN = Full::kBlockN;
constexpr int kLdsBytes = Full::kLdsBytes;
static_assert(kBlockM == 256 && MTail::kBlockM == 128, "the slots of grouped_slot");
static_assert(NTail::kLdsBytes <= kLdsBytes && MTail::kLdsBytes <= kLdsBytes &&
              NHalf::kLdsBytes <= kLdsBytes, "LDS");

// s_waitcnt immediate (gfx9 encoding): vmcnt(vm) lgkmcnt(lgkm), expcnt not waited on.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | ((lgkm & 0xF) << 8);
}
static_assert(waitcnt_imm(24, 15) == 0x4F78 && waitcnt_imm(12, 0) == 0x007C &&
              waitcnt_imm(0, 15) == 0x0F70, "waitcnt encoding");
}  // namespace big

typedef float float16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// One output tile of shape C summing over the elements [k_begin, k_end) of the contraction
// (both multiples of 64; K is the operands' row length; a k_begin that is not a multiple of
// 128 needs FIRST_HALF). With `accumulate` (a K-split tile) the scaled partial sums are added
// to D with hardware float atomics (D pre-zeroed by the caller), else stored. EXT: the output
// goes to `ext` as KIND instead, a K-split tile's partial sums to ext.part.
template <class C, bool FIRST_HALF = false, int KIND = kOutF32, bool EXT = false>
__device__ __forceinline__ void gemm_tile_big(Operand A, Operand B, int64_t m0, int64_t m1,
                                              int64_t n0, int64_t n1, int64_t K, int64_t k_begin,
                                              int64_t k_end, bool accumulate, float alpha,
                                              float* __restrict__ D, int64_t ldd, uint8_t* lds,
                                              const ExtOut ext = ExtOut{nullptr, 0, nullptr, nullptr},
                                              const TileNext nx = TileNext{false, 0, 0, 0, 0},
                                              bool prefetched = false) {
  using big::kFragBytes;
  using big::kFragScaleBytes;
  using big::kStages;
  constexpr int kFragsM = C::kFragsM, kFragsN = C::kFragsN, kFragsA = C::kFragsA;
  constexpr int kWaveM = C::kWaveM, kWaveN = C::kWaveN;
  constexpr int kPanelFrags = C::kPanelFrags, kCodeBytes = C::kCodeBytes;
  constexpr int kStageBytes = C::kStageBytes, kDmaPerWaveStep = C::kDmaPerWaveStep;
  // the lane index counted by the hardware (mbcnt) rather than taken from the thread index: in
  // a loop over tiles that would keep the thread index, and values derived from it, live
  // through the main loop, which needs every vector register
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  // the wave index is uniform: held in a scalar register, everything derived from it (DMA
  // rows, LDS addresses) is scalar arithmetic
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 31, h = lane >> 5;
  const int wm = wave / C::kWavesN, wn = wave % C::kWavesN;
  const uint32_t rs_codes = (uint32_t)(K >> 1), rs_scales = (uint32_t)(K >> 4);
  constexpr uint32_t kBeyond = 0x80000000u;                  // > any 31-bit buffer size
  // K steps (128 elements) as uniform 32-bit values, so the step loop and the per-step DMA
  // offsets stay in scalar registers
  const int s0 = __builtin_amdgcn_readfirstlane((int)(k_begin / kStepK));
  const int s1 = __builtin_amdgcn_readfirstlane((int)((k_end + kStepK - 1) / kStepK));

  const __amdgpu_buffer_rsrc_t a_codes = make_rsrc(A.codes, A.rows * (K >> 1));
  const __amdgpu_buffer_rsrc_t b_codes = make_rsrc(B.codes, B.rows * (K >> 1));
  const __amdgpu_buffer_rsrc_t a_scales = make_rsrc(A.scales, A.rows * (K >> 4));
  const __amdgpu_buffer_rsrc_t b_scales = make_rsrc(B.scales, B.rows * (K >> 4));

  // DMA: this wave moves fragments f = wave + 4*i (A fragments f < kFragsA, then B), two 1 KB
  // halves each; lane (r, h) of half q carries row 32*f' + r (f' = f, or f - kFragsA for B),
  // bytes [32h + 16q, 32h + 16q + 16) of the step -> LDS f*2 KB + q*1 KB + lane*16. Its scale
  // dword (bytes [4h, 4h + 4) of the row's 8 scale bytes of the step) -> LDS scales + f*256 +
  // lane*4. Fragments past the panel (f >= kPanelFrags, only in the last slot) are padding.
  // Offsets split into the lane's part (row r of the fragment, half h; a vector register) and
  // the fragment's and step's part (uniform, scalar), so each DMA costs one vector add.
  const uint32_t lane_codes = (uint32_t)r * rs_codes + (uint32_t)(h * 32);
  const uint32_t lane_scales = (uint32_t)r * rs_scales + (uint32_t)(h * 4);
  // Scale blocks outside [k_begin, k_end). With both ends multiples of 64 a lane's scale dword
  // of a step (4 blocks) lies wholly inside or outside the range; only a first half step
  // (k_begin % 128 == 64: half 0 lies before the range) and a last half step (k_end % 128 ==
  // 64: half 1 lies past it, in the next group or the next row) have lanes outside. Their
  // offset is pushed out of range so the DMA delivers zero scales, which zero whatever codes
  // they meet. (When the step is not live either, the two pushes wrap to an in-range offset
  // of a dummy load whose LDS buffer is never read.)
  // A tile's DMA parameters (uniform): its first A and B rows for this wave, its step range
  // end and its half steps.
  struct DmaTile { uint32_t row_a, row_b; int s1, first_half_step, last_half_step; };
  auto dma_tile = [&](int64_t tm0, int64_t tn0, int64_t kb, int64_t ke) {
    DmaTile t;
    t.row_a = __builtin_amdgcn_readfirstlane((uint32_t)(tm0 + wave * 32));
    t.row_b = __builtin_amdgcn_readfirstlane((uint32_t)(tn0 + wave * 32));
    t.s1 = __builtin_amdgcn_readfirstlane((int)((ke + kStepK - 1) / kStepK));
    t.first_half_step = __builtin_amdgcn_readfirstlane((kb % kStepK) ? (int)(kb / kStepK) : -1);
    t.last_half_step = __builtin_amdgcn_readfirstlane((ke % kStepK) ? (int)(ke / kStepK) : -1);
    return t;
  };
  const DmaTile cur = dma_tile(m0, n0, k_begin, k_end);

  // One of the wave's DMA operations of a step: part p = 3*i + q moves half q (q < 2) of
  // fragment wave + 4*i, or (q == 2) its scale dwords. Steps past the last one are issued too
  // (the pipeline then has no branches and always the same number of operations in flight)
  // with an offset beyond every buffer's range, which the buffer unit answers with zeros
  // without touching memory; their LDS buffers are never read. Padding operations are issued
  // the same way (out of range) into a 1 KB LDS area behind the stages that nothing reads.
  auto issue_dma_part_of = [&](const DmaTile& t, int step, int buf, int p) {
    uint8_t* base = lds + buf * kStageBytes;
    const int i = p / 3, q = p % 3;
    const bool is_a = 4 * i < kFragsA;                        // same for every wave
    const int f = wave + 4 * i;
    const int ib = is_a ? i : i - kFragsA / 4;                // slot among the wave's A or B
    const bool real = 4 * i + 3 < kPanelFrags || f < kPanelFrags;
    const bool live = step < t.s1 && real;
    const uint32_t row = (is_a ? t.row_a : t.row_b) + 128u * (uint32_t)ib;   // first row, uniform
    uint8_t* pad = lds + kStages * kStageBytes;
    if (q < 2) {
      const uint32_t su = row * rs_codes + (uint32_t)(step * (kStepK / 2)) + 16u * q;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? a_codes : b_codes,
                                               (lds_ptr_t)(real ? base + f * kFragBytes + q * 1024 : pad),
                                               16, lane_codes + (live ? su : kBeyond), 0, 0, 0);
    } else {
      const uint32_t su = row * rs_scales + (uint32_t)(step * (kStepK / 16));
      uint32_t lsc;
      if constexpr (FIRST_HALF) {
        const uint32_t push_h0 = step == t.first_half_step ? kBeyond : 0u;   // uniform
        const uint32_t push_h1 = step == t.last_half_step ? kBeyond : 0u;
        lsc = lane_scales + (h ? push_h1 : push_h0);
      } else {
        lsc = lane_scales + (step == t.last_half_step ? (h ? kBeyond : 0u) : 0u);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? a_scales : b_scales,
                                               (lds_ptr_t)(real ? base + kCodeBytes + f * kFragScaleBytes : pad),
                                               4, lsc + (live ? su : kBeyond), 0, 0, 0);
    }
  };
  auto issue_dma_part = [&](int step, int buf, int p) { issue_dma_part_of(cur, step, buf, p); };
  auto issue_dma = [&](int step, int buf) {
#pragma unroll
    for (int p = 0; p < kDmaPerWaveStep; ++p) issue_dma_part(step, buf, p);
  };

  float16v acc[kFragsM][kFragsN];
#pragma unroll
  for (int i = 0; i < kFragsM; ++i)
#pragma unroll
    for (int j = 0; j < kFragsN; ++j) acc[i][j] = float16v{};

  // Pipeline. DMA runs up to 3 K steps ahead (3 LDS buffers). A lane's 64-code run of a step
  // sits in two register halves: half 0 (octets 0-3) and half 1 (octets 4-7). Half 1 of step
  // s is read from LDS when step s starts and lands while octets 0-3 compute; at octet 4 the
  // wave meets the next step's barrier and refills half 0 (free by then) with step s+1, so
  // no LDS latency sits between steps and the barrier wait overlaps in-flight MFMAs. Before
  // that barrier each wave waits for its own DMA of step s+1 and for its LDS reads of step s,
  // whose buffer the DMA of step s+3 refills right after it.
  static_assert(kStages == 3, "waitcnt immediates below");
  constexpr int kWaitStep0 = big::waitcnt_imm(2 * kDmaPerWaveStep, 15);   // 2 steps may fly
  constexpr int kWaitNext = big::waitcnt_imm(kDmaPerWaveStep, 0);         // 1 step, no LDS
  constexpr int kWaitAll = big::waitcnt_imm(0, 15);
  auto barrier = [] {
    // plain s_barrier: a fence would also wait for the DMA still in flight; the empty asm
    // statements keep the compiler from moving LDS accesses across it
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  v4u32 ar0[kFragsM], ar1[kFragsM], br0[kFragsN], br1[kFragsN];
  uint32_t sa[kFragsM], sb[kFragsN];
  auto read_half = [&](int b, int q, v4u32 (&ra)[kFragsM], v4u32 (&rb)[kFragsN]) {
    const uint8_t* cur = lds + b * kStageBytes + q * 1024 + lane * 16;
#pragma unroll
    for (int j = 0; j < kFragsN; ++j)
      rb[j] = *reinterpret_cast<const v4u32*>(cur + (kFragsA + wn * kFragsN + j) * kFragBytes);
#pragma unroll
    for (int i = 0; i < kFragsM; ++i)
      ra[i] = *reinterpret_cast<const v4u32*>(cur + (wm * kFragsM + i) * kFragBytes);
  };
  // raw scale dwords (blocks past K arrive as zeros from the DMA); they need not land before
  // the step that uses them
  auto read_scales = [&](int b) {
    const uint8_t* cur = lds + b * kStageBytes + kCodeBytes + lane * 4;
#pragma unroll
    for (int j = 0; j < kFragsN; ++j)
      sb[j] = *reinterpret_cast<const uint32_t*>(cur + (kFragsA + wn * kFragsN + j) * kFragScaleBytes);
#pragma unroll
    for (int i = 0; i < kFragsM; ++i)
      sa[i] = *reinterpret_cast<const uint32_t*>(cur + (wm * kFragsM + i) * kFragScaleBytes);
  };

  if (prefetched) {
    // the stages came with the previous tile's epilogue: wait for them (and its stores)
    __builtin_amdgcn_s_waitcnt(kWaitAll);
  } else {
#pragma unroll
    for (int p = 0; p < kStages; ++p) issue_dma(s0 + p, p);
    __builtin_amdgcn_s_waitcnt(kWaitStep0);                   // step 0 landed
  }
  barrier();
  read_half(0, 0, ar0, br0);
  read_scales(0);

  // FP16 scale pair (S * 2^-8 twice) of block q of a scale dword:
  // (b << 7) | (b << 23) = b * 0x00800080
  auto pair = [](uint32_t sc, int q) {
    return __builtin_bit_cast(half2v, ((sc >> (8 * q)) & 0xFFu) * 0x00800080u);
  };

  // 8 * kFragsM phases per step (t = K octet, i = A fragment), each kFragsN MFMAs. Decodes run
  // one phase ahead: while phase (t, i) issues its MFMAs, the A fragment of the next phase and
  // B fragments i, i + kFragsM, ... of octet t+1 are decoded, so every MFMA finds its operands
  // ready and the vector
  // ALU works under the matrix core; the last octet already decodes octet 0 of the next step
  // (its half 0 and scales arrive at octet 4), so steps join without a gap. sched_barrier
  // keeps the compiler from regrouping phases.
  half8 bv[kFragsN], bn[kFragsN], av;
#pragma unroll
  for (int j = 0; j < kFragsN; ++j) bv[j] = decode8(br0[j].x, pair(sb[j], 0));
  av = decode8(ar0[0].x, pair(sa[0], 0));

  int b_cur = 0;
  for (int s = s0; s < s1; ++s) {
    const int b_next = b_cur == kStages - 1 ? 0 : b_cur + 1;
    read_half(b_cur, 1, ar1, br1);

    half2v pa[kFragsM][4], pb[kFragsN][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int i = 0; i < kFragsM; ++i) pa[i][q] = pair(sa[i], q);
#pragma unroll
      for (int j = 0; j < kFragsN; ++j) pb[j][q] = pair(sb[j], q);
    }

    auto araw = [&](int i, int t) { return word(t < 4 ? ar0[i] : ar1[i], t & 3); };
    auto braw = [&](int j, int t) { return word(t < 4 ? br0[j] : br1[j], t & 3); };
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t == 4) {
        // unconditional (on the last step the reads fetch an unused buffer): with the block
        // behind a branch the compiler's wait analysis, merging the two paths, would make
        // the wave wait for these new reads before decoding data that has long landed.
        // Steps s+1 and s+2 are in flight here; wait for s+1.
        __builtin_amdgcn_s_waitcnt(kWaitNext);                  // step s+1 landed, LDS reads done
        barrier();
        read_half(b_next, 0, ar0, br0);                         // sa, sb now step s+1's
        read_scales(b_next);
      }
#pragma unroll
      for (int i = 0; i < kFragsM; ++i) {
        // the DMA of step s+3 refills the buffer step s was read from, spread over the phases
        // of octets 5-7 (one per phase for the 256 x 256 tile): a burst would stall the
        // wave's issue while its matrix
        // pipe runs dry, and the compiler orders each LDS-bound DMA after the wave's pending
        // LDS reads (it cannot tell the buffers apart), so the DMA waits one octet for the
        // reads issued at the barrier to land
        if (t >= 5) {
#pragma unroll
          for (int p = (t - 5) * kFragsM + i; p < kDmaPerWaveStep; p += 3 * kFragsM)
            issue_dma_part(s + 3, b_cur, p);
        }
        const int tn = i + 1 < kFragsM ? t : t + 1;           // next phase
        const int in_ = i + 1 < kFragsM ? i + 1 : 0;
        const half8 an = tn < 8 ? decode8(araw(in_, tn), pa[in_][tn >> 1])
                                : decode8(ar0[0].x, pair(sa[0], 0));
#pragma unroll
        for (int j = i; j < kFragsN; j += kFragsM)              // B fragment j of octet t+1
          bn[j] = t + 1 < 8 ? decode8(braw(j, t + 1), pb[j][(t + 1) >> 1])
                            : decode8(br0[j].x, pair(sb[j], 0));
#pragma unroll
        for (int j = 0; j < kFragsN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv[j], acc[i][j], 0, 0, 0);
        av = an;
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < kFragsN; ++j) bv[j] = bn[j];
    }
    b_cur = b_next;
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);                       // no DMA may outlive the tile
  if (nx.valid) {
    // every wave done with the stage buffers (LDS reads landed), then the next tile's first
    // stages into them; the next call waits for them instead of issuing its own
    __builtin_amdgcn_s_waitcnt(big::waitcnt_imm(0, 0));
    barrier();
    const DmaTile nt = dma_tile(nx.m0, nx.n0, nx.k_begin, nx.k_end);
    const int ns0 = __builtin_amdgcn_readfirstlane((int)(nx.k_begin / kStepK));
#pragma unroll
    for (int p = 0; p < kStages; ++p)
#pragma unroll
      for (int q = 0; q < kDmaPerWaveStep; ++q) issue_dma_part_of(nt, ns0 + p, p, q);
  }

  // D fragment layout (32 x 32): lane l holds column l % 32 and, for q = 0..15, row
  // 8*(q/4) + 4*(l/32) + q%4.
  float mx = 0.0f;
  // Plain FP32 and BF16 outputs, and FP32 D += tile without an amax output (not a K-split
  // tile's partial sums), go through a buffer resource from the tile's corner to its last
  // element in the output (row m1 - 1, column n1 - 1): stores and atomics to rows past m1 fall
  // outside it and the buffer unit drops them, columns past n1 get an offset beyond any range. An element's offset is the lane's column offset
  // (per j, a vector register) plus its row's offset (per i and q, uniform): no per-element
  // bounds test or 64-bit address arithmetic, which cost about 8 us per 256 x 256 tile with one
  // wave per SIMD. The maximum for the amax output counts only elements inside
  // the tile's bounds (a grouped tile's rows past m1 hold the next group's products). A row
  // pitch of at most 2^20 elements keeps every offset, pushed past the range or not, below 2^32.
  {
    constexpr int kES = (EXT && KIND == kOutBF16) ? 2 : 4;          // output element bytes
    // (D += tile without an amax output adds by float atomics, fire and forget; the FP32
    // outputs with an amax keep the path further below: with this one their kernels spill
    // registers, holding the loaded old values)
    constexpr bool kFast = !EXT || KIND == kOutBF16 || KIND == kOutF32Add;
    const int64_t ldo = EXT ? ext.ldd : ldd;
    const bool no_amax_add = !(EXT && KIND == kOutF32Add) || ext.amax == nullptr;
    if (kFast && !accumulate && no_amax_add && ldo <= (int64_t(1) << 20)) {
      uint8_t* const out = EXT ? static_cast<uint8_t*>(ext.d) : reinterpret_cast<uint8_t*>(D);
      const uint32_t ldb = (uint32_t)ldo * kES;
      // base and size made scalar: the compiler cannot see that they are uniform, and a
      // resource in vector registers makes it loop over the lanes for every access
      const uint64_t base = reinterpret_cast<uint64_t>(out + (m0 * ldo + n0) * kES);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
      const int64_t size = __builtin_amdgcn_readfirstlane((uint32_t)(((m1 - m0 - 1) * ldo + (n1 - n0)) * kES));
      const __amdgpu_buffer_rsrc_t dr =
          make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), size);
      uint32_t voff[kFragsN];
      bool cok[kFragsN];
#pragma unroll
      for (int j = 0; j < kFragsN; ++j) {
        const int cl = wn * kWaveN + 32 * j + r;                    // column within the tile
        cok[j] = n0 + cl < n1;
        voff[j] = cok[j] ? (uint32_t)(4 * h) * ldb + (uint32_t)cl * kES : kBeyond;
      }
      const int rlim = (int)(m1 - m0) - 4 * h;       // row (less the lane's 4h) inside iff below
      auto row_of = [&](int i, int q) { return wm * kWaveM + 32 * i + 8 * (q >> 2) + (q & 3); };
      auto take = [&](bool in, float v) {
        if constexpr (EXT) mx = fmaxf(mx, in ? fabsf(v) : 0.0f);
      };
      if constexpr (EXT && KIND == kOutBF16) {
        // rows q and q + 1 of the lane's column converted by one instruction
#pragma unroll
        for (int i = 0; i < kFragsM; ++i) {
#pragma unroll
          for (int q = 0; q < 16; q += 2) {
            const int ri = row_of(i, q);
#pragma unroll
            for (int j = 0; j < kFragsN; ++j) {
              const uint32_t b = bf16_rn_pair(acc[i][j][q] * alpha, acc[i][j][q + 1] * alpha);
              const uint32_t o = voff[j] + (uint32_t)ri * ldb;
              __builtin_amdgcn_raw_buffer_store_b16((uint16_t)b, dr, o, 0, 2);
              __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(b >> 16), dr, o + ldb, 0, 2);
              take(cok[j] && ri < rlim, __uint_as_float(b << 16));
              take(cok[j] && ri + 1 < rlim, __uint_as_float(b & 0xFFFF0000u));
            }
          }
        }
      } else if constexpr (EXT && KIND == kOutF32Add) {
        // D += tile: one float atomic add per element, done where the line lives (L2), so the
        // old values never come into registers and the epilogue does not wait for them
#pragma unroll
        for (int i = 0; i < kFragsM; ++i) {
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int ri = row_of(i, q);
#pragma unroll
            for (int j = 0; j < kFragsN; ++j)
              (void)__builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[i][j][q] * alpha, dr,
                                                                   voff[j] + (uint32_t)ri * ldb, 0, 0);
          }
        }
      } else {
        // FP32, non-temporal: D goes out to HBM while this compute-bound kernel runs instead of
        // sitting dirty in the caches and being written back during the next kernel
#pragma unroll
        for (int i = 0; i < kFragsM; ++i) {
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int ri = row_of(i, q);
#pragma unroll
            for (int j = 0; j < kFragsN; ++j)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][q] * alpha), dr,
                                                    voff[j] + (uint32_t)ri * ldb, 0, 2);
          }
        }
      }
      if constexpr (EXT) {
        if (ext.amax != nullptr) group_amax(mx, ext.amax);          // uniform
      }
      return;
    }
  }
  if constexpr (EXT && KIND == kOutF32Add) {
    if (!accumulate) {
      // D += tile: the old values of a row of fragments are all requested before any is
      // used, so the loads overlap instead of paying one round trip per element
      float* Df = static_cast<float*>(ext.d);
#pragma unroll
      for (int i = 0; i < kFragsM; ++i) {
        float old[kFragsN][16];
#pragma unroll
        for (int j = 0; j < kFragsN; ++j) {
          const int64_t col = n0 + wn * kWaveN + 32 * j + r;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int64_t row = m0 + wm * kWaveM + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
            old[j][q] = (row < m1 && col < n1) ? Df[row * ext.ldd + col] : 0.0f;
          }
        }
#pragma unroll
        for (int j = 0; j < kFragsN; ++j) {
          const int64_t col = n0 + wn * kWaveN + 32 * j + r;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int64_t row = m0 + wm * kWaveM + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
            if (row < m1 && col < n1) {
              const float sum = old[j][q] + acc[i][j][q] * alpha;
              Df[row * ext.ldd + col] = sum;
              mx = fmaxf(mx, fabsf(sum));
            }
          }
        }
      }
      if (ext.amax != nullptr) group_amax(mx, ext.amax);
      return;
    }
  }
  if constexpr (EXT && KIND == kOutBF16) {
    if (!accumulate) {
      // BF16: the lane's values q and q + 1 (rows row and row + 1) converted by one instruction
      uint16_t* Db = static_cast<uint16_t*>(ext.d);
#pragma unroll
      for (int i = 0; i < kFragsM; ++i) {
#pragma unroll
        for (int j = 0; j < kFragsN; ++j) {
          const int64_t col = n0 + wn * kWaveN + 32 * j + r;
          if (col >= n1) continue;
#pragma unroll
          for (int q = 0; q < 16; q += 2) {
            const int64_t row = m0 + wm * kWaveM + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
            const uint32_t b = bf16_rn_pair(acc[i][j][q] * alpha, acc[i][j][q + 1] * alpha);
            if (row < m1) {
              __builtin_nontemporal_store((uint16_t)b, Db + row * ext.ldd + col);
              mx = fmaxf(mx, fabsf(__uint_as_float(b << 16)));
            }
            if (row + 1 < m1) {
              __builtin_nontemporal_store((uint16_t)(b >> 16), Db + (row + 1) * ext.ldd + col);
              mx = fmaxf(mx, fabsf(__uint_as_float(b & 0xFFFF0000u)));
            }
          }
        }
      }
      if (ext.amax != nullptr) group_amax(mx, ext.amax);
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < kFragsM; ++i) {
#pragma unroll
    for (int j = 0; j < kFragsN; ++j) {
      const int64_t col = n0 + wn * kWaveN + 32 * j + r;
      if (col >= n1) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm * kWaveM + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
        if (row < m1) {
          const float v = acc[i][j][q] * alpha;
          // non-temporal: D goes out to HBM while this compute-bound kernel runs instead of
          // sitting dirty in the caches and being written back during the next kernel
          if constexpr (!EXT) {
            if (accumulate) unsafeAtomicAdd(&D[row * ldd + col], v);
            else __builtin_nontemporal_store(v, &D[row * ldd + col]);
          } else if (accumulate) {
            __builtin_nontemporal_store(v, &ext.part[(row - m0) * C::kBlockN + (col - n0)]);
          } else {
            mx = fmaxf(mx, put_out<KIND>(ext.d, ext.ldd, row, col, v));
          }
        }
      }
    }
  }
  if constexpr (EXT) {
    if (ext.amax != nullptr && !accumulate) group_amax(mx, ext.amax);   // uniform
  }
}

// Workgroup b (b < 4 rem) of the column quarters of the last rem tiles: its tile (counted from
// the first of them) and quarter. Each run of 32 consecutive workgroups takes 8 tiles with the
// four quarters of a tile 8 workgroups apart, so the four run on one XCD (workgroups are dealt
// to the 8 XCDs round robin) and read the tile's A panel through one L2; the last rem % 8
// tiles take the remaining workgroups in order.
__device__ __forceinline__ void quarter_of(int64_t b, int64_t rem, int64_t& tile, int64_t& quarter) {
  const int64_t whole = rem / 8 * 32;
  if (b < whole) {
    tile = b / 32 * 8 + b % 8;
    quarter = b % 32 / 8;
  } else {
    const int64_t r = rem % 8, c = b - whole;                  // r > 0 here
    tile = rem / 8 * 8 + c % r;
    quarter = c / r;
  }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_big(Operand A, const float* __restrict__ ag, Operand B, const float* __restrict__ bg,
                int64_t K, float* __restrict__ D, int64_t ldd, int64_t tail_first, int splits) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  using namespace big;
  const int64_t tiles_m = (A.rows + kBlockM - 1) / kBlockM;
  const int64_t tiles_n = (B.rows + kBlockN - 1) / kBlockN;
  const int64_t steps = (K + kStepK - 1) / kStepK;
  // splits < 0: workgroups past tail_first take the last tiles in quarters of 64 columns, all
  // of K (a last round of at most a quarter of the CUs then fills one round, with no atomics)
  if (splits < 0 && (int64_t)blockIdx.x >= tail_first) {
    int64_t tile, quarter;
    quarter_of((int64_t)blockIdx.x - tail_first, tiles_m * tiles_n - tail_first, tile, quarter);
    const int64_t t = tail_first + tile;
    int64_t tm, tn;
    tile_of(t, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = tm * kBlockM, n0 = tn * kBlockN + quarter * NTail::kBlockN;
    if (n0 >= B.rows) return;                        // a narrower last column tile
    const int64_t m1 = m0 + kBlockM < A.rows ? m0 + kBlockM : A.rows;
    const int64_t n1 = n0 + NTail::kBlockN < B.rows ? n0 + NTail::kBlockN : B.rows;
    gemm_tile_big<NTail>(A, B, m0, m1, n0, n1, K, 0, K, false, ag[0] * bg[0], D, ldd, lds_dyn);
    return;
  }
  // workgroups past tail_first share the last tiles, `splits` per tile, each over a K range
  int64_t t = blockIdx.x, s0 = 0, s1 = steps;
  if (t >= tail_first) {
    const int64_t part = (t - tail_first) % splits;
    t = tail_first + (t - tail_first) / splits;
    s0 = steps * part / splits;
    s1 = steps * (part + 1) / splits;
  }
  int64_t tm, tn;
  tile_of(t, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * kBlockM, n0 = tn * kBlockN;
  const int64_t m1 = m0 + kBlockM < A.rows ? m0 + kBlockM : A.rows;
  const int64_t n1 = n0 + kBlockN < B.rows ? n0 + kBlockN : B.rows;
  const int64_t k_end = s1 * kStepK < K ? s1 * kStepK : K;
  gemm_tile_big<Full>(A, B, m0, m1, n0, n1, K, s0 * kStepK, k_end, blockIdx.x >= tail_first,
                      ag[0] * bg[0], D, ldd, lds_dyn);
}

// Zeroes the D region of the K-split tiles tail_first, tail_first + 1, ... of k_gemm_big:
// workgroup b clears rows 16 * (b % kZeroParts) .. +15 of tile tail_first + b / kZeroParts, one
// 16-byte store per lane and row where the row stride and D allow it.
constexpr int kZeroParts = big::kBlockM / 16;

__global__ __launch_bounds__(kThreads) void k_zero_tiles(int64_t M, int64_t N, float* __restrict__ D,
                                                         int64_t ldd, int64_t tail_first, int vec) {
  using namespace big;
  const int64_t tiles_m = (M + kBlockM - 1) / kBlockM;
  const int64_t tiles_n = (N + kBlockN - 1) / kBlockN;
  int64_t tm, tn;
  tile_of(tail_first + blockIdx.x / kZeroParts, tiles_m, tiles_n, tm, tn);
  const int64_t r0 = tm * kBlockM + (blockIdx.x % kZeroParts) * 16;
  const int64_t c = tn * kBlockN + (threadIdx.x & 63) * 4;
#pragma unroll
  for (int i = 0; i < 16 / (kThreads / 64); ++i) {
    const int64_t r = r0 + (threadIdx.x >> 6) + i * (kThreads / 64);
    if (r >= M) break;
    float* p = D + r * ldd + c;
    if (vec && c + 3 < N) {
      *reinterpret_cast<float4*>(p) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (c + q < N) p[q] = 0.0f;
    }
  }
}

// k_gemm_big with the extended output: a split tile's two parts store their partial sums in
// the workspace, [split tile][part][256 x 256], and k_split_fixup finishes those tiles.
template <int KIND>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_big_ext(Operand A, const float* __restrict__ ag, Operand B, const float* __restrict__ bg,
                    int64_t K, void* D, int64_t ldd, float* amax, float* part, int64_t tail_first,
                    int splits) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  using namespace big;
  const int64_t tiles_m = (A.rows + kBlockM - 1) / kBlockM;
  const int64_t tiles_n = (B.rows + kBlockN - 1) / kBlockN;
  const int64_t steps = (K + kStepK - 1) / kStepK;
  if (splits < 0 && (int64_t)blockIdx.x >= tail_first) {         // column quarters, as k_gemm_big
    int64_t tile, quarter;
    quarter_of((int64_t)blockIdx.x - tail_first, tiles_m * tiles_n - tail_first, tile, quarter);
    const int64_t t = tail_first + tile;
    int64_t tm, tn;
    tile_of(t, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = tm * kBlockM, n0 = tn * kBlockN + quarter * NTail::kBlockN;
    if (n0 >= B.rows) return;                        // a narrower last column tile
    const int64_t m1 = m0 + kBlockM < A.rows ? m0 + kBlockM : A.rows;
    const int64_t n1 = n0 + NTail::kBlockN < B.rows ? n0 + NTail::kBlockN : B.rows;
    const ExtOut ext{D, ldd, nullptr, amax};
    gemm_tile_big<NTail, false, KIND, true>(A, B, m0, m1, n0, n1, K, 0, K, false, ag[0] * bg[0], nullptr,
                                            ldd, lds_dyn, ext);
    return;
  }
  int64_t t = blockIdx.x, s0 = 0, s1 = steps;
  const bool split = t >= tail_first;
  if (split) {
    const int64_t part_i = (t - tail_first) % splits;
    t = tail_first + (t - tail_first) / splits;
    s0 = steps * part_i / splits;
    s1 = steps * (part_i + 1) / splits;
  }
  int64_t tm, tn;
  tile_of(t, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * kBlockM, n0 = tn * kBlockN;
  const int64_t m1 = m0 + kBlockM < A.rows ? m0 + kBlockM : A.rows;
  const int64_t n1 = n0 + kBlockN < B.rows ? n0 + kBlockN : B.rows;
  const int64_t k_end = s1 * kStepK < K ? s1 * kStepK : K;
  const ExtOut ext{D, ldd, split ? part + (blockIdx.x - tail_first) * (int64_t)(kBlockM * kBlockN) : nullptr,
                   amax};
  gemm_tile_big<Full, false, KIND, true>(A, B, m0, m1, n0, n1, K, s0 * kStepK, k_end, split,
                                         ag[0] * bg[0], nullptr, ldd, lds_dyn, ext);
}

// Finishes the split tiles of k_gemm_big_ext: element = part 0 + part 1 (the lower K half
// first, so the result does not depend on which part ran first), stored as KIND. Workgroup b
// takes rows 16 * (b % kZeroParts) .. +15 of split tile b / kZeroParts (tile tail_first + that).
template <int KIND>
__global__ __launch_bounds__(kThreads) void k_split_fixup(int64_t M, int64_t N, void* D, int64_t ldd,
                                                          const float* __restrict__ part,
                                                          int64_t tail_first, float* amax) {
  using namespace big;
  constexpr int64_t kTile = (int64_t)kBlockM * kBlockN;
  const int64_t tiles_m = (M + kBlockM - 1) / kBlockM;
  const int64_t tiles_n = (N + kBlockN - 1) / kBlockN;
  const int64_t tl = blockIdx.x / kZeroParts;
  int64_t tm, tn;
  tile_of(tail_first + tl, tiles_m, tiles_n, tm, tn);
  const float* p0 = part + tl * 2 * kTile;
  const float* p1 = p0 + kTile;
  const int lr0 = (int)(blockIdx.x % kZeroParts) * 16;
  const int c4 = (threadIdx.x & 63) * 4;
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < 16 / (kThreads / 64); ++i) {
    const int lr = lr0 + (threadIdx.x >> 6) + i * (kThreads / 64);
    const int64_t row = tm * kBlockM + lr;
    if (row >= M) break;
    const float4 a = *reinterpret_cast<const float4*>(p0 + lr * kBlockN + c4);
    const float4 b = *reinterpret_cast<const float4*>(p1 + lr * kBlockN + c4);
    const float v[4] = {a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t col = tn * kBlockN + c4 + q;
      if (col < N) mx = fmaxf(mx, put_out<KIND>(D, ldd, row, col, v[q]));
    }
  }
  if (amax != nullptr) group_amax(mx, amax);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_grouped_gemm_big(int64_t G, const int64_t* __restrict__ off, Operand A,
                        const float* __restrict__ ag, Operand B, const float* __restrict__ bg,
                        int64_t N, int64_t K, float* __restrict__ D, int64_t ldd) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  using namespace big;
  const int64_t tiles_n = (N + kBlockN - 1) / kBlockN;
  // A last column at most 128 wide is computed by the narrower 256 x 64 / 256 x 128 tiles.
  const bool narrow_last = tiles_n > 1 && N - (tiles_n - 1) * kBlockN <= NHalf::kBlockN;
  const int64_t cols_main = narrow_last ? tiles_n - 1 : tiles_n;
  // Workgroups are dealt to the 8 XCDs round robin (XCD x runs ids x, x + 8, ...), and XCD x
  // takes its share of the slots whole (grouped_slot): every column tile of a slot runs on one
  // XCD, so the slot's A panel and its group's B panels enter that XCD's L2 once.
  int64_t g, m0, m1, tn;
  if (!grouped_slot(G, off, A.rows, blockIdx.x % 8, blockIdx.x / 8, cols_main, tiles_n, g, m0, m1, tn))
    return;
  const int64_t n0 = tn * kBlockN;
  const int64_t n1 = n0 + kBlockN < N ? n0 + kBlockN : N;
  const Operand Bg{B.codes + g * N * (K >> 1), B.scales + g * N * (K >> 4), N};
  const float alpha = ag[g] * bg[g];
  // a last column at most 64 or 128 wide and a group's last slot at most 128 high take the
  // narrower tiles, which cost about 0.4, 0.55 and 0.7 of the full one
  if (n1 - n0 <= NTail::kBlockN)
    gemm_tile_big<NTail>(A, Bg, m0, m1, n0, n1, K, 0, K, false, alpha, D, ldd, lds_dyn);
  else if (n1 - n0 <= NHalf::kBlockN)
    gemm_tile_big<NHalf>(A, Bg, m0, m1, n0, n1, K, 0, K, false, alpha, D, ldd, lds_dyn);
  else if (m1 - m0 <= MTail::kBlockM)
    gemm_tile_big<MTail>(A, Bg, m0, m1, n0, n1, K, 0, K, false, alpha, D, ldd, lds_dyn);
  else
    gemm_tile_big<Full>(A, Bg, m0, m1, n0, n1, K, 0, K, false, alpha, D, ldd, lds_dyn);
}

// Groups along the contraction: group g sums over elements [koff[g], koff[g+1]) of A's and B's
// rows into its own M x N block of D (rows g*M ..). Tile b: group b / tiles, tile b % tiles
// (XCD-aware order within the group). Offsets are clamped into [0, K] and made non-decreasing;
// an empty group writes zeros. Workgroup w computes tiles w, w + gridDim.x, ... (one per
// workgroup when the grid covers them all); when the next of them has the same shape, its first
// DMA stages are issued under the current tile's epilogue. The launch gives each workgroup a few
// tiles far apart in the walk (groups of different sizes) and leaves the balancing to the
// hardware's dispatch of workgroups: a grid of one workgroup per CU walking a fixed share of the
// tiles measured 1-9% slower on a Zipf-routed expert mix, the prefetch gain lost to imbalance.
struct KTile {
  int64_t g, m0, m1, n0, n1, k0, k1;
  int shape;                                    // 0: Full, 1: NHalf (256 x 128), 2: MTail (128 x 256)
};
__device__ __forceinline__ KTile ktile_of(int64_t b, int64_t tiles, int64_t tiles_m, int64_t tiles_n,
                                          const int64_t* __restrict__ koff, int64_t K, int64_t M, int64_t N) {
  using namespace big;
  // the divisors taken through an empty asm, so that the reciprocals of the divisions below are
  // formed here on every call instead of being hoisted out of the tile loop into vector
  // registers that would have to live through the main loop
  asm volatile("" : "+s"(tiles), "+s"(tiles_m), "+s"(tiles_n));
  KTile t;
  t.g = b / tiles;
  int64_t tm, tn;
  // the XCD region of the group's tile grid (tile_of deals regions by the id's residue mod 8)
  // rotated by the group: the cheaper narrow tiles of the last tile row and column fall in a few
  // regions, which with a fixed assignment went to the same XCDs for every group (one XCD
  // finished 15% of the call early on the expert layer)
  // (within whole runs of 8 ids only, so the ids stay a permutation of [0, tiles))
  const int64_t q = b - t.g * tiles, q8 = q - q % 8;
  tile_of(q8 + 8 <= tiles ? q8 + (q % 8 + t.g) % 8 : q, tiles_m, tiles_n, tm, tn);
  int64_t k0 = koff[t.g], k1 = koff[t.g + 1];
  k0 = k0 < 0 ? 0 : (k0 > K ? K : k0);
  k1 = k1 < k0 ? k0 : (k1 > K ? K : k1);
  t.k0 = k0;
  t.k1 = k1;
  t.m0 = tm * kBlockM;
  t.n0 = tn * kBlockN;
  t.m1 = t.m0 + kBlockM < M ? t.m0 + kBlockM : M;
  t.n1 = t.n0 + kBlockN < N ? t.n0 + kBlockN : N;
  // a last row tile at most 128 high or a last column tile at most 128 wide takes the
  // narrower tile (about half the work of the full one; the corner takes the 128-high one)
  t.shape = t.m1 - t.m0 <= MTail::kBlockM ? 2 : (t.n1 - t.n0 <= NHalf::kBlockN ? 1 : 0);
  return t;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_grouped_gemm_k_big(int64_t G, const int64_t* __restrict__ koff, Operand A,
                          const float* __restrict__ ag, Operand B, const float* __restrict__ bg,
                          int64_t K, float* __restrict__ D, int64_t ldd) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  using namespace big;
  const int64_t tiles_m = (A.rows + kBlockM - 1) / kBlockM;
  const int64_t tiles_n = (B.rows + kBlockN - 1) / kBlockN;
  const int64_t tiles = tiles_m * tiles_n;
  const int64_t total = G * tiles;
  bool prefetched = false;
  for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
    const KTile t = ktile_of(b, tiles, tiles_m, tiles_n, koff, K, A.rows, B.rows);
    TileNext nx{false, 0, 0, 0, 0};
    if (b + gridDim.x < total) {
      const KTile u = ktile_of(b + gridDim.x, tiles, tiles_m, tiles_n, koff, K, A.rows, B.rows);
      if (u.shape == t.shape) nx = TileNext{true, u.m0, u.n0, u.k0, u.k1};
    }
    const float alpha = ag[t.g] * bg[t.g];
    float* Dg = D + t.g * A.rows * ldd;
    const ExtOut none{nullptr, 0, nullptr, nullptr};
    if (t.shape == 2)
      gemm_tile_big<MTail, true>(A, B, t.m0, t.m1, t.n0, t.n1, K, t.k0, t.k1, false, alpha, Dg, ldd, lds_dyn,
                                 none, nx, prefetched);
    else if (t.shape == 1)
      gemm_tile_big<NHalf, true>(A, B, t.m0, t.m1, t.n0, t.n1, K, t.k0, t.k1, false, alpha, Dg, ldd, lds_dyn,
                                 none, nx, prefetched);
    else
      gemm_tile_big<Full, true>(A, B, t.m0, t.m1, t.n0, t.n1, K, t.k0, t.k1, false, alpha, Dg, ldd, lds_dyn,
                                none, nx, prefetched);
    prefetched = nx.valid;
  }
}

// =========================================================================================
// general kernel: 128 x 128 tiles, operands straight into registers (any K % 16 == 0)
// =========================================================================================
namespace small {
constexpr int kFragsM = 4, kFragsN = 4;                       // wave tile 64 x 64
constexpr int kWaveM = 16 * kFragsM, kWaveN = 16 * kFragsN;
constexpr int kBlockM = 2 * kWaveM, kBlockN = 2 * kWaveN;     // 128 x 128
}  // namespace small

struct FragLoad { v4u32 codes; uint32_t scales; };

// 32 codes of row `row` starting at element k (multiple of 32) and their two scale bytes;
// elements at or beyond K read as zero codes and zero scales.
__device__ __forceinline__ FragLoad load_frag(const uint8_t* __restrict__ codes,
                                              const uint8_t* __restrict__ scales, int64_t row,
                                              int64_t K, int64_t k) {
  FragLoad f{v4u32{0, 0, 0, 0}, 0};
  const int64_t left = K - k;
  if (left <= 0) return f;
  const uint8_t* cp = codes + row * (K >> 1) + (k >> 1);
  const uint8_t* sp = scales + row * (K >> 4) + (k >> 4);
  const v2u32 a = *reinterpret_cast<const v2u32*>(cp);
  if (left >= 32) {
    const v2u32 b = *reinterpret_cast<const v2u32*>(cp + 8);
    f.codes = v4u32{a.x, a.y, b.x, b.y};
    f.scales = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
  } else {                                  // exactly 16 elements remain (K % 16 == 0)
    f.codes = v4u32{a.x, a.y, 0, 0};
    f.scales = (uint32_t)sp[0];
  }
  return f;
}

template <int KIND = kOutF32, bool EXT = false>
__device__ __forceinline__ void gemm_tile_small(Operand A, Operand B, int64_t m0, int64_t m1,
                                                int64_t n0, int64_t n1, int64_t K, float alpha,
                                                float* __restrict__ D, int64_t ldd,
                                                const ExtOut ext = ExtOut{nullptr, 0, nullptr, nullptr}) {
  using namespace small;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t wm0 = m0 + (wave >> 1) * kWaveM;
  const int64_t wn0 = n0 + (wave & 1) * kWaveN;

  int64_t arow[kFragsM], brow[kFragsN];
#pragma unroll
  for (int i = 0; i < kFragsM; ++i) {
    const int64_t rr = wm0 + 16 * i + r;
    arow[i] = rr < m1 ? rr : m0;                 // rows past the end reload row m0
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
#pragma unroll
  for (int i = 0; i < kFragsM; ++i) fa[i] = load_frag(A.codes, A.scales, arow[i], K, g * 32);
#pragma unroll
  for (int j = 0; j < kFragsN; ++j) fb[j] = load_frag(B.codes, B.scales, brow[j], K, g * 32);

  for (int64_t k0 = 0; k0 < K; k0 += kStepK) {
    FragLoad na[kFragsM], nb[kFragsN];
    const int64_t kn = k0 + kStepK + g * 32;
#pragma unroll
    for (int i = 0; i < kFragsM; ++i) na[i] = load_frag(A.codes, A.scales, arow[i], K, kn);
#pragma unroll
    for (int j = 0; j < kFragsN; ++j) nb[j] = load_frag(B.codes, B.scales, brow[j], K, kn);
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

  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < kFragsM; ++i) {
#pragma unroll
    for (int j = 0; j < kFragsN; ++j) {
      const int64_t col = wn0 + 16 * j + r;
      if (col >= n1) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = wm0 + 16 * i + 4 * g + q;
        if (row < m1) {
          if constexpr (EXT) mx = fmaxf(mx, put_out<KIND>(ext.d, ext.ldd, row, col, acc[i][j][q] * alpha));
          else D[row * ldd + col] = acc[i][j][q] * alpha;
        }
      }
    }
  }
  if constexpr (EXT) {
    if (ext.amax != nullptr) group_amax(mx, ext.amax);
  }
}

__global__ __launch_bounds__(kThreads)
void k_gemm_small(Operand A, const float* __restrict__ ag, Operand B, const float* __restrict__ bg,
                  int64_t K, float* __restrict__ D, int64_t ldd) {
  using namespace small;
  const int64_t tiles_m = (A.rows + kBlockM - 1) / kBlockM;
  const int64_t tiles_n = (B.rows + kBlockN - 1) / kBlockN;
  int64_t tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * kBlockM, n0 = tn * kBlockN;
  const int64_t m1 = m0 + kBlockM < A.rows ? m0 + kBlockM : A.rows;
  const int64_t n1 = n0 + kBlockN < B.rows ? n0 + kBlockN : B.rows;
  gemm_tile_small(A, B, m0, m1, n0, n1, K, ag[0] * bg[0], D, ldd);
}

template <int KIND>
__global__ __launch_bounds__(kThreads)
void k_gemm_small_ext(Operand A, const float* __restrict__ ag, Operand B, const float* __restrict__ bg,
                      int64_t K, void* D, int64_t ldd, float* amax) {
  using namespace small;
  const int64_t tiles_m = (A.rows + kBlockM - 1) / kBlockM;
  const int64_t tiles_n = (B.rows + kBlockN - 1) / kBlockN;
  int64_t tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * kBlockM, n0 = tn * kBlockN;
  const int64_t m1 = m0 + kBlockM < A.rows ? m0 + kBlockM : A.rows;
  const int64_t n1 = n0 + kBlockN < B.rows ? n0 + kBlockN : B.rows;
  gemm_tile_small<KIND, true>(A, B, m0, m1, n0, n1, K, ag[0] * bg[0], nullptr, ldd,
                              ExtOut{D, ldd, nullptr, amax});
}

__global__ __launch_bounds__(kThreads)
void k_grouped_gemm_small(int64_t G, const int64_t* __restrict__ off, Operand A,
                          const float* __restrict__ ag, Operand B, const float* __restrict__ bg,
                          int64_t N, int64_t K, float* __restrict__ D, int64_t ldd) {
  using namespace small;
  const int64_t tiles_n = (N + kBlockN - 1) / kBlockN;
  const int64_t slot_m = blockIdx.x / tiles_n;
  const int64_t tn = blockIdx.x - slot_m * tiles_n;
  int64_t g, m0, m1;
  if (!group_of(G, off, A.rows, kBlockM, slot_m, g, m0, m1)) return;
  const int64_t n0 = tn * kBlockN;
  const int64_t n1 = n0 + kBlockN < N ? n0 + kBlockN : N;
  const Operand Bg{B.codes + g * N * (K >> 1), B.scales + g * N * (K >> 4), N};
  gemm_tile_small(A, Bg, m0, m1, n0, n1, K, ag[g] * bg[g], D, ldd);
}

// ---------------------------------------------------------------------------------------
// MXFP4 GEMM on gfx950's block-scaled FP4 matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4
// with both operands E2M1): the format's power-of-two scale per 32 elements is exactly what
// the instruction applies per lane, so the codes go from LDS to the matrix core untouched.
// Lane l of a 32x32x64 instruction holds row l % 32, elements 32*(l/32) .. +31 of the 64
// (16 bytes) and that block's E8M0 scale in byte 0 of its scale operand (checked on the
// device). D = sum over k of a*b with FP32 accumulation; MXFP4 has no tensor scale.
//
// Tile 256 x 256, 8 waves of 64 x 128 (2 x 4 instructions per 64 elements; two waves per
// SIMD, so one wave's waits hide under the other's instructions: 0-7% faster than 4 waves of
// 128 x 128 in interleaved timing, bit-identical), K steps of 128 (K % 128 == 0), DMA four
// steps deep. The matrix instruction consumes a step's operands four times faster than the
// FP16 path, so what limits this kernel is the number of L2 requests the buffer-to-LDS DMA
// makes, not bytes: four lanes read a row's 64 bytes of a step (one request per row and step
// instead of two). The scales are stored K step by K step (all rows' four E8M0 bytes of one
// 128-element step contiguous, see mxfp4_tensor), so a wave's scale DMA of a step is 256
// contiguous bytes (two requests for 64 rows, where row-major scales took one request per
// row), lands in LDS as one dword per row, and the per-row scale reads are conflict-free
// (row-major groups of 16 bytes per row put rows r, r+8, r+16, r+24 in one bank). (Stages
// of 256 elements, whose rows are whole 128-byte lines, fit only two deep in LDS and were
// slower: the prefetch distance matters more than the request count.) In LDS a fragment is
// 32 rows x 64 bytes, row-major, with the 16-byte chunk c of row r stored at slot c ^ sw(r)
// (below), so the instruction's 16-byte reads (row r, chunk 2s + h) fall in distinct banks.
namespace mx {
constexpr int kBlockM = 256, kBlockN = 256, kFragsA = 8, kFrags = 16;
constexpr int kFragBytes = 2048;                                  // 32 rows x 64 bytes
constexpr int kCodeBytes = kFrags * kFragBytes;                   // 32 KB per K step
constexpr int kStages = 4;
constexpr int kScaleStageBytes = (kBlockM + kBlockN) * 4;         // a step's E8M0 dword per row
constexpr int kScaleBase = kStages * kCodeBytes;
constexpr int kLdsBytes = kScaleBase + kStages * kScaleStageBytes;  // 136 KB
}  // namespace mx
constexpr int kMxThreads = 512;                                   // 8 waves, 2 per SIMD

typedef int int32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float16v mfma_mx(v4u32 a, v4u32 b, float16v c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
      int32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0},
      int32x8{(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0}, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

__global__ __launch_bounds__(kMxThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm_mx(Operand A, Operand B, int64_t K, float* __restrict__ D, int64_t ldd) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  uint8_t* lds = lds_dyn;
  using namespace mx;
  const int64_t tiles_m = (A.rows + kBlockM - 1) / kBlockM;
  const int64_t tiles_n = (B.rows + kBlockN - 1) / kBlockN;
  int64_t tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * kBlockM, n0 = tn * kBlockN;
  const int64_t m1 = m0 + kBlockM < A.rows ? m0 + kBlockM : A.rows;
  const int64_t n1 = n0 + kBlockN < B.rows ? n0 + kBlockN : B.rows;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 31, h = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t rs_codes = (uint32_t)(K >> 1);
  constexpr uint32_t kBeyond = 0x80000000u;
  const int steps = __builtin_amdgcn_readfirstlane((int)(K / kStepK));
  const __amdgpu_buffer_rsrc_t a_codes = make_rsrc(A.codes, A.rows * (K >> 1));
  const __amdgpu_buffer_rsrc_t b_codes = make_rsrc(B.codes, B.rows * (K >> 1));
  const __amdgpu_buffer_rsrc_t a_scales = make_rsrc(A.scales, A.rows * (K >> 5));
  const __amdgpu_buffer_rsrc_t b_scales = make_rsrc(B.scales, B.rows * (K >> 5));
  // scale DMA: wave w moves the step's dwords of rows 64 w .. 64 w + 63 of the tile's 512 (A
  // rows for w < 4, then B), lane l one row; rows past the operand read as zero (a row's dword
  // of step s sits at (s * rows + row) * 4, so a row past the end would alias the next step)
  const int sblk = wave;
  const bool s_is_a = sblk < 4;
  const int64_t s_rows = s_is_a ? A.rows : B.rows;
  const int64_t s_row = (s_is_a ? m0 : n0) + 64 * (s_is_a ? sblk : sblk - 4) + lane;
  const uint32_t lane_scales = s_row < s_rows ? (uint32_t)(s_row * 4) : kBeyond;
  const uint32_t step_scales = (uint32_t)(s_rows * 4);      // bytes per K step of scales
  // DMA for K step `step` (into code buffer `buf`), 5 operations per wave:
  //  p = 0..3: half q = p & 1 (rows 16q .. +15) of fragment f = wave + 8 (p >> 1) (A for
  //    p < 2, B after); lane l reads row 16q + l/4, chunk (l & 3) ^ sw(16q + l/4) of the
  //    step's 64 bytes into LDS f * 2 KB + q * 1 KB + l * 16 (row r's chunk c sits at 16-byte
  //    slot c ^ sw(r) of the row's 64 bytes; sw(16q + l/4) = ((l >> 3) & 3) ^ ((l >> 5) & 1)).
  //  p = 4: the step's E8M0 dwords of rows 64 wave .. +63 of the 512 (A then B), lane l one
  //    row, into the stage's scale buffer.
  // Steps past the last are issued out of range too (zeros, no memory traffic) into buffers
  // nobody reads again, so the loop has no branches.
  constexpr int kOps = 5;
  const uint32_t lane_codes = (uint32_t)(lane >> 2) * rs_codes +
                              16u * (uint32_t)((lane & 3) ^ ((lane >> 3) & 3) ^ ((lane >> 5) & 1));
  auto issue_dma_part = [&](int step, int buf, int p) {
    const bool live = step < steps;
    if (p == 4) {
      uint8_t* dst = lds + kScaleBase + buf * kScaleStageBytes + sblk * 256;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_is_a ? a_scales : b_scales, (lds_ptr_t)dst, 4,
                                               live ? lane_scales + (uint32_t)step * step_scales : kBeyond,
                                               0, 0, 0);
    } else {
      const int q = p & 1, f = wave + 8 * (p >> 1);
      const bool is_a = (p >> 1) == 0;
      const uint32_t row = __builtin_amdgcn_readfirstlane(
          (uint32_t)((is_a ? m0 : n0) + 32 * (is_a ? f : f - kFragsA) + 16 * q));
      const uint32_t su = row * rs_codes + (uint32_t)(step * (kStepK / 2));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? a_codes : b_codes,
                                               (lds_ptr_t)(lds + buf * kCodeBytes + f * kFragBytes + q * 1024), 16,
                                               lane_codes + (live ? su : kBeyond), 0, 0, 0);
    }
  };
  float16v acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float16v{};
  // operands of the 64-element half s2 of a step: lane (r, h) reads row r, chunk 2 s2 + h,
  // stored at slot (2 s2 + h) ^ sw(r); the E8M0 byte 2 s2 + h of the row's scale dword moved
  // to byte 0 (the byte the instruction reads). The swizzle sw(r) = ((r >> 1) & 3) ^
  // ((r >> 3) & 1) spreads the 16-byte reads of any 8 consecutive rows over the 128 bytes of
  // 32 banks and of any 16 consecutive rows over the 256 bytes of 64 banks.
  // The step's scale dwords (one per row, consecutive rows in consecutive banks) are read
  // with half 0 and kept for half 1.
  struct Ops { v4u32 a[2], b[4]; uint32_t sa[2], sb[4]; };
  uint32_t raw_sa[2], raw_sb[4];
  auto read_ops = [&](int step, int buf, int s2, Ops& o) {
    const int off = r * 64 + (((2 * s2 + h) ^ ((r >> 1) & 3) ^ ((r >> 3) & 1)) << 4);
    const uint8_t* base = lds + buf * kCodeBytes + off;
#pragma unroll
    for (int i = 0; i < 2; ++i) o.a[i] = *reinterpret_cast<const v4u32*>(base + (wm * 2 + i) * kFragBytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) o.b[j] = *reinterpret_cast<const v4u32*>(base + (kFragsA + wn * 4 + j) * kFragBytes);
    if (s2 == 0) {
      const uint8_t* sc = lds + kScaleBase + buf * kScaleStageBytes + r * 4;
#pragma unroll
      for (int i = 0; i < 2; ++i) raw_sa[i] = *reinterpret_cast<const uint32_t*>(sc + ((wm * 2 + i) * 32) * 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) raw_sb[j] = *reinterpret_cast<const uint32_t*>(sc + (kBlockM + (wn * 4 + j) * 32) * 4);
    }
    const int sh = 8 * (2 * s2 + h);
#pragma unroll
    for (int i = 0; i < 2; ++i) o.sa[i] = raw_sa[i] >> sh;
#pragma unroll
    for (int j = 0; j < 4; ++j) o.sb[j] = raw_sb[j] >> sh;
  };
  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // With dma_step >= 0 that step's DMA into dma_buf is issued behind the first instructions,
  // so the wave's pending LDS reads land before the compiler's ordering of LDS-bound DMA after
  // them can stall issue.
  auto mma = [&](const Ops& o, int dma_step, int dma_buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = mfma_mx(o.a[i], o.b[j], acc[i][j], o.sa[i], o.sb[j]);
        if (dma_step >= 0 && (i * 4 + j) < kOps) issue_dma_part(dma_step, dma_buf, i * 4 + j);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
#pragma unroll
  for (int p = 0; p < kStages; ++p)
#pragma unroll
    for (int q = 0; q < kOps; ++q) issue_dma_part(p, p, q);
  __builtin_amdgcn_s_waitcnt(big::waitcnt_imm((kStages - 1) * kOps, 15));
  barrier();
  // One step: half 1 is read while half 0's instructions run; then the barrier (every wave
  // has read step s's buffer, step s+1 and its scale group have landed); then half 0 of step
  // s+1 is read while half 1 runs with the DMA of step s+4 into step s's buffer.
  int b_cur = 0;
  Ops cur, nxt;
  read_ops(0, 0, 0, cur);
  for (int s = 0; s < steps; ++s) {
    const int b_next = b_cur == kStages - 1 ? 0 : b_cur + 1;
    read_ops(s, b_cur, 1, nxt);
    mma(cur, -1, 0);
    __builtin_amdgcn_s_waitcnt(big::waitcnt_imm((kStages - 2) * kOps, 0));
    barrier();
    read_ops(s + 1, b_next, 0, cur);
    mma(nxt, s + kStages, b_cur);
    b_cur = b_next;
  }
  __builtin_amdgcn_s_waitcnt(big::waitcnt_imm(0, 15));
  if (ldd <= (int64_t(1) << 20)) {
    // stores through a buffer resource bounded at the tile's last element, as in the FP16-path
    // kernel's epilogue: rows past m1 fall outside it, columns past n1 are pushed beyond it,
    // and each element costs one add of a uniform row offset to the lane's column offset
    const uint32_t ld4 = (uint32_t)ldd * 4u;
    const uint64_t base = reinterpret_cast<uint64_t>(D + m0 * ldd + n0);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
    const int64_t size = __builtin_amdgcn_readfirstlane((uint32_t)(((m1 - m0 - 1) * ldd + (n1 - n0)) * 4));
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), size);
    uint32_t voff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cl = wn * 128 + 32 * j + r;
      voff[j] = n0 + cl < n1 ? (uint32_t)(4 * h) * ld4 + (uint32_t)cl * 4u : kBeyond;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const uint32_t ro = (uint32_t)(wm * 64 + 32 * i + 8 * (q >> 2) + (q & 3)) * ld4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][q]), dr, voff[j] + ro, 0, 2);
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + 32 * j + r;
      if (col >= n1) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm * 64 + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
        if (row < m1) __builtin_nontemporal_store(acc[i][j][q], &D[row * ldd + col]);
      }
    }
}

bool use_big(int64_t K) { return K > 0 && (K % 64) == 0; }

// Compute units of the current device (queried once).
int64_t compute_units() {
  static const int64_t n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return (int64_t)256;
    return (int64_t)cus;
  }();
  return n;
}

hipError_t enable_big_lds() {
  static hipError_t once = [] {
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm_big,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, big::kLdsBytes);
    if (e != hipSuccess) return e;
    for (const void* f : {(const void*)k_gemm_big_ext<kOutF32>, (const void*)k_gemm_big_ext<kOutF32Add>,
                          (const void*)k_gemm_big_ext<kOutBF16>}) {
      e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, big::kLdsBytes);
      if (e != hipSuccess) return e;
    }
    e = hipFuncSetAttribute((const void*)k_grouped_gemm_big,
                            hipFuncAttributeMaxDynamicSharedMemorySize, big::kLdsBytes);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)k_grouped_gemm_k_big,
                               hipFuncAttributeMaxDynamicSharedMemorySize, big::kLdsBytes);
  }();
  return once;
}

// One workgroup per CU: when the tiles leave a partial last round of at most half the CUs,
// its tiles (tail_first ..) are split along K in two halves; a last round of at most a quarter
// of the CUs is instead cut into column quarters (splits = -1: four 256 x 64 tiles per tile,
// all of K, one round, no partial sums). In launch_gemm the halves are
// atomically added into zeroed D: two parts keep D reproducible (0 + a + b rounds the same in
// either order); more parts would make the rounding depend on the order the atomics land in.
void split_plan(int64_t tiles, int64_t K, int64_t& tail_first, int64_t& splits) {
  const int64_t cus = compute_units();
  const int64_t steps = (K + kStepK - 1) / kStepK;
  const int64_t rem = tiles % cus;
  if (rem && 4 * rem <= cus) {                     // column quarters: splits = -1
    tail_first = tiles - rem;
    splits = -1;
    return;
  }
  splits = rem ? cus / rem : 1;
  splits = splits > 2 ? 2 : splits;
  splits = splits > steps ? steps : splits;
  tail_first = splits >= 2 ? tiles - rem : tiles;
  if (splits < 2) splits = 1;
}

int64_t big_tiles(int64_t M, int64_t N) {
  return ((M + big::kBlockM - 1) / big::kBlockM) * ((N + big::kBlockN - 1) / big::kBlockN);
}

}  // namespace

hipError_t launch_gemm(GemmOperand a, GemmOperand b, int64_t M, int64_t N, int64_t K, float* D,
                       int64_t ldd, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const Operand A{a.codes, a.scales, M}, B{b.codes, b.scales, N};
  if (use_big(K)) {
    const hipError_t e = enable_big_lds();
    if (e != hipSuccess) return e;
    const int64_t tiles = big_tiles(M, N);
    int64_t tail_first, splits;
    split_plan(tiles, K, tail_first, splits);
    if (splits < 0) {
      hipLaunchKernelGGL(k_gemm_big, dim3((unsigned)(tail_first + 4 * (tiles - tail_first))), dim3(kThreads),
                         big::kLdsBytes, stream, A, a.global_scale, B, b.global_scale, K, D, ldd, tail_first, -1);
      return hipGetLastError();
    }
    if (tail_first < tiles) {
      const int vec = (ldd % 4) == 0 && (reinterpret_cast<uintptr_t>(D) % 16) == 0;
      hipLaunchKernelGGL(k_zero_tiles, dim3((unsigned)((tiles - tail_first) * kZeroParts)), dim3(kThreads), 0,
                         stream, M, N, D, ldd, tail_first, vec);
    }
    const int64_t grid = tail_first + (tiles - tail_first) * splits;
    hipLaunchKernelGGL(k_gemm_big, dim3((unsigned)grid), dim3(kThreads), big::kLdsBytes, stream,
                       A, a.global_scale, B, b.global_scale, K, D, ldd, tail_first, (int)splits);
  } else {
    const int64_t tiles = ((M + small::kBlockM - 1) / small::kBlockM) * ((N + small::kBlockN - 1) / small::kBlockN);
    hipLaunchKernelGGL(k_gemm_small, dim3((unsigned)tiles), dim3(kThreads), 0, stream, A,
                       a.global_scale, B, b.global_scale, K, D, ldd);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, float* D,
                          int64_t ldd, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  static const hipError_t attr = hipFuncSetAttribute((const void*)k_gemm_mx,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, mx::kLdsBytes);
  if (attr != hipSuccess) return attr;
  const Operand A{a_codes, a_scales, M}, B{b_codes, b_scales, N};
  const int64_t tiles = ((M + mx::kBlockM - 1) / mx::kBlockM) * ((N + mx::kBlockN - 1) / mx::kBlockN);
  hipLaunchKernelGGL(k_gemm_mx, dim3((unsigned)tiles), dim3(kMxThreads), mx::kLdsBytes, stream, A, B, K, D, ldd);
  return hipGetLastError();
}

size_t gemm_ex_workspace_bytes(int64_t M, int64_t N) {
  if (M <= 0 || N <= 0) return 0;
  const int64_t tiles = big_tiles(M, N);
  int64_t tail_first, splits;
  split_plan(tiles, 2 * kStepK, tail_first, splits);          // any K of two or more steps
  if (splits < 2) return 0;                                   // no K-split tiles (column quarters)
  return (size_t)(tiles - tail_first) * (size_t)splits * big::kBlockM * big::kBlockN * sizeof(float);
}

hipError_t launch_gemm_ex(GemmOperand a, GemmOperand b, int64_t M, int64_t N, int64_t K, int kind,
                          void* D, int64_t ldd, float* amax, float* ws, hipStream_t stream) {
  if (amax) {
    const hipError_t e = launch_fill(amax, 1, 0.0f, stream);
    if (e != hipSuccess) return e;
  }
  if (M == 0 || N == 0) return hipGetLastError();
  const Operand A{a.codes, a.scales, M}, B{b.codes, b.scales, N};
  if (use_big(K)) {
    const hipError_t e = enable_big_lds();
    if (e != hipSuccess) return e;
    const int64_t tiles = big_tiles(M, N);
    int64_t tail_first, splits;
    split_plan(tiles, K, tail_first, splits);
    const int64_t grid = tail_first + (tiles - tail_first) * (splits < 0 ? 4 : splits);
#define NVFP4_GX(KD)                                                                                  \
  hipLaunchKernelGGL(k_gemm_big_ext<KD>, dim3((unsigned)grid), dim3(kThreads), big::kLdsBytes, stream, \
                     A, a.global_scale, B, b.global_scale, K, D, ldd, amax, ws, tail_first, (int)splits); \
  if (tail_first < tiles && splits > 0)                                                               \
    hipLaunchKernelGGL(k_split_fixup<KD>, dim3((unsigned)((tiles - tail_first) * kZeroParts)),         \
                       dim3(kThreads), 0, stream, M, N, D, ldd, ws, tail_first, amax)
    if (kind == kOutBF16) { NVFP4_GX(kOutBF16); }
    else if (kind == kOutF32Add) { NVFP4_GX(kOutF32Add); }
    else { NVFP4_GX(kOutF32); }
#undef NVFP4_GX
  } else {
    const int64_t tiles = ((M + small::kBlockM - 1) / small::kBlockM) * ((N + small::kBlockN - 1) / small::kBlockN);
#define NVFP4_GS(KD) hipLaunchKernelGGL(k_gemm_small_ext<KD>, dim3((unsigned)tiles), dim3(kThreads), 0, stream, \
                                        A, a.global_scale, B, b.global_scale, K, D, ldd, amax)
    if (kind == kOutBF16) NVFP4_GS(kOutBF16);
    else if (kind == kOutF32Add) NVFP4_GS(kOutF32Add);
    else NVFP4_GS(kOutF32);
#undef NVFP4_GS
  }
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(int64_t G, const int64_t* m_offsets, GemmOperand a, GemmOperand b,
                               int64_t total_m, int64_t N, int64_t K, float* D, int64_t ldd,
                               hipStream_t stream) {
  if (total_m == 0 || N == 0) return hipSuccess;
  const Operand A{a.codes, a.scales, total_m}, B{b.codes, b.scales, G * N};
  if (use_big(K)) {
    const hipError_t e = enable_big_lds();
    if (e != hipSuccess) return e;
    const int64_t tiles_n = (N + big::kBlockN - 1) / big::kBlockN;
    const int64_t slots_m = total_m / big::kBlockM + G;       // >= sum_g ceil(M_g / 256)
    // 8 XCDs, each with at most ceil(T c / 8) + ceil(T / 8) <= ceil(T tiles_n / 8) + 1 tiles
    // (T <= slots_m slots, c + 1 = tiles_n column tiles before the last when that one is narrow;
    // ceil(T tiles_n / 8) when it is not)
    hipLaunchKernelGGL(k_grouped_gemm_big, dim3((unsigned)(8 * ((slots_m * tiles_n + 7) / 8 + 1))),
                       dim3(kThreads), big::kLdsBytes, stream, G, m_offsets, A, a.global_scale, B,
                       b.global_scale, N, K, D, ldd);
  } else {
    const int64_t tiles_n = (N + small::kBlockN - 1) / small::kBlockN;
    const int64_t slots_m = total_m / small::kBlockM + G;
    hipLaunchKernelGGL(k_grouped_gemm_small, dim3((unsigned)(slots_m * tiles_n)), dim3(kThreads),
                       0, stream, G, m_offsets, A, a.global_scale, B, b.global_scale, N, K, D, ldd);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_k(int64_t G, const int64_t* k_offsets, GemmOperand a, GemmOperand b,
                                 int64_t M, int64_t N, int64_t K, float* D, int64_t ldd,
                                 hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const hipError_t e = enable_big_lds();
  if (e != hipSuccess) return e;
  const Operand A{a.codes, a.scales, M}, B{b.codes, b.scales, N};
  const int64_t tiles = ((M + big::kBlockM - 1) / big::kBlockM) * ((N + big::kBlockN - 1) / big::kBlockN);
  // about kTilesPerGroup tiles per workgroup, the grid a multiple of 8 so that a workgroup's
  // tiles all belong to its XCD's share of the tile order
  // (2: with the XCD regions rotated per group, 2, 3, 4 and 6 tiles per workgroup measured
  // 1324, 1327, 1345 and 1345 us on the expert layer's weight gradient)
  constexpr int64_t kTilesPerGroup = 2;
  const int64_t total = G * tiles;
  if (total == 0) return hipSuccess;
  int64_t grid = ((total + kTilesPerGroup - 1) / kTilesPerGroup + 7) / 8 * 8;
  if (grid > total) grid = total;
  hipLaunchKernelGGL(k_grouped_gemm_k_big, dim3((unsigned)grid), dim3(kThreads), big::kLdsBytes, stream,
                     G, k_offsets, A, a.global_scale, B, b.global_scale, K, D, ldd);
  return hipGetLastError();
}

}  // namespace nvfp4
