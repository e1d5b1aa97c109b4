// C ABI of libnvfp4 (declared in include/nvfp4.h): host-side validation, workspace
// sizing and dispatch to the gfx950 kernels. Nothing here allocates device memory.
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/nvfp4.h"
#include "launch.h"

// Device memory of nvfp4_quantize_noalloc: the partial or per-segment tensor maxima of its amax
// pass, which nvfp4_quantize keeps in the caller's workspace. One copy per device (the module is
// loaded on each device it runs on), held until the process ends. In host code `scratch` names
// a host-side stand-in, not device memory: kernels get the device address that
// hipGetSymbolAddress returns for the current device (scratch_on_device below), never `scratch`.
constexpr int64_t kNoAllocScratchFloats = 16384;        // 64 KiB: up to 16384 segments
static_assert(kNoAllocScratchFloats >= nvfp4::kMaxAmaxPartials, "scratch holds the amax partials");
static __device__ __align__(256) float scratch[kNoAllocScratchFloats];

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return NVFP4_OK;
  return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

int scratch_on_device(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(NVFP4_ERR_UNSUPPORTED, "device %d beyond the %d devices supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(NVFP4_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_addr[dev] = p;
  }
  *out = static_cast<float*>(g_scratch_addr[dev]);
  return NVFP4_OK;
}

constexpr size_t kWsAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Checks an output tensor descriptor for a [rows, cols] quantization.
// An empty output (no rows or no columns) is never written, so its buffers may be NULL.
int check_out(const nvfp4_tensor* t, int64_t rows, int64_t cols, const char* name) {
  if (!t) return fail(NVFP4_ERR_INVALID, "%s is NULL", name);
  if (t->rows != rows || t->cols != cols)
    return fail(NVFP4_ERR_INVALID, "%s shape [%lld, %lld] does not match [%lld, %lld]", name,
                (long long)t->rows, (long long)t->cols, (long long)rows, (long long)cols);
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (!t->codes || !t->scales || !t->global_scale)
    return fail(NVFP4_ERR_INVALID, "%s has a NULL codes/scales/global_scale pointer", name);
  if (!aligned(t->codes, 16))
    return fail(NVFP4_ERR_INVALID, "%s codes must be 16-byte aligned", name);
  return NVFP4_OK;
}

// Row-blocked kernels read 16-byte vectors along rows (rows_vec = true); the Hadamard kernel
// reads column pairs across rows and only needs the pair to be aligned.
int check_input(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                bool rows_vec = true) {
  if (dt != NVFP4_IN_BF16 && dt != NVFP4_IN_FP32) return fail(NVFP4_ERR_INVALID, "bad dtype %d", (int)dt);
  if (rows < 0 || cols < 1) return fail(NVFP4_ERR_INVALID, "bad shape [%lld, %lld]", (long long)rows, (long long)cols);
  if (ld < cols) return fail(NVFP4_ERR_INVALID, "ld (%lld) < cols (%lld)", (long long)ld, (long long)cols);
  if (rows == 0) return NVFP4_OK;                 // an empty input is never read (x may be NULL)
  if (!x) return fail(NVFP4_ERR_INVALID, "x is NULL");
  const size_t esz = dt == NVFP4_IN_BF16 ? 2 : 4;
  if (!rows_vec) {
    if (!aligned(x, 2 * esz)) return fail(NVFP4_ERR_UNSUPPORTED, "x must be %zu-byte aligned", 2 * esz);
    return NVFP4_OK;
  }
  const int64_t vec = (int64_t)(16 / esz);              // elements per 16 bytes
  if (!aligned(x, 16) || ld % vec != 0)
    return fail(NVFP4_ERR_UNSUPPORTED, "x must be 16-byte aligned with ld a multiple of %lld", (long long)vec);
  return NVFP4_OK;
}

}  // namespace

extern "C" {

const char* nvfp4_last_error(void) { return g_last_error.c_str(); }

size_t nvfp4_workspace_size(int op, int64_t rows, int64_t cols, int64_t nseg) {
  (void)rows;
  (void)cols;
  const size_t partials = (size_t)nvfp4::kMaxAmaxPartials * sizeof(float);
  switch (op) {
    case NVFP4_OP_QUANTIZE: {
      const size_t segs = (size_t)(nseg < 1 ? 1 : nseg) * sizeof(float);
      return round_up(segs > partials ? segs : partials, kWsAlign);
    }
    case NVFP4_OP_RHT_QUANTIZE: {
      const size_t segs = (size_t)(nseg < 1 ? 1 : nseg) * sizeof(float);
      return round_up(segs > partials ? segs : partials, kWsAlign);
    }
    case NVFP4_OP_AMAX_PAIR: return round_up(2 * partials, kWsAlign);
    case NVFP4_OP_GEMM_EX: return round_up(nvfp4::gemm_ex_workspace_bytes(rows, cols), kWsAlign);
    default: return 0;
  }
}

int nvfp4_amax(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
               const int64_t* segments, int64_t nseg, int rht, uint16_t sign_mask,
               float* amax_out, void* workspace, size_t ws_bytes, void* hip_stream) {
  if (rht < 0 || rht > 2) return fail(NVFP4_ERR_INVALID, "bad rht selector %d", rht);
  int st = check_input(x, dt, rows, cols, ld, rht != 1);
  if (st) return st;
  if (!amax_out) return fail(NVFP4_ERR_INVALID, "amax_out is NULL");
  if (nseg < 1 || (!segments && nseg != 1)) return fail(NVFP4_ERR_INVALID, "bad segment table (nseg=%lld)", (long long)nseg);
  if (rows == 0) return hip_status(nvfp4::launch_fill(amax_out, nseg, 0.0f, (hipStream_t)hip_stream), "amax of nothing");
  if (rht == 2) {                                   // rowwise rotation, unsegmented
    if (segments) return fail(NVFP4_ERR_UNSUPPORTED, "the rowwise rotation takes no segments");
    if (cols % 16) return fail(NVFP4_ERR_INVALID, "cols (%lld) must be a multiple of 16", (long long)cols);
    const size_t need = nvfp4_workspace_size(NVFP4_OP_QUANTIZE, rows, cols, 1);
    if (!workspace || ws_bytes < need || !aligned(workspace, kWsAlign))
      return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) required, got %zu", need, ws_bytes);
    float* ws = static_cast<float*>(workspace);
    int parts = 1;
    hipStream_t s = (hipStream_t)hip_stream;
    if ((st = hip_status(nvfp4::launch_rot_amax_parts(x, dt == NVFP4_IN_FP32, rows, cols, ld, sign_mask, ws, &parts, s),
                         "rotated amax"))) return st;
    return hip_status(nvfp4::launch_reduce_partials(ws, parts, amax_out, s), "amax reduce");
  }
  if (rht && rows % 16) return fail(NVFP4_ERR_INVALID, "tokens (%lld) must be a multiple of 16", (long long)rows);
  if (!rht && cols % 16) return fail(NVFP4_ERR_INVALID, "cols (%lld) must be a multiple of 16", (long long)cols);
  const bool need_ws = !segments;
  if (need_ws) {
    const size_t need = nvfp4_workspace_size(rht ? NVFP4_OP_RHT_QUANTIZE : NVFP4_OP_QUANTIZE, rows, cols, nseg);
    if (!workspace || ws_bytes < need || !aligned(workspace, kWsAlign))
      return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) required, got %zu", need, ws_bytes);
  }
  hipStream_t s = (hipStream_t)hip_stream;
  const bool f32 = dt == NVFP4_IN_FP32;
  int parts = 1;
  if (rht) {
    if (segments)                                 // token segments: per-segment maxima directly
      return hip_status(nvfp4::launch_rht_amax_parts(x, f32, rows, cols, ld, sign_mask, false, segments,
                                                     nseg, amax_out, &parts, s), "rht amax");
    float* ws = static_cast<float*>(workspace);
    if ((st = hip_status(nvfp4::launch_rht_amax_parts(x, f32, rows, cols, ld, sign_mask, false, nullptr, 1,
                                                      ws, &parts, s), "rht amax"))) return st;
    return hip_status(nvfp4::launch_reduce_partials(ws, parts, amax_out, s), "amax reduce");
  }
  if (segments)
    return hip_status(nvfp4::launch_amax_parts(x, f32, rows, cols, ld, segments, nseg, amax_out, &parts, s), "amax");
  float* ws = static_cast<float*>(workspace);
  if ((st = hip_status(nvfp4::launch_amax_parts(x, f32, rows, cols, ld, nullptr, 1, ws, &parts, s), "amax"))) return st;
  return hip_status(nvfp4::launch_reduce_partials(ws, parts, amax_out, s), "amax reduce");
}

int nvfp4_rht_rows_quantize(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                            uint16_t sign_mask, nvfp4_round rnd, uint64_t seed, uint64_t offset,
                            const float* amax_in, nvfp4_tensor* out, void* workspace, size_t ws_bytes,
                            void* hip_stream) {
  int st;
  if ((st = check_input(x, dt, rows, cols, ld))) return st;
  if (cols % 16) return fail(NVFP4_ERR_INVALID, "cols (%lld) must be a multiple of 16", (long long)cols);
  if (rnd != NVFP4_ROUND_RN && rnd != NVFP4_ROUND_SR) return fail(NVFP4_ERR_INVALID, "bad rounding %d", (int)rnd);
  if ((st = check_out(out, rows, cols, "out"))) return st;
  if (rows == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)hip_stream;
  const bool f32 = dt == NVFP4_IN_FP32;
  const float* amax = amax_in;
  int parts = 1;
  if (!amax) {
    const size_t need = nvfp4_workspace_size(NVFP4_OP_QUANTIZE, rows, cols, 1);
    if (!workspace || ws_bytes < need || !aligned(workspace, kWsAlign))
      return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) required, got %zu", need, ws_bytes);
    float* ws = static_cast<float*>(workspace);
    if ((st = hip_status(nvfp4::launch_rot_amax_parts(x, f32, rows, cols, ld, sign_mask, ws, &parts, s), "rotated amax")))
      return st;
    amax = ws;
  }
  const nvfp4::QuantOut q{out->codes, out->scales, out->global_scale};
  return hip_status(nvfp4::launch_encode_rot(x, f32, rows, cols, ld, sign_mask, rnd == NVFP4_ROUND_SR, seed, offset,
                                             amax, parts, q, s), "rotated encode");
}

int nvfp4_amax_pair(const void* x, nvfp4_dtype dt, int64_t tokens, int64_t cols, int64_t ld,
                    uint16_t sign_mask, float* amax_out, void* workspace, size_t ws_bytes,
                    void* hip_stream) {
  int st = check_input(x, dt, tokens, cols, ld, false);
  if (st) return st;
  if (!amax_out) return fail(NVFP4_ERR_INVALID, "amax_out is NULL");
  if (tokens % 16) return fail(NVFP4_ERR_INVALID, "tokens (%lld) must be a multiple of 16", (long long)tokens);
  if (tokens == 0) return hip_status(nvfp4::launch_fill(amax_out, 2, 0.0f, (hipStream_t)hip_stream), "amax of nothing");
  const size_t need = nvfp4_workspace_size(NVFP4_OP_AMAX_PAIR, tokens, cols, 1);
  if (!workspace || ws_bytes < need || !aligned(workspace, kWsAlign))
    return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) required, got %zu", need, ws_bytes);
  hipStream_t s = (hipStream_t)hip_stream;
  float* ws = static_cast<float*>(workspace);
  int parts = 1;
  if ((st = hip_status(nvfp4::launch_rht_amax_parts(x, dt == NVFP4_IN_FP32, tokens, cols, ld, sign_mask,
                                                    true, nullptr, 1, ws, &parts, s), "amax pair")))
    return st;
  // partials [0, parts) of |x| and [parts, 2 parts) of |Hx| fold into amax_out[0] and [1]
  return hip_status(nvfp4::launch_reduce_partials(ws, parts, amax_out, s, 2), "amax reduce");
}

}  // extern "C"

namespace {

// nvfp4_quantize; with use_scratch the amax pass (when amax_in is NULL) takes the device's
// static scratch array instead of the caller's workspace, looked up after validation.
int quantize_impl(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                  nvfp4_block blk, nvfp4_round rnd, uint64_t seed, uint64_t offset,
                  const int64_t* segments, int64_t nseg, const float* amax_in,
                  nvfp4_tensor* out, nvfp4_tensor* out_t, void* workspace, size_t ws_bytes,
                  void* hip_stream, bool use_scratch) {
  int st = check_input(x, dt, rows, cols, ld);
  if (st) return st;
  if (blk != NVFP4_BLOCK_1X16 && blk != NVFP4_BLOCK_16X16) return fail(NVFP4_ERR_INVALID, "bad block mode %d", (int)blk);
  if (rnd != NVFP4_ROUND_RN && rnd != NVFP4_ROUND_SR) return fail(NVFP4_ERR_INVALID, "bad rounding mode %d", (int)rnd);
  if (cols % 16) return fail(NVFP4_ERR_INVALID, "cols (%lld) must be a multiple of 16", (long long)cols);
  if (blk == NVFP4_BLOCK_16X16 && rows % 16) return fail(NVFP4_ERR_INVALID, "rows (%lld) must be a multiple of 16 for 16x16 blocks", (long long)rows);
  if (nseg < 1 || (!segments && nseg != 1)) return fail(NVFP4_ERR_INVALID, "bad segment table (nseg=%lld)", (long long)nseg);
  if (out_t && blk != NVFP4_BLOCK_16X16) return fail(NVFP4_ERR_INVALID, "out_t requires 16x16 blocks");
  if (blk == NVFP4_BLOCK_16X16 && rnd == NVFP4_ROUND_SR) return fail(NVFP4_ERR_UNSUPPORTED, "stochastic rounding applies to 1x16 gradient blocks only");
  if (out_t && segments && (rows % nseg || (rows / nseg) % 16))
    return fail(NVFP4_ERR_UNSUPPORTED, "transposed emission of a segmented tensor needs %lld equal segments of a multiple of 16 rows (rows = %lld)",
                (long long)nseg, (long long)rows);
  if ((st = check_out(out, rows, cols, "out"))) return st;
  if (out_t && (st = check_out(out_t, segments ? nseg * cols : cols, rows / nseg, "out_t"))) return st;
  if (rows == 0) return NVFP4_OK;
  const float* amax = amax_in;
  if (!amax && use_scratch) {
    if (nseg > kNoAllocScratchFloats)
      return fail(NVFP4_ERR_UNSUPPORTED, "nvfp4_quantize_noalloc handles at most %lld segments (got %lld); "
                  "use nvfp4_quantize with a workspace", (long long)kNoAllocScratchFloats, (long long)nseg);
    float* ws = nullptr;
    if ((st = scratch_on_device(&ws))) return st;
    workspace = ws;
    ws_bytes = (size_t)kNoAllocScratchFloats * sizeof(float);
  }
  if (!amax) {
    const size_t need = nvfp4_workspace_size(NVFP4_OP_QUANTIZE, rows, cols, nseg);
    if (!workspace || ws_bytes < need || !aligned(workspace, kWsAlign))
      return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) required, got %zu", need, ws_bytes);
  }
  hipStream_t s = (hipStream_t)hip_stream;
  const bool f32 = dt == NVFP4_IN_FP32;
  int parts = 1;
  if (!amax) {
    float* ws = static_cast<float*>(workspace);
    if ((st = hip_status(nvfp4::launch_amax_parts(x, f32, rows, cols, ld, segments, nseg, ws, &parts, s), "amax"))) return st;
    amax = ws;
  }
  const nvfp4::QuantOut q{out->codes, out->scales, out->global_scale};
  if (blk == NVFP4_BLOCK_1X16)
    return hip_status(nvfp4::launch_encode_1x16(x, f32, rows, cols, ld, rnd == NVFP4_ROUND_SR, seed,
                                                offset, segments, nseg, amax, parts, q, s), "encode 1x16");
  nvfp4::QuantOut qt{};
  if (out_t) qt = nvfp4::QuantOut{out_t->codes, out_t->scales, out_t->global_scale};
  return hip_status(nvfp4::launch_encode_16x16(x, f32, rows, cols, ld, segments, nseg, amax, parts, q,
                                               out_t ? &qt : nullptr, s), "encode 16x16");
}

}  // namespace

extern "C" {

int nvfp4_quantize(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                   nvfp4_block blk, nvfp4_round rnd, uint64_t seed, uint64_t offset,
                   const int64_t* segments, int64_t nseg, const float* amax_in,
                   nvfp4_tensor* out, nvfp4_tensor* out_t, void* workspace, size_t ws_bytes,
                   void* hip_stream) {
  return quantize_impl(x, dt, rows, cols, ld, blk, rnd, seed, offset, segments, nseg, amax_in, out, out_t,
                       workspace, ws_bytes, hip_stream, false);
}

int nvfp4_quantize_noalloc(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                           nvfp4_block blk, nvfp4_round rnd, uint64_t seed, uint64_t offset,
                           const int64_t* segments, int64_t nseg, const float* amax_in,
                           nvfp4_tensor* out, nvfp4_tensor* out_t, void* hip_stream) {
  return quantize_impl(x, dt, rows, cols, ld, blk, rnd, seed, offset, segments, nseg, amax_in, out, out_t,
                       nullptr, 0, hip_stream, true);
}

int nvfp4_rht_quantize(const void* x, nvfp4_dtype dt, int64_t tokens, int64_t cols, int64_t ld,
                       uint16_t sign_mask, nvfp4_round rnd, uint64_t seed, uint64_t offset,
                       const int64_t* segments, int64_t nseg, const float* amax_in,
                       nvfp4_tensor* out, void* workspace, size_t ws_bytes, void* hip_stream) {
  int st = check_input(x, dt, tokens, cols, ld, false);
  if (st) return st;
  if (rnd != NVFP4_ROUND_RN && rnd != NVFP4_ROUND_SR) return fail(NVFP4_ERR_INVALID, "bad rounding mode %d", (int)rnd);
  if (tokens % 16) return fail(NVFP4_ERR_INVALID, "tokens (%lld) must be a multiple of 16", (long long)tokens);
  if (nseg < 1 || (!segments && nseg != 1)) return fail(NVFP4_ERR_INVALID, "bad segment table (nseg=%lld)", (long long)nseg);
  if ((st = check_out(out, cols, tokens, "out"))) return st;
  if (tokens == 0) return NVFP4_OK;
  const float* amax = amax_in;
  if (!amax) {
    const size_t need = nvfp4_workspace_size(NVFP4_OP_RHT_QUANTIZE, tokens, cols, nseg);
    if (!workspace || ws_bytes < need || !aligned(workspace, kWsAlign))
      return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) required, got %zu", need, ws_bytes);
  }
  hipStream_t s = (hipStream_t)hip_stream;
  const bool f32 = dt == NVFP4_IN_FP32;
  int parts = 1;
  if (!amax) {
    float* ws = static_cast<float*>(workspace);
    if ((st = hip_status(nvfp4::launch_rht_amax_parts(x, f32, tokens, cols, ld, sign_mask, false, segments,
                                                      nseg, ws, &parts, s), "rht amax"))) return st;
    amax = ws;
  }
  const nvfp4::QuantOut q{out->codes, out->scales, out->global_scale};
  return hip_status(nvfp4::launch_rht_encode(x, f32, tokens, cols, ld, sign_mask, rnd == NVFP4_ROUND_SR,
                                             seed, offset, segments, nseg, amax, parts, q, s), "rht encode");
}

// An operand without rows is never read (no output row or column depends on it), so its
// buffers may be NULL.
static int check_operand(const nvfp4_tensor* t, const char* name) {
  if (!t) return fail(NVFP4_ERR_INVALID, "%s is NULL", name);
  if (t->rows < 0 || t->cols < 0 || t->cols % 16)
    return fail(NVFP4_ERR_INVALID, "%s shape [%lld, %lld]: cols must be a non-negative multiple of 16", name,
                (long long)t->rows, (long long)t->cols);
  if (t->rows == 0) return NVFP4_OK;
  if (!t->codes || !t->scales || !t->global_scale)
    return fail(NVFP4_ERR_INVALID, "%s has a NULL codes/scales/global_scale pointer", name);
  if (!aligned(t->codes, 16)) return fail(NVFP4_ERR_INVALID, "%s codes must be 16-byte aligned", name);
  // the GEMM kernels address an operand through 32-bit buffer offsets
  if (t->rows * (t->cols / 2) > (int64_t)0x7FFFFFFF)
    return fail(NVFP4_ERR_UNSUPPORTED, "%s codes exceed 2 GiB", name);
  return NVFP4_OK;
}

int nvfp4_gemm(const nvfp4_tensor* A, const nvfp4_tensor* B, float* D, int64_t ldd, void* hip_stream) {
  int st;
  if ((st = check_operand(A, "A")) || (st = check_operand(B, "B"))) return st;
  if (A->cols != B->cols) return fail(NVFP4_ERR_INVALID, "K mismatch: A has %lld, B has %lld", (long long)A->cols, (long long)B->cols);
  if (!D && A->rows > 0 && B->rows > 0) return fail(NVFP4_ERR_INVALID, "D is NULL");   // an empty D is never written
  if (ldd < B->rows) return fail(NVFP4_ERR_INVALID, "ldd (%lld) < N (%lld)", (long long)ldd, (long long)B->rows);
  const nvfp4::GemmOperand a{A->codes, A->scales, A->global_scale};
  const nvfp4::GemmOperand b{B->codes, B->scales, B->global_scale};
  return hip_status(nvfp4::launch_gemm(a, b, A->rows, B->rows, A->cols, D, ldd, (hipStream_t)hip_stream), "gemm");
}

int mxfp4_quantize_columns(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                           nvfp4_round rnd, uint64_t seed, uint64_t offset, mxfp4_tensor* out,
                           void* hip_stream) {
  int st;
  if ((st = check_input(x, dt, rows, cols, ld, false))) return st;
  if (rows % 32) return fail(NVFP4_ERR_INVALID, "rows (%lld) must be a multiple of 32", (long long)rows);
  if (rnd != NVFP4_ROUND_RN && rnd != NVFP4_ROUND_SR) return fail(NVFP4_ERR_INVALID, "bad rounding %d", (int)rnd);
  if (!out) return fail(NVFP4_ERR_INVALID, "out is NULL");
  if (out->rows != cols || out->cols != rows)
    return fail(NVFP4_ERR_INVALID, "out shape [%lld, %lld] does not match [%lld, %lld]", (long long)out->rows,
                (long long)out->cols, (long long)cols, (long long)rows);
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (!out->codes || !out->scales) return fail(NVFP4_ERR_INVALID, "out buffers are NULL");
  if (!aligned(out->codes, 16) || !aligned(out->scales, 8))
    return fail(NVFP4_ERR_INVALID, "out codes must be 16-byte and scales 8-byte aligned");
  return hip_status(nvfp4::launch_encode_mx_cols(x, dt == NVFP4_IN_FP32, rows, cols, ld, rnd == NVFP4_ROUND_SR,
                                                 seed, offset, out->codes, out->scales, (hipStream_t)hip_stream),
                    "mxfp4 column encode");
}

int mxfp4_quantize(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                   nvfp4_round rnd, uint64_t seed, uint64_t offset, mxfp4_tensor* out,
                   void* hip_stream) {
  int st;
  if ((st = check_input(x, dt, rows, cols, ld))) return st;
  if (cols % 32) return fail(NVFP4_ERR_INVALID, "cols (%lld) must be a multiple of 32", (long long)cols);
  if (rnd != NVFP4_ROUND_RN && rnd != NVFP4_ROUND_SR) return fail(NVFP4_ERR_INVALID, "bad rounding %d", (int)rnd);
  if (!out) return fail(NVFP4_ERR_INVALID, "out is NULL");
  if (out->rows != rows || out->cols != cols)
    return fail(NVFP4_ERR_INVALID, "out shape [%lld, %lld] does not match [%lld, %lld]", (long long)out->rows,
                (long long)out->cols, (long long)rows, (long long)cols);
  if (rows == 0) return NVFP4_OK;
  if (!out->codes || !out->scales) return fail(NVFP4_ERR_INVALID, "out buffers are NULL");
  if (!aligned(out->codes, 8)) return fail(NVFP4_ERR_INVALID, "out codes must be 8-byte aligned");
  return hip_status(nvfp4::launch_encode_mx(x, dt == NVFP4_IN_FP32, rows, cols, ld, rnd == NVFP4_ROUND_SR, seed,
                                            offset, out->codes, out->scales, (hipStream_t)hip_stream),
                    "mxfp4 encode");
}

static int check_mx_operand(const mxfp4_tensor* t, const char* name) {
  if (!t) return fail(NVFP4_ERR_INVALID, "%s is NULL", name);
  if (t->rows < 0 || t->cols < 0 || t->cols % 32)
    return fail(NVFP4_ERR_INVALID, "%s shape [%lld, %lld]: cols must be a non-negative multiple of 32", name,
                (long long)t->rows, (long long)t->cols);
  if (t->rows == 0) return NVFP4_OK;
  if (!t->codes || !t->scales) return fail(NVFP4_ERR_INVALID, "%s has a NULL codes/scales pointer", name);
  if (!aligned(t->codes, 16)) return fail(NVFP4_ERR_INVALID, "%s codes must be 16-byte aligned", name);
  if (!aligned(t->scales, 4)) return fail(NVFP4_ERR_INVALID, "%s scales must be 4-byte aligned", name);
  if (t->rows * (t->cols / 2) > (int64_t)0x7FFFFFFF)
    return fail(NVFP4_ERR_UNSUPPORTED, "%s codes exceed 2 GiB", name);
  return NVFP4_OK;
}

int mxfp4_gemm(const mxfp4_tensor* A, const mxfp4_tensor* B, float* D, int64_t ldd, void* hip_stream) {
  int st;
  if ((st = check_mx_operand(A, "A")) || (st = check_mx_operand(B, "B"))) return st;
  if (A->cols != B->cols) return fail(NVFP4_ERR_INVALID, "K mismatch: A has %lld, B has %lld", (long long)A->cols, (long long)B->cols);
  if (!D && A->rows > 0 && B->rows > 0) return fail(NVFP4_ERR_INVALID, "D is NULL");   // an empty D is never written
  if (ldd < B->rows) return fail(NVFP4_ERR_INVALID, "ldd (%lld) < N (%lld)", (long long)ldd, (long long)B->rows);
  if (A->cols % 128) return fail(NVFP4_ERR_UNSUPPORTED, "K (%lld) must be a multiple of 128", (long long)A->cols);
  return hip_status(nvfp4::launch_gemm_mx(A->codes, A->scales, B->codes, B->scales, A->rows, B->rows, A->cols, D, ldd,
                                          (hipStream_t)hip_stream), "mxfp4 gemm");
}

int nvfp4_gemm_ex(const nvfp4_tensor* A, const nvfp4_tensor* B, void* D, int64_t ldd, nvfp4_out out_kind,
                  float* amax_out, void* workspace, size_t ws_bytes, void* hip_stream) {
  int st;
  if ((st = check_operand(A, "A")) || (st = check_operand(B, "B"))) return st;
  if (A->cols != B->cols) return fail(NVFP4_ERR_INVALID, "K mismatch: A has %lld, B has %lld", (long long)A->cols, (long long)B->cols);
  if (!D && A->rows > 0 && B->rows > 0) return fail(NVFP4_ERR_INVALID, "D is NULL");   // an empty D is never written
  if (out_kind != NVFP4_OUT_FP32 && out_kind != NVFP4_OUT_FP32_ACCUMULATE && out_kind != NVFP4_OUT_BF16)
    return fail(NVFP4_ERR_INVALID, "bad output kind %d", (int)out_kind);
  if (ldd < B->rows) return fail(NVFP4_ERR_INVALID, "ldd (%lld) < N (%lld)", (long long)ldd, (long long)B->rows);
  if (!aligned(D, out_kind == NVFP4_OUT_BF16 ? 2 : 4)) return fail(NVFP4_ERR_INVALID, "D is not aligned to its element size");
  const size_t need = nvfp4_workspace_size(NVFP4_OP_GEMM_EX, A->rows, B->rows, 1);
  if (need && (!workspace || ws_bytes < need))
    return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : (size_t)0);
  if (need && !aligned(workspace, kWsAlign)) return fail(NVFP4_ERR_INVALID, "workspace must be 256-byte aligned");
  const nvfp4::GemmOperand a{A->codes, A->scales, A->global_scale};
  const nvfp4::GemmOperand b{B->codes, B->scales, B->global_scale};
  return hip_status(nvfp4::launch_gemm_ex(a, b, A->rows, B->rows, A->cols, (int)out_kind, D, ldd, amax_out,
                                          static_cast<float*>(workspace), (hipStream_t)hip_stream), "gemm_ex");
}

int nvfp4_grouped_gemm(int64_t G, const int64_t* m_offsets, const nvfp4_tensor* A,
                       const nvfp4_tensor* B, int64_t N, float* D, int64_t ldd, void* workspace,
                       size_t ws_bytes, void* hip_stream) {
  (void)workspace;
  (void)ws_bytes;
  int st;
  if (G < 1) return fail(NVFP4_ERR_INVALID, "G (%lld) must be >= 1", (long long)G);
  if (!m_offsets) return fail(NVFP4_ERR_INVALID, "m_offsets is NULL");
  if ((st = check_operand(A, "A")) || (st = check_operand(B, "B"))) return st;
  if (A->cols != B->cols) return fail(NVFP4_ERR_INVALID, "K mismatch: A has %lld, B has %lld", (long long)A->cols, (long long)B->cols);
  if (N < 1 || B->rows != G * N) return fail(NVFP4_ERR_INVALID, "B rows (%lld) must equal G*N (%lld)", (long long)B->rows, (long long)(G * N));
  if (!D && A->rows > 0) return fail(NVFP4_ERR_INVALID, "D is NULL");   // an empty D is never written
  if (ldd < N) return fail(NVFP4_ERR_INVALID, "ldd (%lld) < N (%lld)", (long long)ldd, (long long)N);
  const nvfp4::GemmOperand a{A->codes, A->scales, A->global_scale};
  const nvfp4::GemmOperand b{B->codes, B->scales, B->global_scale};
  return hip_status(nvfp4::launch_grouped_gemm(G, m_offsets, a, b, A->rows, N, A->cols, D, ldd,
                                               (hipStream_t)hip_stream), "grouped gemm");
}

int nvfp4_grouped_gemm_k(int64_t G, const int64_t* k_offsets, const nvfp4_tensor* A,
                         const nvfp4_tensor* B, float* D, int64_t ldd, void* hip_stream) {
  int st;
  if (G < 1) return fail(NVFP4_ERR_INVALID, "G (%lld) must be >= 1", (long long)G);
  if (!k_offsets) return fail(NVFP4_ERR_INVALID, "k_offsets is NULL");
  if ((st = check_operand(A, "A")) || (st = check_operand(B, "B"))) return st;
  if (A->cols != B->cols) return fail(NVFP4_ERR_INVALID, "K mismatch: A has %lld, B has %lld", (long long)A->cols, (long long)B->cols);
  if (A->cols % 64) return fail(NVFP4_ERR_UNSUPPORTED, "K (%lld) must be a multiple of 64", (long long)A->cols);
  if (!D && A->rows > 0 && B->rows > 0) return fail(NVFP4_ERR_INVALID, "D is NULL");   // an empty D is never written
  if (ldd < B->rows) return fail(NVFP4_ERR_INVALID, "ldd (%lld) < N (%lld)", (long long)ldd, (long long)B->rows);
  const nvfp4::GemmOperand a{A->codes, A->scales, A->global_scale};
  const nvfp4::GemmOperand b{B->codes, B->scales, B->global_scale};
  return hip_status(nvfp4::launch_grouped_gemm_k(G, k_offsets, a, b, A->rows, B->rows, A->cols, D, ldd,
                                                 (hipStream_t)hip_stream), "grouped gemm (K groups)");
}

int nvfp4_dequantize(const nvfp4_tensor* q, const int64_t* segments, int64_t nseg, float* y,
                     void* hip_stream) {
  int st;
  if ((st = check_operand(q, "q"))) return st;
  if (q->rows == 0 || q->cols == 0) return NVFP4_OK;
  if (!y) return fail(NVFP4_ERR_INVALID, "y is NULL");
  if (nseg < 1 || (!segments && nseg != 1)) return fail(NVFP4_ERR_INVALID, "bad segment table (nseg=%lld)", (long long)nseg);
  return hip_status(nvfp4::launch_dequantize(q->codes, q->scales, q->global_scale, segments, nseg,
                                             q->rows, q->cols, y, (hipStream_t)hip_stream), "dequantize");
}

}  // extern "C"
