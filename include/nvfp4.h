/*
 * nvfp4.h - C ABI of libnvfp4: NVFP4 block quantization and block-scaled GEMMs on MI355X.
 *
 * The format (from "Nemotron NVFP4" explainer, ai.thesatyajit.com, section "What NVFP4
 * actually is"): every element is a 4-bit E2M1 float (1 sign, 2 exponent, 1 mantissa bit),
 * every 16 consecutive elements share one FP8 E4M3 scale, and the whole tensor shares one
 * FP32 scale, 4.5 bits per element in total. Activations and gradients use 1x16 blocks,
 * weights use 16x16 blocks (artiverse.ca "NVIDIA's 4-bit floating point pushes AI training
 * limits", stabilizer paragraph); gradients are rounded stochastically, everything else to
 * nearest (same page; explainer section "Why 4-bit training normally falls apart - and the
 * three fixes"); the weight-gradient GEMM's operands go through a 16-point random-sign
 * Hadamard transform first (same explainer section).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers on the current HIP device. The caller
 *     allocates every buffer and owns it; the library allocates nothing and keeps no state
 *     between calls, so calls are re-entrant on different streams.
 *   - All work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL = the null
 *     stream). The library never synchronizes; a device fault surfaces at the caller's next
 *     synchronization.
 *   - Arguments are validated on the host before anything is enqueued. On any non-OK status
 *     nothing was enqueued (except NVFP4_ERR_HIP, where a launch itself failed) and
 *     nvfp4_last_error() describes the problem (thread-local string).
 *   - Device-resident arguments (segment/offset tables, amax values) cannot be checked on the
 *     host; their preconditions are stated per function. Violating them gives unspecified
 *     output but never an out-of-bounds access: kernels clamp table lookups.
 *   - Non-finite inputs (Inf/NaN) are outside the contract: outputs are unspecified, the
 *     kernels still terminate normally.
 *   - Empty tensors are valid: with no rows (or an output without rows or columns) nothing is
 *     read or written and the buffer pointers may be NULL; the amax of an empty tensor is 0
 *     (amax_out is still written).
 *
 * NVFP4 tensor layout (nvfp4_tensor), for a logical matrix [rows, cols] quantized along cols:
 *   codes        uint8 [rows, cols/2] row-major; element 2i in the low nibble, 2i+1 in the
 *                high nibble; nibble = sign<<3 | exponent<<1 | mantissa (E2M1, bias 1).
 *   scales       uint8 [rows, cols/16] row-major E4M3 (OCP "FN": bias 7, max 448) codes.
 *                A 16x16 weight tile stores its one scale in each of its 16 rows.
 *   global_scale float [nseg] decode scale s_dec = amax/2688 per segment (1.0 if amax = 0).
 *   Dequantized value: e2m1(code) * e4m3(scale) * global_scale[segment of row].
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID = -1,      /* bad pointer, shape, enum or size                     */
  NVFP4_ERR_UNSUPPORTED = -2,  /* valid request this library does not implement        */
  NVFP4_ERR_WORKSPACE = -3,    /* workspace missing or smaller than nvfp4_workspace_size */
  NVFP4_ERR_HIP = -4           /* a HIP launch failed (message holds hipGetErrorString) */
} nvfp4_status;

typedef enum { NVFP4_IN_BF16 = 0, NVFP4_IN_FP32 = 1 } nvfp4_dtype;
typedef enum { NVFP4_BLOCK_1X16 = 0, NVFP4_BLOCK_16X16 = 1 } nvfp4_block;
typedef enum { NVFP4_ROUND_RN = 0, NVFP4_ROUND_SR = 1 } nvfp4_round;
typedef enum {
  NVFP4_OP_QUANTIZE = 0, NVFP4_OP_RHT_QUANTIZE = 1, NVFP4_OP_GEMM = 2,
  NVFP4_OP_GROUPED_GEMM = 3, NVFP4_OP_AMAX_PAIR = 4, NVFP4_OP_GEMM_EX = 5
} nvfp4_op;
/* Output of nvfp4_gemm_ex: FP32, FP32 added to what D holds, or BF16. */
typedef enum { NVFP4_OUT_FP32 = 0, NVFP4_OUT_FP32_ACCUMULATE = 1, NVFP4_OUT_BF16 = 2 } nvfp4_out;

typedef struct nvfp4_tensor {
  uint8_t* codes;        /* device, [rows, cols/2]                       */
  uint8_t* scales;       /* device, [rows, cols/16]                      */
  float* global_scale;   /* device, [nseg] (1 for an unsegmented tensor) */
  int64_t rows;
  int64_t cols;          /* the quantized (contraction) dimension, % 16 == 0 */
} nvfp4_tensor;

/* MXFP4 tensor [rows, cols] quantized along cols: codes as nvfp4_tensor, one E8M0 scale per
 * 32 elements (value 2^(code - 127)), no tensor-level scale. The scales are stored K step by
 * K step: scale j of row r (elements 32j .. 32j+31) at byte ((j / 4) * rows + r) * 4 + j % 4,
 * ceil(cols/128) * rows * 4 bytes, so the four scales of one 128-element step of all rows are
 * contiguous (one DMA request per 32 rows in the GEMM, conflict-free reads in LDS); bytes past
 * a row's last block (cols % 128 != 0) are left unwritten. */
typedef struct mxfp4_tensor {
  uint8_t* codes;        /* device, [rows, cols/2]                     */
  uint8_t* scales;       /* device, [ceil(cols/128), rows, 4] (above)  */
  int64_t rows;
  int64_t cols;          /* % 32 == 0 */
} mxfp4_tensor;

/*
 * nvfp4_quantize - two-level block quantization of x[rows, cols] along cols.
 * Defined by: "Nemotron NVFP4" explainer, "What NVFP4 actually is" (E2M1 elements, one E4M3
 * scale per 16 elements, one FP32 tensor scale) and "Why 4-bit training normally falls
 * apart - and the three fixes" (2D weight blocks; stochastic rounding for gradients).
 *
 *   x         device BF16 or FP32 (dt), element (r, c) at x[r*ld + c]; ld >= cols.
 *   blk       NVFP4_BLOCK_1X16 (scale per 16 consecutive elements of a row) or
 *             NVFP4_BLOCK_16X16 (one scale per aligned 16x16 tile; rows % 16 == 0).
 *   rnd       NVFP4_ROUND_RN, or NVFP4_ROUND_SR (1x16 only): element j of the block with
 *             row-major index b uses byte j%4 of word j/4 of Philox4x32-10 with key
 *             (lo32 seed, hi32 seed) and counter (lo32 b, hi32 b, lo32 offset, hi32 offset);
 *             it rounds up iff frac + byte/256 >= 1.
 *   segments  NULL (nseg must be 1) or device int64[nseg+1] row offsets with
 *             segments[0] = 0 <= ... <= segments[nseg] = rows (non-decreasing; multiples
 *             of 16 for 16X16). Each segment gets its own amax and global scale (expert
 *             stacks of a mixture-of-experts layer).
 *   amax_in   NULL, or device float[nseg] holding max|x| per segment; then the amax pass is
 *             skipped and no workspace is needed.
 *   out       codes/scales/global_scale as documented above; out->rows == rows,
 *             out->cols == cols.
 *   out_t     NULL, or (16X16) a second tensor receiving the quantization of x^T ([cols, rows]
 *             along rows): the same tile scales and codes, transposed. With segments (a
 *             stack of nseg expert weights) they must be nseg equal blocks of n = rows/nseg
 *             rows (n % 16 == 0; the table must match) and out_t is [nseg*cols, n]: rows
 *             g*cols .. hold expert g's transpose, with global_scale[g] (the operand of the
 *             grouped activation-gradient GEMM).
 *   workspace device scratch of at least nvfp4_workspace_size(NVFP4_OP_QUANTIZE, rows,
 *             cols, nseg) bytes, 256-byte aligned; may be NULL when amax_in is given.
 * Errors: NVFP4_ERR_INVALID (null pointers, cols % 16, rows % 16 for 16X16, ld < cols, bad
 * enum, nseg < 1, segments == NULL with nseg != 1, out_t without 16X16, tensor shape
 * mismatch), NVFP4_ERR_UNSUPPORTED (SR with 16X16, out_t with unequal or misaligned segments),
 * NVFP4_ERR_WORKSPACE, NVFP4_ERR_HIP.
 */
int nvfp4_quantize(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                   nvfp4_block blk, nvfp4_round rnd, uint64_t seed, uint64_t offset,
                   const int64_t* segments, int64_t nseg, const float* amax_in,
                   nvfp4_tensor* out, nvfp4_tensor* out_t,
                   void* workspace, size_t ws_bytes, void* hip_stream);

/*
 * nvfp4_quantize_noalloc - nvfp4_quantize for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation. Same
 * arguments, results and errors as nvfp4_quantize minus the workspace: the amax pass keeps its
 * partial (or per-segment) maxima in a static device array of the library, 64 KiB per device,
 * held until the process ends. The call allocates nothing (its first call on a device looks up
 * that device's array once); anything that must start at zero is cleared by a kernel, not a
 * memset, so the call can be captured in a graph.
 *   nseg       at most 16384 (NVFP4_ERR_UNSUPPORTED beyond, nothing enqueued).
 * Every call on one device shares that device's array: calls that overlap on one device (on
 * different streams, or from several threads without ordering) race and give unspecified
 * results. Calls ordered on one stream are safe.
 */
int nvfp4_quantize_noalloc(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                           nvfp4_block blk, nvfp4_round rnd, uint64_t seed, uint64_t offset,
                           const int64_t* segments, int64_t nseg, const float* amax_in,
                           nvfp4_tensor* out, nvfp4_tensor* out_t, void* hip_stream);

/*
 * nvfp4_rht_quantize - random Hadamard transform along tokens, then 1x16 quantization of
 * the transposed result. Defined by: "Nemotron NVFP4" explainer, "Why 4-bit training
 * normally falls apart - and the three fixes" (a random Hadamard matrix on the wgrad inputs,
 * undone analytically inside the GEMM) and thelatentdaily "What matters for NVFP4
 * training?", "A methodological warning" (random sign vectors of the rotations).
 *
 *   x          device BF16/FP32 [tokens, cols], element (t, c) at x[t*ld + c];
 *              tokens % 16 == 0.
 *   sign_mask  bit j set => sign -1 on element j of every 16-token block. Both operands of
 *              one wgrad GEMM must use the same mask so that the transform cancels.
 *   transform  for column c and block t: y_i = rn32(1/4 * sum_j H[i][j] s_j x[16t+j, c]),
 *              H[i][j] = (-1)^popcount(i & j): the exact sum rounded once to FP32 (nearest,
 *              ties to even), +0 for an exactly zero sum, for every input (blocks of any
 *              exponent spread; a sum beyond the FP32 range gives infinity).
 *   out        tensor [cols, tokens]: row c holds column c's transformed values quantized in
 *              1x16 blocks along tokens (out->rows == cols, out->cols == tokens).
 *   rnd/seed/offset as for nvfp4_quantize (SR block index is over the output [cols, tokens]).
 *   segments   NULL (nseg must be 1) or device int64[nseg+1] TOKEN offsets, multiples of 16,
 *              non-decreasing from 0 to tokens: the tokens routed to each expert of a
 *              mixture-of-experts layer, whose weight gradients are separate GEMMs over their
 *              own tokens (nvfp4_grouped_gemm_k). Each token range gets its own amax (over its
 *              transformed values) and global scale: out->global_scale[nseg]; out's column
 *              range of segment g uses global_scale[g]. A 16-token block belongs to the
 *              segment of its first token; unchecked device data, never an out-of-bounds
 *              access.
 *   amax_in    NULL or device float[nseg] = max|y| of the transformed values per segment.
 *   workspace  >= nvfp4_workspace_size(NVFP4_OP_RHT_QUANTIZE, tokens, cols, nseg) bytes
 *              unless amax_in is given.
 * Errors: as nvfp4_quantize (tokens % 16, cols < 1, ld < cols, nseg < 1, segments == NULL
 * with nseg != 1, ...).
 */
int nvfp4_rht_quantize(const void* x, nvfp4_dtype dt, int64_t tokens, int64_t cols, int64_t ld,
                       uint16_t sign_mask, nvfp4_round rnd, uint64_t seed, uint64_t offset,
                       const int64_t* segments, int64_t nseg, const float* amax_in,
                       nvfp4_tensor* out, void* workspace, size_t ws_bytes, void* hip_stream);

/*
 * mxfp4_quantize - MXFP4 quantization of x[rows, cols] along cols, the format the pages set
 * against NVFP4 ("Nemotron NVFP4" explainer, "What NVFP4 actually is": E2M1 elements, one
 * power-of-two E8M0 scale per 32 elements, 4.25 bits per element, no tensor scale). The
 * scale rule is the OCP Microscaling v1.0 conversion: shared exponent e = floor(log2(block
 * amax)) - 2 clamped to [-127, 127] (-127 for an all-zero block), element = E2M1(x * 2^-e)
 * rounded to nearest even (RN) or stochastically with the Philox bytes of nvfp4_quantize's SR
 * (16-element half-block index b = (row*cols + col)/16), saturating at 6. One pass, no
 * workspace.
 *   x    device BF16 or FP32 (dt), element (r, c) at x[r*ld + c]; 16-byte aligned, ld a
 *        multiple of 16 bytes' worth of elements.
 *   out  codes/scales, out->rows == rows, out->cols == cols (cols % 32 == 0).
 * Errors: NVFP4_ERR_INVALID (null pointers, shapes, enums), NVFP4_ERR_UNSUPPORTED (alignment),
 * NVFP4_ERR_HIP.
 */
int mxfp4_quantize(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                   nvfp4_round rnd, uint64_t seed, uint64_t offset, mxfp4_tensor* out,
                   void* hip_stream);

/*
 * mxfp4_quantize_columns - MXFP4 quantization of x's columns: out [cols, rows] holds x^T
 * quantized along its rows, exactly mxfp4_quantize of the transposed tensor (same scale rule,
 * rounding and SR counters, with the half-block index b = (out_row*rows + out_col)/16 of the
 * output), without materializing x^T. The activation- and weight-gradient GEMMs contract W,
 * dY and X over their other dimension ("Nemotron NVFP4" explainer, "What NVFP4 actually is":
 * the MXFP4 comparison format, 32-element blocks along the contraction).
 *   x    device BF16 or FP32 [rows, cols], element (r, c) at x[r*ld + c]; element pairs aligned
 *        (ld any); rows % 32 == 0.
 *   out  out->rows == cols, out->cols == rows; codes 16-byte, scales 8-byte aligned.
 * Errors: NVFP4_ERR_INVALID (null pointers, shapes, rows % 32, enums, alignment of out),
 * NVFP4_ERR_UNSUPPORTED (misaligned x), NVFP4_ERR_HIP.
 */
int mxfp4_quantize_columns(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                           nvfp4_round rnd, uint64_t seed, uint64_t offset, mxfp4_tensor* out,
                           void* hip_stream);

/*
 * mxfp4_gemm - D[M, N] (FP32, row stride ldd) = A[M, K] * B[N, K]^T with both operands MXFP4
 * (mxfp4_quantize along K): the comparison format of the pages ("Nemotron NVFP4" explainer,
 * "What NVFP4 actually is") on gfx950's block-scaled FP4 matrix instruction, which applies
 * the E8M0 scales of each 32-element block itself. Products exact, FP32 accumulation.
 *   A: rows = M, cols = K; B: rows = N, cols = K (same K, K % 128 == 0); ldd >= N; each
 *   operand's codes below 2 GiB, codes 16-byte and scales 4-byte aligned.
 * Errors: NVFP4_ERR_INVALID (null pointers, K mismatch, cols % 32, ldd < N, alignment),
 * NVFP4_ERR_UNSUPPORTED (K % 128, operand size), NVFP4_ERR_HIP.
 */
int mxfp4_gemm(const mxfp4_tensor* A, const mxfp4_tensor* B, float* D, int64_t ldd, void* hip_stream);

/*
 * nvfp4_rht_rows_quantize - the rowwise random-sign Hadamard transform then 1x16 quantization
 * along the rows: every 16-element block of a row goes through y = 1/4 * H16 * diag(s) * v
 * (the butterfly and rounding of nvfp4_rht_quantize, signs from sign_mask) and is quantized
 * as nvfp4_quantize's 1x16 blocks, with the tensor scale from max|y|. This is the activation
 * gradient of the Mosaic variant's activation-gradient GEMM (thelatentdaily "What matters for
 * NVFP4 training?": Hadamard transforms on both backward GEMMs, 1D weight quantization): with
 * B = nvfp4_rht_quantize(W, same mask) (W^T transformed along the output features), the
 * product of the two equals dY * W since the transform is orthogonal.
 *   x          device BF16/FP32 [rows, cols], cols % 16 == 0, 16-byte aligned rows.
 *   rnd, seed, offset  as nvfp4_quantize (block index b = row*(cols/16) + col/16).
 *   amax_in    NULL or device float[1] = max|y| (nvfp4_amax with rht = 2); then no workspace.
 *   out        [rows, cols], global_scale[1].
 *   workspace  nvfp4_workspace_size(NVFP4_OP_QUANTIZE, rows, cols, 1) bytes when amax_in is NULL.
 * Errors: NVFP4_ERR_INVALID, NVFP4_ERR_UNSUPPORTED (alignment), NVFP4_ERR_WORKSPACE, NVFP4_ERR_HIP.
 */
int nvfp4_rht_rows_quantize(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                            uint16_t sign_mask, nvfp4_round rnd, uint64_t seed, uint64_t offset,
                            const float* amax_in, nvfp4_tensor* out, void* workspace, size_t ws_bytes,
                            void* hip_stream);

/*
 * nvfp4_gemm - D[M, N] (FP32, row stride ldd) = A[M, K] * B[N, K]^T with both operands
 * NVFP4 (each quantized along K), products accumulated in FP32, scaled by
 * A->global_scale[0] * B->global_scale[0]. Covers the forward, activation-gradient and
 * weight-gradient GEMMs of a linear layer (artiverse.ca "NVIDIA's 4-bit floating point
 * pushes AI training limits", paragraph on which parts run in 4-bit).
 *   A: rows = M, cols = K; B: rows = N, cols = K (same K, % 16 == 0); ldd >= N.
 * Errors: NVFP4_ERR_INVALID (null pointers, K mismatch, K % 16, ldd < N),
 * NVFP4_ERR_UNSUPPORTED (an operand's codes above 2 GiB: the kernels use 32-bit buffer
 * offsets; the same limit holds for every GEMM entry point), NVFP4_ERR_HIP.
 */
int nvfp4_gemm(const nvfp4_tensor* A, const nvfp4_tensor* B, float* D, int64_t ldd,
               void* hip_stream);

/*
 * nvfp4_gemm_ex - nvfp4_gemm with the outputs a linear layer needs around its three GEMMs
 * (artiverse.ca "NVIDIA's 4-bit floating point pushes AI training limits", paragraph on which
 * parts run in 4-bit: the GEMMs take NVFP4 operands, the layer's other tensors stay in higher
 * precision): the forward output and the activation gradient handed on in BF16, the weight
 * gradient accumulated into an FP32 main gradient, and the output's amax produced by the GEMM
 * itself, so the next quantization of D (amax_in) is a single pass.
 *   A, B       as nvfp4_gemm (rows M and N, same K, % 16 == 0).
 *   D          device [M, N] with row stride ldd >= N elements:
 *              NVFP4_OUT_FP32             float, D = s_A s_B A B^T (as nvfp4_gemm);
 *              NVFP4_OUT_FP32_ACCUMULATE  float, D = D + s_A s_B A B^T (one FP32 addition per
 *                                         element; D must hold finite values);
 *              NVFP4_OUT_BF16             bfloat16 bits (uint16), the FP32 result rounded to
 *                                         nearest, ties to even.
 *   amax_out   NULL, or device float[1] receiving max |D| over the values as stored (after the
 *              BF16 rounding; after the addition when accumulating). The library clears it.
 *   workspace  device scratch of nvfp4_workspace_size(NVFP4_OP_GEMM_EX, M, N, 1) bytes, sized
 *              for the current device, 256-byte aligned (0 bytes, NULL allowed, when the
 *              tiles fill whole rounds of the device's compute units, or leave a last round of
 *              at most a quarter of them, which is then computed as 64-column quarters of its
 *              tiles over all of K): a partial last round of more than a quarter and at most
 *              half of the compute units is split along K and the two halves' sums meet there
 *              (lower half first), so D is reproducible.
 * The result is deterministic for a given device. Errors: NVFP4_ERR_INVALID (null pointers,
 * K mismatch, K % 16, ldd < N, bad kind, misaligned D), NVFP4_ERR_WORKSPACE, NVFP4_ERR_HIP.
 */
int nvfp4_gemm_ex(const nvfp4_tensor* A, const nvfp4_tensor* B, void* D, int64_t ldd, nvfp4_out out_kind,
                  float* amax_out, void* workspace, size_t ws_bytes, void* hip_stream);

/*
 * nvfp4_grouped_gemm - one GEMM per group (mixture-of-experts expert GEMMs; "Nemotron
 * NVFP4" explainer, "The model underneath" and "The honest part: this is not end-to-end
 * FP4": the expert GEMMs carry most of the compute and run in NVFP4).
 *   m_offsets  device int64[G+1], 0 = m_offsets[0] <= ... <= m_offsets[G] = A->rows.
 *   A          [sum M_g, K], global_scale[G] (one per group, as produced by nvfp4_quantize
 *              with segments = m_offsets).
 *   B          [G*N, K] stacked per-group weights, global_scale[G].
 *   D          [sum M_g, N] FP32, row stride ldd: rows of group g hold A_g * B_g^T scaled by
 *              A->global_scale[g] * B->global_scale[g]. Empty groups are allowed.
 *   workspace  may be NULL (nvfp4_workspace_size returns 0 for this op).
 * Errors: NVFP4_ERR_INVALID (G < 1, B->rows != G*N, K mismatch, ...), NVFP4_ERR_HIP.
 */
int nvfp4_grouped_gemm(int64_t G, const int64_t* m_offsets, const nvfp4_tensor* A,
                       const nvfp4_tensor* B, int64_t N, float* D, int64_t ldd,
                       void* workspace, size_t ws_bytes, void* hip_stream);

/*
 * nvfp4_grouped_gemm_k - GEMMs grouped along the contraction dimension, as the MoE weight
 * gradient needs: expert g's gradient sums over the tokens routed to it ("Nemotron NVFP4"
 * explainer, "The model underneath": expert layers; "Why 4-bit training normally falls apart -
 * and the three fixes": the weight-gradient GEMM). For g < G:
 *   D[g*M + m, n] = A.global_scale[g] * B.global_scale[g] *
 *                   sum over k in [k_offsets[g], k_offsets[g+1]) of a[m, k] * b[n, k]
 * with a, b the E2M1 x E4M3 values, FP32 accumulation.
 *   A          NVFP4 [M, K], B NVFP4 [N, K], quantized along K, each with global_scale[G]
 *              (one per group of K).
 *   k_offsets  device int64[G+1], non-decreasing, multiples of 64 (unchecked device data:
 *              values are clamped into [0, K]; misaligned ones give unspecified output).
 *   D          device FP32 [G*M, N] with row stride ldd >= N; an empty group writes zeros.
 * Errors: NVFP4_ERR_INVALID (G < 1, NULL pointers, K mismatch, ldd < N), NVFP4_ERR_UNSUPPORTED
 * (K % 64 != 0), NVFP4_ERR_HIP.
 */
int nvfp4_grouped_gemm_k(int64_t G, const int64_t* k_offsets, const nvfp4_tensor* A,
                         const nvfp4_tensor* B, float* D, int64_t ldd, void* hip_stream);

/*
 * nvfp4_amax - max|x| of x[rows, cols] (row stride ld), per row segment, into device
 * amax_out[nseg]: the first level of the two-level scale ("Nemotron NVFP4" explainer, "What
 * NVFP4 actually is": one FP32 scale per tensor). With rht = 1 the maximum is taken over the
 * Hadamard-transformed tensor of nvfp4_rht_quantize (rows = tokens; segments are token
 * ranges as there, multiples of 16); with rht = 2 over the rowwise-transformed tensor of
 * nvfp4_rht_rows_quantize (no segments). Useful to precompute amax_in.
 *   workspace  device scratch of nvfp4_workspace_size(rht == 1 ? NVFP4_OP_RHT_QUANTIZE :
 *              NVFP4_OP_QUANTIZE, rows, cols, nseg) bytes, 256-byte aligned, for the partial
 *              maxima of an unsegmented tensor; may be NULL with segments (amax_out[nseg] is
 *              then written directly).
 * Errors: as nvfp4_quantize; NVFP4_ERR_UNSUPPORTED for rht = 2 with segments.
 */
int nvfp4_amax(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
               const int64_t* segments, int64_t nseg, int rht, uint16_t sign_mask,
               float* amax_out, void* workspace, size_t ws_bytes, void* hip_stream);

/*
 * nvfp4_amax_pair - both tensor maxima of x[tokens, cols] (row stride ld) from one read:
 * amax_out[0] = max|x| (the tensor scale of its 1x16 quantization, as nvfp4_amax with
 * rht = 0) and amax_out[1] = max|y| over the Hadamard-transformed tensor of
 * nvfp4_rht_quantize with this sign_mask (as nvfp4_amax with rht = 1). A tensor that feeds
 * both an fprop/dgrad GEMM and the wgrad GEMM is quantized both ways ("Nemotron NVFP4"
 * explainer, "Why 4-bit training normally falls apart - and the three fixes": only the wgrad
 * operands are transformed); each value can be passed as amax_in of the matching quantize.
 *   x          device, BF16 or FP32; tokens % 16 == 0; element pairs aligned (ld any).
 *   amax_out   device float[2].
 *   workspace  device scratch of nvfp4_workspace_size(NVFP4_OP_AMAX_PAIR, ...) bytes,
 *              256-byte aligned.
 * Both values are exact maxima, so they equal the two nvfp4_amax results bit for bit.
 * Errors: NVFP4_ERR_INVALID (NULL pointer, bad dtype/shape, tokens % 16 != 0),
 * NVFP4_ERR_UNSUPPORTED (misaligned x), NVFP4_ERR_WORKSPACE, NVFP4_ERR_HIP.
 */
int nvfp4_amax_pair(const void* x, nvfp4_dtype dt, int64_t tokens, int64_t cols, int64_t ld,
                    uint16_t sign_mask, float* amax_out, void* workspace, size_t ws_bytes,
                    void* hip_stream);

/* Bytes of device workspace `op` needs for the given shape (0 if none). The library allocates
 * no memory itself (caller-owned buffers, see the conventions above), so the partial maxima of
 * the tensor amax (the FP32 tensor scale of "Nemotron NVFP4" explainer, "What NVFP4 actually
 * is") and the K-split partial sums of nvfp4_gemm_ex live in a workspace the caller sizes with
 * this call. ops: nvfp4_op; rows/cols/nseg as in the call the workspace is for. */
size_t nvfp4_workspace_size(int op, int64_t rows, int64_t cols, int64_t nseg);

/* Thread-local description of the last non-OK status returned on this thread: the error
 * behaviour shared by every entry point (host validation before anything is enqueued). The
 * string stays valid until the thread's next failing call. */
const char* nvfp4_last_error(void);

/*
 * nvfp4_dequantize - test helper: the decoded value of every element, the two-level scale of
 * "Nemotron NVFP4" explainer, "What NVFP4 actually is" (E2M1 element times its block's E4M3
 * scale times the tensor's FP32 scale): y[r, c] = rn32(e2m1 * e4m3 * global_scale[segment(r)])
 * (e2m1 * e4m3 is exact), y FP32 [rows, cols] contiguous. segments as for nvfp4_quantize
 * (NULL, nseg = 1 allowed). Errors: NVFP4_ERR_INVALID (null pointers, shapes), NVFP4_ERR_HIP.
 */
int nvfp4_dequantize(const nvfp4_tensor* q, const int64_t* segments, int64_t nseg, float* y,
                     void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H */
