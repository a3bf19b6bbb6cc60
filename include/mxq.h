/*
 * mxq.h -- C ABI of the MI355X (gfx950) block-scaled weight-quantization library.
 *
 * Five entry points make up the path:
 *   mxq_fake_quantize_mxfp4     per-1x32 MXFP4 projection, output in the input dtype
 *   mxq_mxfp4_to_mxfp8_row      direct MXFP8 rowwise lift (E4M3 payload + E8M0 codes)
 *   mxq_mxfp4_to_fp8_block128   direct 128x128 blockwise FP8 (E4M3 payload + tile codes)
 *   mxq_export_mxfp8            unpadded (*shape[:-1], ceil(K/32)) E8M0 scale export
 *   mxq_dequantize              FP8 payload + E8M0 codes -> bf16 / fp32
 * variants of them:
 *   mxq_fake_quantize_mxfp4_with_mxfp8_row    projection + row lift in one pass
 *   mxq_mxfp4_to_mxfp8_row_guarded,
 *   mxq_mxfp4_to_fp8_block128_guarded         the direct conversions behind a device no-op flag
 *   mxq_mxfp4_to_mxfp8_row_grouped, mxq_fake_quantize_mxfp4_grouped,
 *   mxq_mxfp4_to_fp8_block128_grouped,
 *   mxq_dequantize_grouped                    the row lift / projection / fold / decode of a list
 *                                             of weights in few launches
 * the packed MXFP4 deployment format:
 *   mxq_quantize_mxfp4, mxq_dequantize_mxfp4,
 *   mxq_mxfp4_packed_to_mxfp8_row, mxq_mxfp4_packed_to_fp8_block128,
 *   mxq_quantize_mxfp4_grouped (the encode of a list of weights in few launches)
 * and MXFP8 columnwise (32x1) from the decomposition:
 *   mxq_mxfp4_to_mxfp8_col, mxq_mxfp4_to_mxfp8_row_col (row and column in one pass),
 *   and their no-op-flag-gated forms mxq_mxfp4_to_mxfp8_col_guarded,
 *   mxq_mxfp4_to_mxfp8_row_col_guarded
 *
 * Sources, by page title and section:
 *   [QAT] "[PyTorch] MXFP4 weight QAT on MXFP8 and FP8 block-scaling recipes"
 *         (TransformerEngine pull request 3264): Description, Test results (B200),
 *         Known limitations.
 *   [EXP] "MXFP8TensorStorage.export_components()" (TransformerEngine pull request
 *         3790): Description.
 *
 * Conventions for every entry point:
 *   - A matrix is [rows, K]: leading dimensions are flattened into rows and the
 *     last dimension K is contiguous.  Every ld / scale_ld / tile_ld is a row
 *     stride counted in elements of that buffer.
 *   - All pointers are device pointers.  The caller owns every buffer; the
 *     library never allocates, frees or keeps a pointer, holds no state and is
 *     safe to call from several host threads.
 *   - Work is enqueued on `stream` (0 = the null stream) and is asynchronous.
 *     Argument errors are detected on the host and returned before anything is
 *     enqueued; no kernel asserts on the device.
 *   - rows == 0 or K == 0 returns MXQ_OK and enqueues nothing.
 *   - Results are bit-exact and do not depend on the build's floating-point
 *     flags: the scale exponents are integer arithmetic on bit patterns, and the
 *     kernels set the wave's denormal mode before using the gfx950 scaled
 *     conversions.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of a high-precision buffer.  fp16 exists only to be rejected:
 * the MXFP4 grid exceeds its range ([QAT] Description, STE paragraph, and
 * Known limitations). */
typedef enum { MXQ_BF16 = 0, MXQ_FP32 = 1, MXQ_FP16 = 2 } mxq_dtype;

/* FP8 payload format: OCP E4M3 "FN" (bias 7, max 448, NaN = S.1111.111, no Inf)
 * or E5M2 (bias 15, IEEE Inf/NaN) -- the torch.float8_e4m3fn / float8_e5m2 views
 * of [EXP] Description. */
typedef enum { MXQ_E4M3 = 0, MXQ_E5M2 = 1 } mxq_fp8;

/* Where a payload element's E8M0 code lives: one per 1x32 block of a row
 * (scale[r*scale_ld + c/32]), one per 128x128 tile anchored at (0,0)
 * (scale[(r/128)*scale_ld + c/128]), or one per 32x1 block of a column
 * anchored at row 0 (scale[(r/32)*scale_ld + c]). */
typedef enum { MXQ_SCALE_ROW_1X32 = 0, MXQ_SCALE_TILE_128X128 = 1, MXQ_SCALE_COL_32X1 = 2 } mxq_scale_layout;

/* Status codes. */
enum {
  MXQ_OK = 0,
  MXQ_ERR_NULL = 1,             /* a required pointer is NULL (non-empty shape) */
  MXQ_ERR_SHAPE = 2,            /* negative dims, ld < K, scale_ld / tile_ld too small, too many steps
                                   for one launch, or a matrix spanning 2^56 bytes or more (or past the
                                   end of the address space) */
  MXQ_ERR_DTYPE = 3,            /* fp16 or an unknown dtype / format / layout */
  MXQ_ERR_NO_ROWWISE_DATA = 4,  /* export without payload or scale storage ([EXP]: ValueError) */
  MXQ_ERR_ALIAS = 5,            /* an output overlaps an input (other than the allowed exact in-place) */
  MXQ_ERR_HIP = 6               /* the HIP runtime refused a launch: hipGetLastError() was not
                                   hipSuccess right after it.  That includes an error left pending by
                                   an earlier HIP call on the calling thread, which the call then
                                   consumes, as hipGetLastError() does. */
};

/* Human-readable text of a status code (static storage; never NULL). */
const char* mxq_status_string(int status);

/*
 * MXFP4 projection (fake quantization), [QAT] Description, conversion mode 1.
 * For each 1x32 block of a row (the last block of a row may be shorter and
 * keeps its own scale, [EXP] Description): amax = max |x|; scale exponent
 * e = clamp(ceil(log2(amax/6)), -126, 125), taken from amax's bit pattern;
 * y = RTNE_E2M1(x / 2^e) * 2^e, i.e. x rounded to the nearest of
 * {0, .5, 1, 1.5, 2, 3, 4, 6} * 2^e with ties to the even E2M1 code, sign kept
 * (including -0), saturating at 6 * 2^e ([QAT] Known limitations: amax above
 * 6*2^125 saturates at the cap).  A block holding any Inf or NaN becomes all
 * canonical quiet NaN (0x7FC0 / 0x7FC00000) ([QAT] Test results: non-finite
 * block poisoning).  amax = 0 uses e = -126.
 *   x    [rows, K] bf16 or fp32, row stride ld_x >= K
 *   y    [rows, K] same dtype, row stride ld_y >= K.  y == x with ld_y == ld_x
 *        (in place) is allowed; any other overlap is MXQ_ERR_ALIAS.
 *   dt   MXQ_BF16 or MXQ_FP32 (MXQ_FP16 -> MXQ_ERR_DTYPE)
 */
int mxq_fake_quantize_mxfp4(const void* x, int64_t ld_x, void* y, int64_t ld_y,
                            int64_t rows, int64_t K, mxq_dtype dt, hipStream_t stream);

/*
 * Direct MXFP8 rowwise lift, [QAT] Description, conversion mode 2: a lift by a
 * fixed shift of 6 whose scale stops at UE8M0 code 0, the payload taking up the
 * rest of the shift exactly.
 * From each block's MXFP4 decomposition x ~ p * 2^e of the master weight (the
 * same e and p as mxq_fake_quantize_mxfp4): scale code = max(e + 121, 0), i.e.
 * scale 2^(e-6) clamped at 2^-127, and payload = E4M3(p * 2^min(6, e+127)),
 * which is always exact.  Decoding payload * 2^(code-127) gives back the
 * projection bit for bit.  A poisoned block gets code 255 and payload 0x7F.
 *   x         [rows, K] bf16 or fp32, row stride ld_x >= K
 *   data      [rows, K] uint8 E4M3 payload, contiguous (row stride K)
 *   scale     [rows, scale_ld] uint8 E8M0 codes, scale_ld >= ceil(K/32); columns
 *             j >= ceil(K/32) (padding) are not written
 *   data and scale must not overlap x or each other (MXQ_ERR_ALIAS).
 */
int mxq_mxfp4_to_mxfp8_row(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt,
                           uint8_t* data, uint8_t* scale, int64_t scale_ld, hipStream_t stream);

/*
 * Direct 128x128 blockwise FP8, [QAT] Description, conversion mode 2: the block
 * exponents are folded into one scale per tile, 2^(largest FP4 exponent - 6)
 * with 2^-127 as its floor, and the payload is rounded to nearest-even onto
 * E4M3, subnormals included.  Tiles are anchored at (0,0) and truncated at the
 * edges.  Per tile: M = max e over its finite 1x32 blocks (-126 if none);
 * S = max(M - 6, -127); tile code = S + 127; payload = RTNE_E4M3(p * 2^(e - S))
 * with E4M3 subnormals and ties to even.  Exact while the tile's exponent
 * spread M - e is at most 14 ([QAT] Test results).  Poisoned blocks are left out
 * of M and get payload 0x7F.
 *   x          [rows, K] bf16 or fp32, row stride ld_x >= K
 *   data       [rows, K] uint8 E4M3 payload, contiguous (row stride K)
 *   tile_code  [ceil(rows/128), tile_ld] uint8 E8M0 codes, tile_ld >= ceil(K/128)
 *   data and tile_code must not overlap x or each other (MXQ_ERR_ALIAS).
 */
int mxq_mxfp4_to_fp8_block128(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt,
                              uint8_t* data, uint8_t* tile_code, int64_t tile_ld, hipStream_t stream);

/*
 * Projection and direct MXFP8 row lift in one pass over the weight: writes the
 * outputs of mxq_fake_quantize_mxfp4 (y) and of mxq_mxfp4_to_mxfp8_row (data,
 * scale) from a single read of x.  [QAT] Known limitations names a fused
 * projection + quantize kernel as future work; the results are bit-identical to
 * the two separate calls.  Arguments and rules as for those two calls (y == x
 * with ld_y == ld_x is allowed; every other overlap is MXQ_ERR_ALIAS).
 */
int mxq_fake_quantize_mxfp4_with_mxfp8_row(const void* x, int64_t ld_x, void* y, int64_t ld_y, int64_t rows,
                                           int64_t K, mxq_dtype dt, uint8_t* data, uint8_t* scale,
                                           int64_t scale_ld, hipStream_t stream);

/*
 * mxq_mxfp4_to_mxfp8_row / mxq_mxfp4_to_fp8_block128 gated by a device-side
 * no-op flag: when *noop != 0 at the time the work runs on the stream, every
 * output is left untouched.  For cached-weight updates inside a captured HIP
 * graph, where a replay must be able to keep the existing workspace ([QAT]
 * review: the CUDA-graph skip-update flag must gate the cached update).
 *   noop   device pointer to one int32, read by the kernels; required (NULL ->
 *          MXQ_ERR_NULL).  Other arguments as for the ungated calls.  The
 *          input is read either way (the kernels issue their input loads
 *          before they read the flag), so x must be valid in both cases.
 */
int mxq_mxfp4_to_mxfp8_row_guarded(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt,
                                   uint8_t* data, uint8_t* scale, int64_t scale_ld, const int32_t* noop,
                                   hipStream_t stream);
int mxq_mxfp4_to_fp8_block128_guarded(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt,
                                      uint8_t* data, uint8_t* tile_code, int64_t tile_ld, const int32_t* noop,
                                      hipStream_t stream);

/*
 * One weight of a grouped row lift: the arguments of mxq_mxfp4_to_mxfp8_row for
 * that weight (x, data and scale are device pointers).
 */
typedef struct {
  const void* x;      /* [rows, K], row stride ld_x >= K */
  int64_t ld_x;
  int64_t rows;
  int64_t K;
  uint8_t* data;      /* [rows, K] E4M3 payload, contiguous */
  uint8_t* scale;     /* [rows, scale_ld] E8M0 codes, scale_ld >= ceil(K/32); padding not written */
  int64_t scale_ld;
} mxq_row_group;

/*
 * The direct MXFP8 row lift of mxq_mxfp4_to_mxfp8_row applied to a list of
 * weights of one dtype (the experts of a grouped linear layer, [QAT] Test
 * results, end-to-end cases), in as few launches as possible: every launch
 * carries a fixed cost of a few microseconds, which dominates for small weights.
 * Results are bit-identical to one mxq_mxfp4_to_mxfp8_row call per weight.
 *   groups    HOST array of n_groups descriptors, read during the call only
 *   n_groups  >= 0; groups with rows == 0 or K == 0 are skipped
 *   Every group is checked as mxq_mxfp4_to_mxfp8_row checks its arguments (the
 *   first failing group's status is returned and nothing is enqueued).  In
 *   addition no group's data or scale may overlap any group's x, data or scale
 *   (MXQ_ERR_ALIAS); inputs may overlap each other.
 */
int mxq_mxfp4_to_mxfp8_row_grouped(const mxq_row_group* groups, int64_t n_groups, mxq_dtype dt,
                                   hipStream_t stream);

/*
 * One weight of a grouped projection: the arguments of mxq_fake_quantize_mxfp4
 * for that weight (x and y are device pointers).
 */
typedef struct {
  const void* x;      /* [rows, K], row stride ld_x >= K */
  int64_t ld_x;
  void* y;            /* [rows, K] same dtype, row stride ld_y >= K; y == x with ld_y == ld_x is in place */
  int64_t ld_y;
  int64_t rows;
  int64_t K;
} mxq_proj_group;

/*
 * The MXFP4 projection of mxq_fake_quantize_mxfp4 ([QAT] Description, conversion
 * mode 1, the default mode) applied to a list of weights of one dtype, in as
 * few launches as possible.  Results are bit-identical to one
 * mxq_fake_quantize_mxfp4 call per weight.
 *   groups    HOST array of n_groups descriptors, read during the call only
 *   n_groups  >= 0; groups with rows == 0 or K == 0 are skipped
 *   Every group is checked as mxq_fake_quantize_mxfp4 checks its arguments
 *   (the first failing group's status is returned and nothing is enqueued).
 *   In addition no group's y may overlap any other group's x or y
 *   (MXQ_ERR_ALIAS); inputs may overlap each other, and a group may be in place.
 */
int mxq_fake_quantize_mxfp4_grouped(const mxq_proj_group* groups, int64_t n_groups, mxq_dtype dt,
                                    hipStream_t stream);

/*
 * One weight of a grouped 128x128 fold: the arguments of
 * mxq_mxfp4_to_fp8_block128 for that weight (x, data and tile_code are device
 * pointers).
 */
typedef struct {
  const void* x;      /* [rows, K], row stride ld_x >= K */
  int64_t ld_x;
  int64_t rows;
  int64_t K;
  uint8_t* data;      /* [rows, K] E4M3 payload, contiguous */
  uint8_t* tile_code; /* [ceil(rows/128), tile_ld] E8M0 tile codes, tile_ld >= ceil(K/128) */
  int64_t tile_ld;
} mxq_block128_group;

/*
 * The direct 128x128 blockwise FP8 fold of mxq_mxfp4_to_fp8_block128 ([QAT]
 * Description, conversion mode 2) applied to a list of weights of one dtype,
 * in as few launches as possible.  Results are bit-identical to one
 * mxq_mxfp4_to_fp8_block128 call per weight.
 *   groups    HOST array of n_groups descriptors, read during the call only
 *   n_groups  >= 0; groups with rows == 0 or K == 0 are skipped
 *   Every group is checked as mxq_mxfp4_to_fp8_block128 checks its arguments
 *   (the first failing group's status is returned and nothing is enqueued).
 *   In addition no group's data or tile_code may overlap any group's x, data
 *   or tile_code (MXQ_ERR_ALIAS); inputs may overlap each other.
 */
int mxq_mxfp4_to_fp8_block128_grouped(const mxq_block128_group* groups, int64_t n_groups, mxq_dtype dt,
                                      hipStream_t stream);

/*
 * MXFP8 columnwise from the MXFP4 decomposition ([QAT] Description, conversion
 * mode 2, and its MXFP8 weight dataflow without a backward override, where the
 * dgrad operand is built from the same decomposition): a fresh MXFP8
 * quantization of the projected weight y = p * 2^e over 32x1 blocks, i.e. 32
 * consecutive rows of one column, anchored at row 0 (the last block may be
 * short).  The pages require these bytes to equal the host quantizer's bytes for
 * the projected weight and name its amax rule without writing it out; the rule
 * taken is the OCP MX one: S = floor(log2 amax) - 8 (8 = E4M3's largest
 * exponent), raised to -127 if lower; code = S + 127; payload =
 * RTNE_E4M3(y / 2^S) with subnormals.  On projected weights amax has at most two
 * significant bits, so S also equals ceil(log2(amax / 448)) and nothing
 * saturates.  amax is over the block's finite values: elements of poisoned row
 * blocks (NaN in the projection) get payload 0x7F; a block with no nonzero
 * finite value gets code 0.  Unlike the row lift this re-rounds: decode gives
 * back the projection wherever y / 2^S is a multiple of 2^-9.
 *   x      [rows, K] bf16 or fp32, row stride ld_x >= K
 *   data   [rows, K] uint8 E4M3 payload in x's (untransposed) layout, contiguous
 *   scale  [ceil(rows/32), scale_ld] uint8 E8M0 codes, scale_ld >= K; columns
 *          j >= K of each scale row are left untouched
 *   data and scale must not overlap x or each other (MXQ_ERR_ALIAS).
 */
int mxq_mxfp4_to_mxfp8_col(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt, uint8_t* data,
                           uint8_t* scale, int64_t scale_ld, hipStream_t stream);

/*
 * The MXFP8 rowwise lift (mxq_mxfp4_to_mxfp8_row) and the columnwise conversion
 * (mxq_mxfp4_to_mxfp8_col) from one read of x: the pair the MXFP8 weight
 * dataflow without a backward override keeps for the forward and backward GEMMs
 * ([QAT] Description, weight dataflows).  Outputs are bit-identical to the two
 * separate calls; arguments as for them.  No output may overlap x or another
 * output (MXQ_ERR_ALIAS).
 */
int mxq_mxfp4_to_mxfp8_row_col(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt,
                               uint8_t* row_data, uint8_t* row_scale, int64_t row_scale_ld, uint8_t* col_data,
                               uint8_t* col_scale, int64_t col_scale_ld, hipStream_t stream);

/*
 * mxq_mxfp4_to_mxfp8_col / mxq_mxfp4_to_mxfp8_row_col gated by a device-side
 * no-op flag, as mxq_mxfp4_to_mxfp8_row_guarded: when *noop != 0 at the time
 * the work runs on the stream, every output is left untouched.  [QAT]'s
 * flowchart has the skip-update flag gate every conversion into the cached
 * workspace, the columnwise one included.
 *   noop   device pointer to one int32; required (NULL -> MXQ_ERR_NULL).
 *          Other arguments as for the ungated calls.
 */
int mxq_mxfp4_to_mxfp8_col_guarded(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt,
                                   uint8_t* data, uint8_t* scale, int64_t scale_ld, const int32_t* noop,
                                   hipStream_t stream);
int mxq_mxfp4_to_mxfp8_row_col_guarded(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt,
                                       uint8_t* row_data, uint8_t* row_scale, int64_t row_scale_ld,
                                       uint8_t* col_data, uint8_t* col_scale, int64_t col_scale_ld,
                                       const int32_t* noop, hipStream_t stream);

/*
 * Unpadded export of MXFP8 rowwise scales, [EXP] Description: scale_inv holds
 * E8M0 codes with shape (*shape[:-1], ceil(K/32)), without padding; a partial
 * last block keeps its own scale.  Copies the first ceil(K/32) columns of each
 * row of the padded storage into a compact [rows, ceil(K/32)] array.  The
 * payload needs no copy: it is `data` viewed with the tensor's shape.
 *   data           the payload (only checked for presence)
 *   scale_storage  [rows, scale_ld] uint8, scale_ld >= ceil(K/32)
 *   scale_out      [rows, ceil(K/32)] uint8, contiguous
 * data == NULL or scale_storage == NULL -> MXQ_ERR_NO_ROWWISE_DATA ([EXP]: a
 * tensor without row-scaled data raises ValueError).  scale_out == scale_storage
 * with scale_ld == ceil(K/32) is the view case and returns MXQ_OK without work;
 * any other overlap is MXQ_ERR_ALIAS.
 */
int mxq_export_mxfp8(const uint8_t* data, const uint8_t* scale_storage, int64_t rows, int64_t K,
                     int64_t scale_ld, uint8_t* scale_out, hipStream_t stream);

/*
 * Decode FP8 payload with E8M0 codes: out = RNE_out(FP8(q) * 2^(code - 127)).
 * Code 0 is 2^-127 and code 255 is NaN ([QAT] Description: decode UE8M0 code 0
 * as 2^-127 and code 255 as NaN; Test results: planted extreme codes).  A NaN
 * payload or code 255 gives canonical quiet NaN; an E5M2 infinity stays
 * infinite; values beyond the output range round to Inf.
 *   data     [rows, K] uint8 payload, contiguous (row stride K)
 *   scale    E8M0 codes: [rows, scale_ld] for MXQ_SCALE_ROW_1X32 (scale_ld >=
 *            ceil(K/32)), [ceil(rows/128), scale_ld] for MXQ_SCALE_TILE_128X128
 *            (scale_ld >= ceil(K/128)) or [ceil(rows/32), scale_ld] for
 *            MXQ_SCALE_COL_32X1 (scale_ld >= K)
 *   out      [rows, K] bf16 or fp32, row stride ld_out >= K; must not overlap
 *            data or scale
 */
int mxq_dequantize(const uint8_t* data, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K,
                   mxq_fp8 fmt, mxq_scale_layout layout, void* out, int64_t ld_out, mxq_dtype out_dt,
                   hipStream_t stream);

/*
 * One weight of a grouped decode: the arguments of mxq_dequantize for that
 * weight (data, scale and out are device pointers).
 */
typedef struct {
  const uint8_t* data;   /* [rows, K] uint8 payload, contiguous */
  const uint8_t* scale;  /* E8M0 codes in the call's layout, row stride scale_ld */
  int64_t scale_ld;
  int64_t rows;
  int64_t K;
  void* out;             /* [rows, K] in the call's output dtype, row stride ld_out >= K */
  int64_t ld_out;
} mxq_dequant_group;

/*
 * The decode of mxq_dequantize (code 0 is 2^-127 and code 255 NaN, [QAT]
 * Description; the same NaN and overflow rules) applied to a list of weights
 * with one payload format, scale layout and output dtype (the experts of a
 * grouped linear layer, [QAT] Test results, end-to-end cases), in as few
 * launches as possible.  Results are bit-identical to one mxq_dequantize call
 * per weight.
 *   groups    HOST array of n_groups descriptors, read during the call only
 *   n_groups  >= 0; groups with rows == 0 or K == 0 are skipped
 *   Every group is checked as mxq_dequantize checks its arguments (the first
 *   failing group's status is returned and nothing is enqueued).  In addition
 *   no group's out may overlap any group's data, scale or out (MXQ_ERR_ALIAS);
 *   inputs may overlap each other.
 */
int mxq_dequantize_grouped(const mxq_dequant_group* groups, int64_t n_groups, mxq_fp8 fmt,
                           mxq_scale_layout layout, mxq_dtype out_dt, hipStream_t stream);

/*
 * Packed MXFP4, the deployment format: E2M1 payloads with 1x32 power-of-two
 * E8M0 scales ([QAT] Description: the weight seen in training is the deployed
 * one; the export issue's workflow 2, quantizing weights for inference).
 * Layout: packed [rows, ceil(K/2)] uint8, contiguous, element 2i in the low
 * nibble of byte i and 2i+1 in the high nibble (0 when K is odd); each nibble
 * is S.EE.M (sign, then the 3-bit E2M1 code of {0, .5, 1, 1.5, 2, 3, 4, 6}).
 * scale [rows, scale_ld] uint8 E8M0 codes, scale_ld >= ceil(K/32).
 *
 * mxq_quantize_mxfp4: the projection's decomposition (same blocks, same RTNE),
 * except that above the cap the scale moves to 2^126 ([QAT] Known limitations):
 * e = clamp(ceil(log2(amax/6)), -126, 126), code = e + 127.  Below the cap the
 * decoded packed weight equals mxq_fake_quantize_mxfp4's output bit for bit.
 * A block holding Inf or NaN gets code 255 and zero nibbles.
 */
int mxq_quantize_mxfp4(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt, uint8_t* packed,
                       uint8_t* scale, int64_t scale_ld, hipStream_t stream);

/*
 * One weight of a grouped packed MXFP4 encode: the arguments of
 * mxq_quantize_mxfp4 for that weight (x, packed and scale are device pointers).
 */
typedef struct {
  const void* x;      /* [rows, K], row stride ld_x >= K */
  int64_t ld_x;
  int64_t rows;
  int64_t K;
  uint8_t* packed;    /* [rows, ceil(K/2)] nibble pairs, contiguous */
  uint8_t* scale;     /* [rows, scale_ld] E8M0 codes, scale_ld >= ceil(K/32); padding not written */
  int64_t scale_ld;
} mxq_mxfp4_group;

/*
 * The packed MXFP4 encode of mxq_quantize_mxfp4 (the deployment format, [QAT]
 * Description and Known limitations) applied to a list of weights of one
 * dtype (the experts of a grouped linear layer), in as few launches as
 * possible.  Results are bit-identical to one mxq_quantize_mxfp4 call per
 * weight.
 *   groups    HOST array of n_groups descriptors, read during the call only
 *   n_groups  >= 0; groups with rows == 0 or K == 0 are skipped
 *   Every group is checked as mxq_quantize_mxfp4 checks its arguments (the
 *   first failing group's status is returned and nothing is enqueued).  In
 *   addition no group's packed or scale may overlap any group's x, packed or
 *   scale (MXQ_ERR_ALIAS); inputs may overlap each other.
 */
int mxq_quantize_mxfp4_grouped(const mxq_mxfp4_group* groups, int64_t n_groups, mxq_dtype dt,
                               hipStream_t stream);

/* Decode packed MXFP4: out = RNE_out(E2M1 * 2^(code-127)); code 255 -> canonical
 * NaN; values beyond the output range (codes 253, 254) -> Inf.  out [rows, K]
 * bf16 / fp32 with row stride ld_out >= K; must not overlap the inputs. */
int mxq_dequantize_mxfp4(const uint8_t* packed, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K,
                         void* out, int64_t ld_out, mxq_dtype out_dt, hipStream_t stream);

/* Direct MXFP8 row lift from packed MXFP4 (no bf16 re-encode): the fixed-shift-6
 * lift of mxq_mxfp4_to_mxfp8_row with (p, e = code - 127) read from the packed
 * weight: scale_out code max(code - 6, 0), payload E4M3(p * 2^min(6, code)),
 * exact; code 255 -> code 255 and payload 0x7F.  data [rows, K] contiguous;
 * scale_out [rows, scale_out_ld], padding columns untouched. */
int mxq_mxfp4_packed_to_mxfp8_row(const uint8_t* packed, const uint8_t* scale, int64_t scale_ld, int64_t rows,
                                  int64_t K, uint8_t* data, uint8_t* scale_out, int64_t scale_out_ld,
                                  hipStream_t stream);

/* Direct 128x128 blockwise FP8 from packed MXFP4: the tile fold of
 * mxq_mxfp4_to_fp8_block128 with each block's (p, e) read from the packed
 * weight; blocks with code 255 are the poisoned ones. */
int mxq_mxfp4_packed_to_fp8_block128(const uint8_t* packed, const uint8_t* scale, int64_t scale_ld, int64_t rows,
                                     int64_t K, uint8_t* data, uint8_t* tile_code, int64_t tile_ld,
                                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
