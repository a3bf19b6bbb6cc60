// mxq.hip -- gfx950 kernels and the C ABI of include/mxq.h.
//
// Block-scaled weight quantization: MXFP4 projection, the direct MXFP8 rowwise
// lift, 128x128 tile-exponent folding into E4M3, the unpadded scale export and
// the E8M0 decode; the fused projection + row lift and the no-op-flag-gated
// direct conversions; the packed MXFP4 deployment format (encode, decode, and
// the row lift / tile fold from it); MXFP8 columnwise (32x1) from the MXFP4
// decomposition, alone and with the row lift in one pass.  Sources (page title,
// section):
//   [QAT] "[PyTorch] MXFP4 weight QAT on MXFP8 and FP8 block-scaling recipes":
//         Description (both conversion modes, the weight dataflows, the E8M0
//         decode), Test results, Known limitations.
//   [EXP] "MXFP8TensorStorage.export_components()": Description.
//
// Design (CDNA4, wave64).  Every kernel streams HBM once; nothing here is a
// contraction, so there is no MFMA.  A lane owns one 16-byte chunk of a row per
// step (8 bf16 or 4 fp32), so a 1x32 block spans 4 (bf16) or 8 (fp32)
// neighbouring lanes and its amax is reduced with two or three DPP moves.  The
// block's scale exponent is integer arithmetic on the amax bit pattern.  The
// rounding steps run on CDNA4's scaled conversions:
//   v_cvt_scalef32_pk_fp4_{bf16,f32}  RTNE(x / 2^e) onto E2M1, saturating at 6
//   v_cvt_scalef32_pk_bf16_fp4        E2M1 * 2^e back to bf16 (always exact)
//   v_cvt_scalef32_pk_fp8_bf16        RTNE(y / 2^S) onto E4M3 with subnormals
//   v_cvt_scalef32_{pk_bf16,f32}_{fp8,bf8}  FP8 * 2^(code-127)
// Each was compared bit for bit with the CPU oracle over every bf16 input and
// every scale exponent (fp32: every bf16-widened pattern plus random low
// halves) and matches exactly when the wave keeps denormals; every kernel
// therefore sets the MODE register's denormal field itself, which makes the
// results independent of the build's floating-point flags.  The scale operand
// is passed as an E8M0 code placed in the f32 exponent field (code 0 = 2^-127).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <initializer_list>

#include "mxq.h"
#include "fastdiv.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------------------------
// Launch-shape tunables (compile-time).  The defaults are the best of sweeps at
// 8192 x 8192 bf16 on one MI355X, each burst timed after other kernels, after an
// idle gap and after itself: a one-wave, one-step row lift is the fastest right
// after another streaming kernel but up to 10% slower after idle or after
// itself, where 256 lanes of two steps hold steady within 2%.
// ------------------------------------------------------------------------------------
// Lanes per workgroup of the streaming kernels.
#ifndef MXQ_PROJ_THREADS
#define MXQ_PROJ_THREADS 64       // projection (one wave)
#endif
#ifndef MXQ_ROW_THREADS
#define MXQ_ROW_THREADS 256       // row lift
#endif
#ifndef MXQ_ROW_GROUPED_THREADS
#define MXQ_ROW_GROUPED_THREADS 256   // grouped row lift
#endif
#ifndef MXQ_ROW_GROUPED_STEPS
#define MXQ_ROW_GROUPED_STEPS 2
#endif
#ifndef MXQ_DEQUANT_GROUPED_STEPS
#define MXQ_DEQUANT_GROUPED_STEPS 2   // grouped FP8 decode (64 lanes)
#endif
#ifndef MXQ_Q4_THREADS
#define MXQ_Q4_THREADS 256        // MXFP4 encode
#endif
// Consecutive workgroups per XCD run (see xcd_run): the row-layout FP8 decode
// and the row lift from packed MXFP4, whose neighbouring workgroups can read
// (and, for the latter, write) parts of one line of block codes.  Runs remove
// the duplicate code-line fetches (L2 fetch bytes 1.21x -> 1.00x of the
// decode's reads at 8 per run; 1.20x -> 1.03x for the packed lift at one step
// per workgroup and 4 per run) but cost time (decode 32.4 -> 34.9 us, packed
// lift 18.6 -> 20.9 us at 8192 x 8192), so the plain order (1) is the default.
// At its four steps per workgroup the packed lift's workgroups each take one
// whole line of codes.
// Code stores of the full-step row lift: 1 = the first lane of each 16-lane
// row gathers that row's 16 / lanes-per-block codes and stores them with one
// 4-byte (bf16) or 2-byte (fp32) store; 0 = one byte store per block (sc1).
// AUX is the gathered stores' cache-policy field.  At 8192 x 8192 bf16 the
// gathered plain stores took the row lift from 33.7-34.0 us to 33.1-33.5 us
// (sc1: unchanged, nt: 34.1-34.6); the fused projection + row lift was 0.3 us
// slower with them and keeps the byte stores.
#ifndef MXQ_ROW_CODE_WORDS
#define MXQ_ROW_CODE_WORDS 1
#endif
#ifndef MXQ_CODE_AUX
#define MXQ_CODE_AUX 0
#endif
// The full-step MXFP4 encode's gathered code stores, by input type: 1 = after
// every packed-payload store of the workgroup, 0 = each step's right after its
// payload.  After: fp32 8192 x 8192 51.3 -> 47.9 us, 28672 x 8192 168.6 ->
// 163.3 us; bf16 8192 x 8192 28.7 -> 28.0 us but 16384 x 16384 104.3 -> 107.9
// and 28672 x 8192 91.8 -> 94.4 us (burst means over four orders).
#ifndef MXQ_Q4_CODES_LAST_BF16
#define MXQ_Q4_CODES_LAST_BF16 0
#endif
#ifndef MXQ_Q4_CODES_LAST_FP32
#define MXQ_Q4_CODES_LAST_FP32 1
#endif
#ifndef MXQ_Q4_CODE_WORDS
#define MXQ_Q4_CODE_WORDS 1       // the same for the full-step MXFP4 encode
#endif
#ifndef MXQ_PACKED_CODE_WORDS
#define MXQ_PACKED_CODE_WORDS 1   // and the full-step row lift from packed MXFP4 (4 codes per 8 lanes)
#endif
// The fold's check-free form for whole tile groups, for fp32 weights: 52.1 us
// against 52.5 at 8192 x 8192.  For bf16 it was slower (35.2-35.4 us against
// 34.5, with buffer or global stores alike), so bf16 keeps the checked form.
#ifndef MXQ_EXPORT4
#define MXQ_EXPORT4 1             // the export from 4-byte-aligned padded rows: 16-byte stores
#endif
#ifndef MXQ_FOLD_FULL
#define MXQ_FOLD_FULL 1
#endif
// The fold's workgroup by input type: lanes per tile, and runs of side-by-side
// tiles of a band per XCD (see xcd_run).  Burst means over four orders (after
// the projection, after the row lift, after idle, after itself), from 1024
// lanes in the plain order:
//   bf16, 512 lanes in runs of 8: 8192 x 8192 34.7 -> 34.0 us, 28672 x 8192
//   116.0 -> 109.8 us (1024 lanes in runs of 4: 34.2 / 112.8; 512 in runs of 2
//   or 16: 34.3 / 111.9 and 36.7 / 117.0; 256 lanes: 36.5-39.3 / 115.9-124.4);
//   fp32, 1024 lanes in runs of 4: 8192 x 8192 52.5 -> 52.0 us (512 lanes
//   55.8-56.0); runs of 16-64 were 1-19% slower for both.
#ifndef MXQ_FOLD_THREADS_BF16
#define MXQ_FOLD_THREADS_BF16 512
#endif
#ifndef MXQ_FOLD_THREADS_FP32
#define MXQ_FOLD_THREADS_FP32 1024
#endif
#ifndef MXQ_FOLD_XCD_RUN_BF16
#define MXQ_FOLD_XCD_RUN_BF16 8
#endif
#ifndef MXQ_FOLD_XCD_RUN_FP32
#define MXQ_FOLD_XCD_RUN_FP32 4
#endif
// The columnwise kernel's order of 32-row band groups (see xcd_run), by input
// type.  fp32 in runs of 8 per XCD (burst means over four orders, col / row +
// col: 8192 x 8192 54.8 -> 52.8 us / 68.2 -> 66.3 us, 28672 x 8192 188.3 ->
// 179.7 us / 225.6 -> 219.8 us); bf16 in the plain order (runs of 2-8 were
// within +-1%, faster at one size and slower at the other).
#ifndef MXQ_COL_XCD_RUN_BF16
#define MXQ_COL_XCD_RUN_BF16 1
#endif
#ifndef MXQ_COL_XCD_RUN_FP32
#define MXQ_COL_XCD_RUN_FP32 8
#endif
#ifndef MXQ_FOLD_READLANE
#define MXQ_FOLD_READLANE 1       // the fold's wave maximum from four readlanes (one tile per workgroup)
#endif
#ifndef MXQ_DEQUANT_XCD_RUN
#define MXQ_DEQUANT_XCD_RUN 1
#endif
#ifndef MXQ_PACKED_XCD_RUN
#define MXQ_PACKED_XCD_RUN 1
#endif
#ifndef MXQ_FUSED_THREADS
#define MXQ_FUSED_THREADS 64      // fused projection + row lift
#endif
#ifndef MXQ_DEQUANT_THREADS_BF16
#define MXQ_DEQUANT_THREADS_BF16 64   // FP8 decodes to bf16 (8 elements per lane)
#endif
#ifndef MXQ_DEQUANT_THREADS_FP32
#define MXQ_DEQUANT_THREADS_FP32 128  // FP8 decodes to fp32
#endif
#ifndef MXQ_DQ4_THREADS
#define MXQ_DQ4_THREADS 256       // packed MXFP4 decode (8 elements per lane)
#endif
#ifndef MXQ_PACKED_THREADS
#define MXQ_PACKED_THREADS 64     // row lift from packed MXFP4 (16 elements per lane)
#endif
// Steps (16-byte chunks in flight per lane) per workgroup of the streaming kernels.
#ifndef MXQ_PROJ_STEPS
#define MXQ_PROJ_STEPS 1
#endif
#ifndef MXQ_ROW_STEPS
#define MXQ_ROW_STEPS 2
#endif
#ifndef MXQ_Q4_STEPS
#define MXQ_Q4_STEPS 2
#endif
#ifndef MXQ_FUSED_STEPS
#define MXQ_FUSED_STEPS 1
#endif
// FP8 decodes: to bf16, 64 lanes and two steps (row layout 32.7-33.0 us at
// 8192 x 8192 in every order; one step ran 32.2 after the fold but 36.0 after
// itself; 128 or 256 lanes 33.7-34.7); to fp32, 128 lanes and one step (row /
// tile layout at 28672 x 8192: 181 / 179 us, against 191 / 187 with 64 lanes
// and 196 in the tile layout with two steps).  A check-free form with buffer
// stores was tried for both and was slower or less steady.
#ifndef MXQ_DEQUANT_STEPS_BF16
#define MXQ_DEQUANT_STEPS_BF16 2
#endif
#ifndef MXQ_DEQUANT_STEPS_FP32
#define MXQ_DEQUANT_STEPS_FP32 1
#endif
#ifndef MXQ_DQ4_STEPS
#define MXQ_DQ4_STEPS 2           // packed MXFP4 decode
#endif
// Row lift from packed MXFP4: 64 lanes x 4 steps, so a workgroup takes 4096
// elements of a row, whose 128 block codes fill one 128-byte line.  Burst
// means over four orders, against one step: 8192 x 8192 19.8 -> 18.9 us,
// 28672 x 8192 62.5 -> 57.8 us, and after itself 21.0 -> 19.2 us and 69.0 ->
// 58.6 us (2 or 8 steps, or 128 or 256 lanes, 0.5-5% slower).
#ifndef MXQ_PACKED_STEPS
#define MXQ_PACKED_STEPS 4
#endif
// The banded kernels.
#ifndef MXQ_PFOLD_ROWS
#define MXQ_PFOLD_ROWS 8          // fold from packed MXFP4: band rows per lane (16, 8 or 4)
#endif
#ifndef MXQ_COL_THREADS
#define MXQ_COL_THREADS 64        // columnwise: column lanes per workgroup, one 16-byte chunk each
#endif
#ifndef MXQ_COL_ROWS
#define MXQ_COL_ROWS 4            // columnwise: rows of the 32-row band per lane (a divisor of 32)
#endif
// Cache policy of the streaming accesses.
#ifndef MXQ_NT_LOADS
#define MXQ_NT_LOADS 1            // streaming loads carry the non-temporal hint
#endif
#ifndef MXQ_NT_STORES
#define MXQ_NT_STORES 1           // streaming stores carry the non-temporal hint
#endif
#ifndef MXQ_PROJ_STORE_SC1
#define MXQ_PROJ_STORE_SC1 1      // projection output: buffer stores with the nt and sc1 bits
#endif

constexpr int kThreads = 256;     // 4 waves: workgroup size of the remaining streaming kernels
constexpr int kProjThreads = MXQ_PROJ_THREADS, kRowThreads = MXQ_ROW_THREADS,
              kDq4Threads = MXQ_DQ4_THREADS, kPackedThreads = MXQ_PACKED_THREADS;
constexpr int kProjSteps = MXQ_PROJ_STEPS, kRowSteps = MXQ_ROW_STEPS, kPackedSteps = MXQ_PACKED_STEPS;
// Launch shape of the FP8 decodes by output type: lanes per workgroup (single
// and grouped kernels) and steps per workgroup (single kernel).
template <typename TO>
struct DequantShape {
  static constexpr int kThreads = sizeof(TO) == 2 ? MXQ_DEQUANT_THREADS_BF16 : MXQ_DEQUANT_THREADS_FP32;
  static constexpr int kSteps = sizeof(TO) == 2 ? MXQ_DEQUANT_STEPS_BF16 : MXQ_DEQUANT_STEPS_FP32;
};
constexpr int kFusedThreads = MXQ_FUSED_THREADS, kFusedSteps = MXQ_FUSED_STEPS;
constexpr int kQ4Threads = MXQ_Q4_THREADS, kQ4Steps = MXQ_Q4_STEPS, kDq4Steps = MXQ_DQ4_STEPS;
constexpr int kRowGroupedThreads = MXQ_ROW_GROUPED_THREADS, kRowGroupedSteps = MXQ_ROW_GROUPED_STEPS,
              kDequantGroupedSteps = MXQ_DEQUANT_GROUPED_STEPS;
constexpr int kDequantXcdRun = MXQ_DEQUANT_XCD_RUN, kPackedXcdRun = MXQ_PACKED_XCD_RUN;
constexpr int kPFoldRows = MXQ_PFOLD_ROWS, kPFoldThreads = 4096 / kPFoldRows;   // 128 rows x 32 chunks
static_assert(kPFoldRows * kPFoldThreads == 4096 && kPFoldThreads >= 256, "packed fold geometry");
constexpr int kColThreads = MXQ_COL_THREADS, kColRows = MXQ_COL_ROWS, kColGroups = 32 / kColRows;
static_assert(kColRows * kColGroups == 32 && kColThreads % 64 == 0, "columnwise geometry");

template <typename V>
__device__ __forceinline__ V stream_load(const V* p) {
#if MXQ_NT_LOADS
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}
template <typename V>
__device__ __forceinline__ void stream_store(V v, V* p) {
#if MXQ_NT_STORES
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// 16-byte streaming store at byte offset `off` of a row whose base address is
// the same for the whole wave (nbytes: the row's length, below 2^31).  With
// MXQ_PROJ_STORE_SC1 it is a buffer store carrying the nt and sc1 bits, which
// measured about 3% faster than nt alone for the projection's read-one /
// write-one stream.  The FP8 decodes keep non-temporal global stores: buffer
// stores, with nt, sc1 or both, made their bf16 output 2-4% slower.
__device__ __forceinline__ void stream_store_row_sc1(u32x4 v, void* base, uint32_t nbytes, uint32_t off) {
#if MXQ_PROJ_STORE_SC1
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 2 | 16);   // nt | sc1
#else
  (void)nbytes;
  stream_store(v, reinterpret_cast<u32x4*>(reinterpret_cast<char*>(base) + off));
#endif
}

// 2-, 4-, 8- or 16-byte streaming store at byte offset `off` of a row whose base
// address is the same for the whole wave: a buffer store carrying its
// cache-policy bits (the compiler can drop the non-temporal hint of a plain
// store when it merges code paths; the buffer form keeps it in the
// instruction).  The bits are nt and sc1.  Against nt alone,
// burst means over four orders: row lift bf16 8192 x 8192 33.2 -> 33.0 us,
// 28672 x 8192 109.3 -> 106.8 us, fp32 55.4 -> 53.3 us and 180.7 -> 176.4 us;
// fused projection + row lift bf16 53.8 -> 52.4 us and 184.9 -> 181.3 us; fp32
// MXFP4 encode 48.0 -> 47.5 us and 163.8 -> 160.9 us; the fp32 fold and the row
// lift from packed MXFP4 within 0.5%.  (sc1 alone was 4-5% faster at 8192 x
// 8192 but 4-5% slower at 28672 x 8192.)
#ifndef MXQ_PAYLOAD_AUX
#define MXQ_PAYLOAD_AUX 18
#endif
template <typename V>
__device__ __forceinline__ void stream_store_at(V v, void* base, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, 0x00020000);
  constexpr int A = MXQ_PAYLOAD_AUX;
  if constexpr (sizeof(V) == 16)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, A);
  else if constexpr (sizeof(V) == 8)
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, A);
  else if constexpr (sizeof(V) == 4)
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, A);
  else
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), r, off, 0, A);
}

// ------------------------------------------------------------------------------------
// Conversions
// ------------------------------------------------------------------------------------
// hwreg(HW_REG_MODE, offset 4, size 4): the FP_DENORM field.  0xF keeps
// denormals (f32 and f16/f64 classes, inputs and outputs).
constexpr int kModeFpDenorm = 1 | (4 << 6) | (3 << 11);
__device__ __forceinline__ void keep_denormals() { __builtin_amdgcn_s_setreg(kModeFpDenorm, 0xF); }

// Scale operand of the scaled conversions: E8M0 code in the f32 exponent field.
__device__ __forceinline__ float e8m0(uint32_t code) { return __builtin_bit_cast(float, code << 23); }

__device__ __forceinline__ bf16x2 BF(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }
__device__ __forceinline__ float F(uint32_t v) { return __builtin_bit_cast(float, v); }

// E2M1 nibbles (element k of the chunk in nibble k) of RTNE(x / 2^e).
__device__ __forceinline__ uint32_t fp4_of(u32x4 w, float s, uint16_t) {
  uint32_t f = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, BF(w[0]), s, 0);
  f = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(f, BF(w[1]), s, 1);
  f = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(f, BF(w[2]), s, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(f, BF(w[3]), s, 3);
}
__device__ __forceinline__ uint32_t fp4_of(u32x4 w, float s, uint32_t) {
  uint32_t f = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, F(w[0]), F(w[1]), s, 0);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(f, F(w[2]), F(w[3]), s, 1);
}
// Two bf16 values p * 2^e from nibble pair SEL (byte SEL of f).
template <int SEL>
__device__ __forceinline__ uint32_t bf16_pair(uint32_t f, float s) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f, s, SEL));
}
// Four E4M3 bytes RTNE(y / 2^S) of two bf16 pairs.
__device__ __forceinline__ uint32_t e4m3x4(uint32_t y01, uint32_t y23, float s) {
  s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s16x2{0, 0}, BF(y01), s, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, BF(y23), s, true);
  return __builtin_bit_cast(uint32_t, r);
}

// DPP lane moves inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// Workgroup order in runs per XCD.  The dispatcher deals workgroup b to XCD
// b % 8, and each XCD has its own L2, so in the plain order M neighbouring
// workgroups run on M XCDs (a code line they share is fetched by M L2s).  With
// M > 1, each run of 8 M workgroups is reordered so that XCD x takes the M
// consecutive logical workgroups 8 M g + M x .. 8 M g + M x + M - 1; the last,
// partial run keeps the plain order.  A permutation of 0 .. n - 1.
template <int M>
__device__ __forceinline__ uint32_t xcd_run(uint32_t b, uint32_t n) {
  if constexpr (M == 1) {
    return b;
  } else {
    constexpr uint32_t G = 8u * M;
    if (b >= n - n % G) return b;
    const uint32_t r = b % G;
    return b - r + (r % 8u) * M + r / 8u;
  }
}

constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i within each group of 8

// Max over the LPB lanes that hold one 1x32 block (all lanes must be active).
template <int LPB>
__device__ __forceinline__ uint32_t block_max(uint32_t v) {
  v = max(v, dpp<kQuadXor1>(v));
  v = max(v, dpp<kQuadXor2>(v));
  if constexpr (LPB == 8) v = max(v, dpp<kRowHalfMirror>(v));
  return v;
}

// ------------------------------------------------------------------------------------
// Element formats
// ------------------------------------------------------------------------------------
template <typename T>
struct Fmt;
template <>
struct Fmt<uint16_t> {   // bf16 bit patterns
  static constexpr int kEPL = 8;   // elements per 16-byte chunk
  static constexpr int kLPB = 4;   // lanes per 1x32 block
  static constexpr uint32_t kNaN2 = 0x7FC07FC0u;          // canonical quiet NaN, twice
  static constexpr uint32_t kMag = 0x7FFF7FFFu, kInf = 0x7F80u;
  static constexpr int kMbits = 7;
};
template <>
struct Fmt<uint32_t> {   // fp32 bit patterns
  static constexpr int kEPL = 4;
  static constexpr int kLPB = 8;
  static constexpr uint32_t kNaN2 = 0x7FC00000u;
  static constexpr uint32_t kMag = 0x7FFFFFFFu, kInf = 0x7F800000u;
  static constexpr int kMbits = 23;
};

// ------------------------------------------------------------------------------------
// The scale exponent of one block ([QAT] Description, conversion mode 1)
//
// eb = e + 127 is the biased scale exponent, 1..252.  With A the amax bit
// pattern, 6 * 2^e >= amax first holds at e = E - 2 when the amax mantissa is
// at most 1.5 (and at E - 1 above it), so eb = ((A + half - 1) >> mbits) - 2,
// clamped; zero and subnormal amax land on the clamp at 1 (e = -126).  Any
// Inf / NaN pattern compares above every finite one, so "poisoned" is simply
// A >= the Inf pattern.
// ------------------------------------------------------------------------------------
struct Block {
  uint32_t eb;      // 1..252
  bool poison;
};

// kTop: the largest biased scale exponent, 252 (e = 125) for the projection and
// the direct conversions, 253 (e = 126) for the packed deployment format.
template <typename T, int kTop = 252>
__device__ __forceinline__ Block block_of_amax(uint32_t amax) {
  constexpr int MB = Fmt<T>::kMbits;
  int eb = (int)((amax + ((1u << (MB - 1)) - 1u)) >> MB) - 2;
  eb = min(max(eb, 1), kTop);
  return Block{(uint32_t)eb, amax >= Fmt<T>::kInf};
}

template <typename T>
__device__ __forceinline__ uint32_t chunk_amax(u32x4 w) {
  const uint32_t M = Fmt<T>::kMag;
  if constexpr (sizeof(T) == 2) {
    typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
    const u16x2 m = __builtin_elementwise_max(
        __builtin_elementwise_max(__builtin_bit_cast(u16x2, w[0] & M), __builtin_bit_cast(u16x2, w[1] & M)),
        __builtin_elementwise_max(__builtin_bit_cast(u16x2, w[2] & M), __builtin_bit_cast(u16x2, w[3] & M)));
    return max((uint32_t)m[0], (uint32_t)m[1]);
  } else {
    return max(max(w[0] & M, w[1] & M), max(w[2] & M, w[3] & M));
  }
}

template <typename T, int kTop = 252>
__device__ __forceinline__ Block chunk_block(u32x4 w) {
  return block_of_amax<T, kTop>(block_max<Fmt<T>::kLPB>(chunk_amax<T>(w)));
}

// Projected values p * 2^e of a chunk, as bf16 pairs: 4 words (bf16 chunk) or
// 2 words (fp32 chunk) -- exact, since p has two significant bits and
// p * 2^e >= 2^-127 is a bf16 subnormal at worst.
template <typename T>
struct Proj16 {
  uint32_t p[sizeof(T) == 2 ? 4 : 2];
};
template <typename T>
__device__ __forceinline__ Proj16<T> project(uint32_t f, float s) {
  Proj16<T> y;
  y.p[0] = bf16_pair<0>(f, s);
  y.p[1] = bf16_pair<1>(f, s);
  if constexpr (sizeof(T) == 2) {
    y.p[2] = bf16_pair<2>(f, s);
    y.p[3] = bf16_pair<3>(f, s);
  }
  return y;
}

// Projection output chunk in the input dtype; a poisoned block is all NaN.
template <typename T>
__device__ __forceinline__ u32x4 proj_chunk(const Proj16<T>& y, bool poison) {
  u32x4 o;
  if constexpr (sizeof(T) == 2) {
    o = u32x4{y.p[0], y.p[1], y.p[2], y.p[3]};
  } else {
    o = u32x4{y.p[0] << 16, y.p[0] & 0xFFFF0000u, y.p[1] << 16, y.p[1] & 0xFFFF0000u};
  }
  if (poison) o = u32x4{Fmt<T>::kNaN2, Fmt<T>::kNaN2, Fmt<T>::kNaN2, Fmt<T>::kNaN2};
  return o;
}

// E4M3 payload bytes of a chunk at scale 2^(code-127): 8 bytes (bf16 chunk) or 4
// (fp32 chunk); a poisoned block is all 0x7F (NaN).
template <typename T>
struct PayloadChunk;
template <>
struct PayloadChunk<uint16_t> { typedef u32x2 type; };
template <>
struct PayloadChunk<uint32_t> { typedef uint32_t type; };

template <typename T>
__device__ __forceinline__ typename PayloadChunk<T>::type payload_chunk(const Proj16<T>& y, uint32_t code, bool poison) {
  const float s = e8m0(code);
  if constexpr (sizeof(T) == 2) {
    u32x2 q{e4m3x4(y.p[0], y.p[1], s), e4m3x4(y.p[2], y.p[3], s)};
    if (poison) q = u32x2{0x7F7F7F7Fu, 0x7F7F7F7Fu};
    return q;
  } else {
    return poison ? 0x7F7F7F7Fu : e4m3x4(y.p[0], y.p[1], s);
  }
}

// Direct-row scale code: 2^(e-6) clamped at 2^-127 = max(e + 121, 0); 255 if poisoned.
__device__ __forceinline__ uint32_t row_code(Block b) {
  return b.poison ? 255u : (b.eb > 6u ? b.eb - 6u : 0u);
}

// ------------------------------------------------------------------------------------
// Chunk I/O.  VEC: 16-byte aligned rows with K a multiple of the chunk, so a
// chunk is either fully inside the row or fully outside it.  Otherwise every
// element is loaded / stored on its own with a bounds check.
// ------------------------------------------------------------------------------------
template <typename T, bool VEC>
__device__ __forceinline__ u32x4 load_chunk(const T* __restrict__ row, int64_t col0, int64_t K) {
  constexpr int EPL = Fmt<T>::kEPL;
  u32x4 w = {0u, 0u, 0u, 0u};
  if (col0 >= K) return w;
  if constexpr (VEC) {
    return stream_load(reinterpret_cast<const u32x4*>(row + col0));
  } else {
#pragma unroll
    for (int i = 0; i < EPL; i++) {
      uint32_t v = (col0 + i < K) ? (uint32_t)row[col0 + i] : 0u;
      if constexpr (sizeof(T) == 2) w[i / 2] |= v << (16 * (i % 2));
      else w[i] = v;
    }
    return w;
  }
}

// kSc1: the projection kernel's own stores (see stream_store_row_sc1).
template <typename T, bool VEC, bool kSc1 = false>
__device__ __forceinline__ void store_chunk(T* __restrict__ row, int64_t col0, int64_t K, u32x4 w) {
  constexpr int EPL = Fmt<T>::kEPL;
  if (col0 >= K) return;
  if constexpr (VEC) {
    if constexpr (kSc1) stream_store_row_sc1(w, row, (uint32_t)(K * sizeof(T)), (uint32_t)(col0 * sizeof(T)));
    else stream_store(w, reinterpret_cast<u32x4*>(row + col0));
  } else {
#pragma unroll
    for (int i = 0; i < EPL; i++) {
      if (col0 + i < K) {
        if constexpr (sizeof(T) == 2) row[col0 + i] = (T)(w[i / 2] >> (16 * (i % 2)));
        else row[col0 + i] = w[i];
      }
    }
  }
}

template <typename T, bool VEC>
__device__ __forceinline__ void store_payload(uint8_t* __restrict__ row, int64_t col0, int64_t K,
                                              typename PayloadChunk<T>::type p) {
  constexpr int EPL = Fmt<T>::kEPL;
  if (col0 >= K) return;
  if constexpr (VEC) {
    stream_store(p, reinterpret_cast<typename PayloadChunk<T>::type*>(row + col0));
  } else {
#pragma unroll
    for (int i = 0; i < EPL; i++) {
      if (col0 + i < K) {
        uint32_t word;
        if constexpr (EPL == 8) word = p[i / 4];
        else word = p;
        row[col0 + i] = (uint8_t)(word >> (8 * (i % 4)));
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// Streaming kernels: projection and row lift.  A "step" is the workgroup's
// lanes x one 16-byte chunk (8 bf16 / 4 fp32 elements each) of ONE row; rows
// are padded to whole steps, so the row / segment split is per-step uniform
// (scalar) arithmetic and a block never straddles two rows.
// ------------------------------------------------------------------------------------
template <typename T, int TPB = kThreads>
struct StepGeom {
  static constexpr int kEPL = Fmt<T>::kEPL, kLPB = Fmt<T>::kLPB;
  static constexpr int kBlocksPerStep = TPB / kLPB;
  static constexpr int64_t kElemsPerStep = (int64_t)kBlocksPerStep * 32;
};

// The projection's steps of workgroup wg: kProjSteps steps of kProjThreads
// lanes, all loads issued before the first store.
template <typename T, bool VEC>
__device__ __forceinline__ void proj_steps(const T* __restrict__ x, int64_t ld_x, T* __restrict__ y, int64_t ld_y,
                                           int64_t K, MxqDivisor steps_per_row, uint32_t total_steps, uint32_t wg) {
  using G = StepGeom<T, kProjThreads>;
  const uint32_t tid = threadIdx.x;
  const int64_t lane_col = (int64_t)(tid / G::kLPB) * 32 + (tid % G::kLPB) * G::kEPL;
  u32x4 w[kProjSteps];
#pragma unroll
  for (int u = 0; u < kProjSteps; u++) {
    const uint32_t step = wg * kProjSteps + u;
    w[u] = u32x4{0u, 0u, 0u, 0u};
    if (step < total_steps) {
      const uint32_t row = mxq_quot(step, steps_per_row), seg = step - row * steps_per_row.d;
      w[u] = load_chunk<T, VEC>(x + (int64_t)row * ld_x, seg * G::kElemsPerStep + lane_col, K);
    }
  }
#pragma unroll
  for (int u = 0; u < kProjSteps; u++) {
    const uint32_t step = wg * kProjSteps + u;
    if (step < total_steps) {
      const uint32_t row = mxq_quot(step, steps_per_row), seg = step - row * steps_per_row.d;
      const Block b = chunk_block<T>(w[u]);
      const float s = e8m0(b.eb);
      const Proj16<T> p = project<T>(fp4_of(w[u], s, T{}), s);
      store_chunk<T, VEC, true>(y + (int64_t)row * ld_y, seg * G::kElemsPerStep + lane_col, K,
                                proj_chunk<T>(p, b.poison));
    }
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kProjThreads) void proj_kernel(const T* __restrict__ x, int64_t ld_x, T* __restrict__ y,
                                                            int64_t ld_y, int64_t K, MxqDivisor steps_per_row,
                                                            uint32_t total_steps) {
  keep_denormals();
  proj_steps<T, VEC>(x, ld_x, y, ld_y, K, steps_per_row, total_steps, blockIdx.x);
}

// A no-op flag (device memory): when it is non-zero the launch leaves every
// output untouched, so a captured graph can replay a cached update
// conditionally.  Kernels read it after issuing their input loads (those only
// read the input), so its latency overlaps theirs.
__device__ __forceinline__ bool skipped(const int32_t* __restrict__ noop) {
  return noop != nullptr && *reinterpret_cast<const volatile int32_t*>(noop) != 0;
}

// E8M0 code of a block, stored by the lane that holds the block's first chunk.
// One step's codes are a short run (16 bytes for bf16 at 64 lanes) of a 128-byte
// line whose other runs come from the neighbouring workgroups, which the
// dispatcher deals to other XCDs and so other L2s.  The store carries the sc1
// cache-policy bit: for such partial-line stores it measured faster than a
// plain store, and far faster than a non-temporal one.  base: the step's first
// code, the same address for the whole wave; off: this lane's code from it.
__device__ __forceinline__ void store_code(uint8_t* base, uint32_t off, uint32_t code) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code, r, off, 0, 16);   // sc1
}

// Gathered code stores.  With kLPB lanes per block (2, 4 or 8), the codes of
// kCodes consecutive blocks sit in lanes l, l + kLPB, ... of a group of kLanes
// lanes inside one 16-lane DPP row (row_shl:n moves lane i + n's value to
// lane i).  gather() packs them into the group's first lane, lowest block
// first (little-endian: the code bytes in storage order); every lane must run
// it, and only the first lane's value is meaningful.  store() is that lane's
// one kCodes-byte store at byte offset off of base (both aligned to kCodes).
template <int kLPB>
struct CodeGather {
  static_assert(kLPB == 2 || kLPB == 4 || kLPB == 8, "2, 4 or 8 lanes per block");
  static constexpr int kCodes = kLPB == 8 ? 2 : 4, kLanes = kCodes * kLPB;
  static __device__ __forceinline__ uint32_t gather(uint32_t code) {
    if constexpr (kLPB == 2)
      return code | (dpp<0x102>(code) << 8) | (dpp<0x104>(code) << 16) | (dpp<0x106>(code) << 24);
    else if constexpr (kLPB == 4)
      return code | (dpp<0x104>(code) << 8) | (dpp<0x108>(code) << 16) | (dpp<0x10C>(code) << 24);
    else
      return code | (dpp<0x108>(code) << 8);
  }
  static __device__ __forceinline__ void store(uint8_t* base, uint32_t off, uint32_t codes) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, 0x00020000);
    if constexpr (kCodes == 4)
      __builtin_amdgcn_raw_buffer_store_b32(codes, r, off, 0, MXQ_CODE_AUX);
    else
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)codes, r, off, 0, MXQ_CODE_AUX);
  }
};

// Row lift; with kProj it also writes the projection y (the fused one-pass form).
// Launch shape of the row kernel: the row lift's, or (kProj) the fused pass's.
template <bool kProj, bool kGrouped = false>
struct RowShape {
  static constexpr int kTPB = kGrouped ? kRowGroupedThreads : kProj ? kFusedThreads : kRowThreads;
  static constexpr int kSteps = kGrouped ? kRowGroupedSteps : kProj ? kFusedSteps : kRowSteps;
};

// The row lift's steps of workgroup wg (with kProj, also the projection y);
// all loads are issued before the no-op flag is read and before any store.
// FULL: every step of every workgroup is whole and inside the matrix (16-byte
// path, K a multiple of a step's width, the grid an exact number of steps), so
// there is no bounds check and nothing to branch around before the first load.
template <typename T, bool VEC, bool kProj, bool FULL = false, bool kGrouped = false>
__device__ __forceinline__ void row_steps(const T* __restrict__ x, int64_t ld_x, int64_t K,
                                          uint8_t* __restrict__ data, uint8_t* __restrict__ scale, int64_t scale_ld,
                                          T* __restrict__ y, int64_t ld_y, MxqDivisor steps_per_row,
                                          uint32_t total_steps, uint32_t wg, const int32_t* __restrict__ noop) {
  static_assert(VEC || !FULL, "the full-step form takes the 16-byte path");
  using G = StepGeom<T, RowShape<kProj, kGrouped>::kTPB>;
  constexpr int kRowSteps = RowShape<kProj, kGrouped>::kSteps;
  const uint32_t tid = threadIdx.x;
  const int64_t lane_col = (int64_t)(tid / G::kLPB) * 32 + (tid % G::kLPB) * G::kEPL;
  u32x4 w[kRowSteps];
#pragma unroll
  for (int u = 0; u < kRowSteps; u++) {
    const uint32_t step = wg * kRowSteps + u;
    w[u] = u32x4{0u, 0u, 0u, 0u};
    if (FULL || step < total_steps) {
      const uint32_t row = mxq_quot(step, steps_per_row), seg = step - row * steps_per_row.d;
      if constexpr (FULL)
        w[u] = stream_load(reinterpret_cast<const u32x4*>(x + (int64_t)row * ld_x + seg * G::kElemsPerStep + lane_col));
      else
        w[u] = load_chunk<T, VEC>(x + (int64_t)row * ld_x, seg * G::kElemsPerStep + lane_col, K);
    }
  }
  if (skipped(noop)) return;   // read once the input loads are in flight
#pragma unroll
  for (int u = 0; u < kRowSteps; u++) {
    const uint32_t step = wg * kRowSteps + u;
    if (FULL || step < total_steps) {
      const uint32_t row = mxq_quot(step, steps_per_row), seg = step - row * steps_per_row.d;
      const int64_t col0 = seg * G::kElemsPerStep + lane_col;
      const Block b = chunk_block<T>(w[u]);
      const float s = e8m0(b.eb);
      const uint32_t code = row_code(b);
      const Proj16<T> p = project<T>(fp4_of(w[u], s, T{}), s);
      if constexpr (FULL) {
        if constexpr (kProj)
          stream_store_row_sc1(proj_chunk<T>(p, b.poison), y + (int64_t)row * ld_y, (uint32_t)(K * sizeof(T)),
                               (uint32_t)(col0 * sizeof(T)));
        stream_store_at(payload_chunk<T>(p, code, b.poison), data + (int64_t)row * K, (uint32_t)col0);
        uint8_t* const crow = scale + (int64_t)row * scale_ld + seg * G::kBlocksPerStep;
        if constexpr (MXQ_ROW_CODE_WORDS && !kProj) {
          using CG = CodeGather<G::kLPB>;
          const uint32_t codes = CG::gather(code);
          if (tid % CG::kLanes == 0) CG::store(crow, tid / G::kLPB, codes);
        } else {
          if (tid % G::kLPB == 0) store_code(crow, tid / G::kLPB, code);
        }
      } else {
        // the projection output goes out like the projection kernel's (nt sc1 buffer stores)
        if constexpr (kProj) store_chunk<T, VEC, true>(y + (int64_t)row * ld_y, col0, K, proj_chunk<T>(p, b.poison));
        store_payload<T, VEC>(data + (int64_t)row * K, col0, K, payload_chunk<T>(p, code, b.poison));
        if (tid % G::kLPB == 0 && col0 < K) scale[(int64_t)row * scale_ld + col0 / 32] = (uint8_t)code;
      }
    }
  }
}

template <typename T, bool VEC, bool kProj, bool FULL>
__global__ __launch_bounds__(RowShape<kProj>::kTPB) void row_kernel(const T* __restrict__ x, int64_t ld_x, int64_t K,
                                                                 uint8_t* __restrict__ data,
                                                                 uint8_t* __restrict__ scale, int64_t scale_ld,
                                                                 T* __restrict__ y, int64_t ld_y,
                                                                 MxqDivisor steps_per_row, uint32_t total_steps,
                                                                 const int32_t* __restrict__ noop) {
  keep_denormals();
  row_steps<T, VEC, kProj, FULL>(x, ld_x, K, data, scale, scale_ld, y, ld_y, steps_per_row, total_steps, blockIdx.x,
                                 noop);
}

// ------------------------------------------------------------------------------------
// MXFP8 columnwise (32x1) from the decomposition ([QAT] Description, conversion
// mode 2): the projected weight re-quantized over blocks of 32 consecutive rows
// of one column with the OCP MX scale rule, S = floor(log2 amax) - 8 floored at
// -127, payload RTNE_E4M3(y / 2^S).  Projected magnitudes have at most two
// significant bits, so amax / 2^S is 256 or 384 and never saturates, and the
// rule equals ceil(log2(amax / 448)).  amax skips the NaNs of poisoned row
// blocks; their payload is 0x7F.
//
// A workgroup takes one 32-row band and kColThreads 16-byte column chunks, with
// kColGroups lane groups of kColThreads lanes each taking kColRows of the band's
// rows.  Each lane loads its chunk of its rows before anything else, projects
// them in registers (bf16 words, exact) and keeps the finite column maxima with
// packed 16-bit max; the groups' maxima meet in LDS; then every lane writes its
// rows' payload (group 0 also the band's codes).  With kRow the same pass also
// writes the rowwise lift of every row block.
// ------------------------------------------------------------------------------------
// E4M3 bytes of four bf16 values at four scales: each pair is converted at
// both of its elements' scales and the right byte of each is kept (two byte
// permutes; the second pair's conversion writes the high half of the first's).
__device__ __forceinline__ uint32_t e4m3x4_each(uint32_t y01, uint32_t y23, float s0, float s1, float s2, float s3) {
  const s16x2 a = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s16x2{0, 0}, BF(y01), s0, false);
  const s16x2 b = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s16x2{0, 0}, BF(y01), s1, false);
  // bytes {a0, b1}: perm picks byte k of (b:a), a being bytes 0-3
  const uint32_t lo = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a), 0x0C0C0500u);
  const s16x2 c = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(s16x2, lo), BF(y23), s2, true);
  const s16x2 d = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s16x2{0, 0}, BF(y23), s3, true);
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, d), __builtin_bit_cast(uint32_t, c), 0x07020100u);
}

// Grouped row lift: the row lift of up to kGroupMax weights in one launch, on a
// 2-D grid: blockIdx.y is the weight and blockIdx.x the workgroup within it, so
// a workgroup reads its weight's descriptor from the kernel arguments (scalar
// loads at a uniform offset) and needs no search.  The grid's x extent is the
// largest weight's workgroup count; the workgroups past a smaller weight's own
// count exit at once (the host keeps that padding small).  Aligned (VEC)
// weights only; the host launches the others one by one.
constexpr int kGroupMax = 48;
struct RowGroupDesc {
  const void* x;
  int64_t ld_x, K;
  uint8_t* data;
  uint8_t* scale;
  int64_t scale_ld;
  MxqDivisor steps_per_row;
  uint32_t total_steps;
};
struct RowGroupTable {
  RowGroupDesc g[kGroupMax];
};
static_assert(sizeof(RowGroupTable) <= 3584, "the table must fit the kernel-argument segment");

template <typename T>
__global__ __launch_bounds__(kRowGroupedThreads) void row_grouped_kernel(const RowGroupTable tab) {
  const RowGroupDesc d = tab.g[blockIdx.y];
  if (blockIdx.x * kRowGroupedSteps >= d.total_steps) return;   // uniform: past this weight's steps
  keep_denormals();
  row_steps<T, true, false, false, true>(static_cast<const T*>(d.x), d.ld_x, d.K, d.data, d.scale, d.scale_ld,
                                         nullptr, 0, d.steps_per_row, d.total_steps, blockIdx.x, nullptr);
}

// Grouped projection, on the same pattern as the grouped row lift: blockIdx.y
// is the weight, blockIdx.x the workgroup within it, with the projection's own
// launch shape and stores.  A weight may be in place (y == x).
struct ProjGroupDesc {
  const void* x;
  int64_t ld_x, K;
  void* y;
  int64_t ld_y;
  MxqDivisor steps_per_row;
  uint32_t total_steps;
};
struct ProjGroupTable {
  ProjGroupDesc g[kGroupMax];
};
static_assert(sizeof(ProjGroupTable) <= 3584, "the table must fit the kernel-argument segment");

template <typename T>
__global__ __launch_bounds__(kProjThreads) void proj_grouped_kernel(const ProjGroupTable tab) {
  const ProjGroupDesc d = tab.g[blockIdx.y];
  if (blockIdx.x * kProjSteps >= d.total_steps) return;      // uniform: past this weight's steps
  keep_denormals();
  proj_steps<T, true>(static_cast<const T*>(d.x), d.ld_x, static_cast<T*>(d.y), d.ld_y, d.K, d.steps_per_row,
                      d.total_steps, blockIdx.x);
}

template <typename T, bool VEC, bool kRow>
__global__ __launch_bounds__(kColThreads * kColGroups) void col_kernel(
    const T* __restrict__ x, int64_t ld_x, int64_t rows, int64_t K, uint8_t* __restrict__ cdata,
    uint8_t* __restrict__ cscale, int64_t cscale_ld, uint8_t* __restrict__ rdata, uint8_t* __restrict__ rscale,
    int64_t rscale_ld, MxqDivisor groups, const int32_t* __restrict__ noop) {
  using G = StepGeom<T>;
  constexpr int EPL = Fmt<T>::kEPL, NW = sizeof(T) == 2 ? 4 : 2;   // elements, bf16 words per chunk
  constexpr int R = kColRows;
  __shared__ uint32_t s_cmax[kColGroups > 1 ? kColGroups : 1][NW][kColThreads];
  keep_denormals();
  const uint32_t lane = threadIdx.x % kColThreads, rg = threadIdx.x / kColThreads;   // rg: uniform per wave
  const uint32_t bid = xcd_run<sizeof(T) == 2 ? MXQ_COL_XCD_RUN_BF16 : MXQ_COL_XCD_RUN_FP32>(blockIdx.x, gridDim.x);
  const uint32_t band = mxq_quot(bid, groups), grp = bid - band * groups.d;
  const int64_t col0 = (int64_t)grp * (kColThreads * EPL) + (int64_t)lane * EPL;
  const int64_t rb = (int64_t)band * 32 + (int64_t)rg * R;   // this lane group's first row
  const bool in = col0 < K;

  // Loads.  Rows past the matrix's end repeat its last row (never stored, and
  // they cannot raise a column maximum).  VEC: no branch around a load, so each
  // row is used as soon as it lands; a lane past K reads the row's last chunk
  // and takes no part in the block maxima.  Otherwise elements past K load as 0.
  u32x4 w[R];
  {
    int64_t r = min(rb, rows - 1);
    const T* px = x + r * ld_x;
    if constexpr (VEC) px += in ? col0 : K - EPL;
#pragma unroll
    for (int i = 0; i < R; i++) {
      if constexpr (VEC) w[i] = stream_load(reinterpret_cast<const u32x4*>(px));
      else w[i] = load_chunk<T, false>(px, col0, K);
      if (r + 1 < rows) px += ld_x, r++;
    }
  }
  if (skipped(noop)) return;   // read once the input loads are in flight (uniform: before any barrier)

  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  u16x2 cmax[NW];
#pragma unroll
  for (int j = 0; j < NW; j++) cmax[j] = u16x2{0, 0};
  uint32_t poison = 0u;
#pragma unroll
  for (int i = 0; i < R; i++) {
    uint32_t a = chunk_amax<T>(w[i]);
    if constexpr (VEC) a = in ? a : 0u;
    const Block b = block_of_amax<T>(block_max<Fmt<T>::kLPB>(a));
    const float s = e8m0(b.eb);
    // a poisoned block's nibbles are zeroed: its y (unused) stays out of the maxima
    const Proj16<T> y = project<T>(b.poison ? 0u : fp4_of(w[i], s, T{}), s);
    if constexpr (kRow) {
      if (rb + i < rows) {
        const uint32_t code = row_code(b);
        store_payload<T, VEC>(rdata + (rb + i) * K, col0, K, payload_chunk<T>(y, code, b.poison));
        if (lane % G::kLPB == 0 && in) rscale[(rb + i) * rscale_ld + col0 / 32] = (uint8_t)code;
      }
    }
    poison |= (uint32_t)b.poison << i;
#pragma unroll
    for (int j = 0; j < NW; j++) {
      w[i][j] = y.p[j];
      cmax[j] = __builtin_elementwise_max(cmax[j], __builtin_bit_cast(u16x2, y.p[j] & 0x7FFF7FFFu));
    }
  }
  if constexpr (kColGroups > 1) {     // the band's column maxima over the lane groups
#pragma unroll
    for (int j = 0; j < NW; j++) s_cmax[rg][j][lane] = __builtin_bit_cast(uint32_t, cmax[j]);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NW; j++) {
      cmax[j] = u16x2{0, 0};
#pragma unroll
      for (int g = 0; g < kColGroups; g++)
        cmax[j] = __builtin_elementwise_max(cmax[j], __builtin_bit_cast(u16x2, s_cmax[g][j][lane]));
    }
  }

  // code = S + 127 = max(E - 8, 0) with E the bf16 exponent field of the column amax
  float sc[EPL];
  uint32_t codes[EPL];
#pragma unroll
  for (int k = 0; k < EPL; k++) {
    const uint32_t E = (uint32_t)cmax[k / 2][k % 2] >> 7;
    codes[k] = E > 8u ? E - 8u : 0u;
    sc[k] = e8m0(codes[k]);
  }
  if (rg == 0) {
    uint8_t* crow = cscale + (int64_t)band * cscale_ld;
#pragma unroll
    for (int k = 0; k < EPL; k++)
      if (col0 + k < K) crow[col0 + k] = (uint8_t)codes[k];
  }

  uint8_t* pd = cdata + rb * K;
#pragma unroll
  for (int i = 0; i < R; i++) {
    if (rb + i < rows) {
      typename PayloadChunk<T>::type q;
      if constexpr (sizeof(T) == 2) {
        q = u32x2{e4m3x4_each(w[i][0], w[i][1], sc[0], sc[1], sc[2], sc[3]),
                  e4m3x4_each(w[i][2], w[i][3], sc[4], sc[5], sc[6], sc[7])};
        if ((poison >> i) & 1u) q = u32x2{0x7F7F7F7Fu, 0x7F7F7F7Fu};
      } else {
        q = (poison >> i) & 1u ? 0x7F7F7F7Fu : e4m3x4_each(w[i][0], w[i][1], sc[0], sc[1], sc[2], sc[3]);
      }
      store_payload<T, VEC>(pd, col0, K, q);
      pd += K;
    }
  }
}

// ------------------------------------------------------------------------------------
// 128x128 tile fold, one HBM pass.  A workgroup folds J tiles that sit side by
// side in one 128-row band, so each row of the band contributes a contiguous
// run of J * 256 bytes (bf16) per load.  Each lane keeps only the E2M1 nibbles,
// block exponents and poison bits of its chunks (all in one tile); the largest
// finite block exponent of every tile is reduced with DPP inside each 16-lane
// row, readlanes (one tile per workgroup) or shuffles across the rows of the
// wave, and LDS across the workgroup's waves; then every lane folds and writes
// its payload.
// ------------------------------------------------------------------------------------
#ifndef MXQ_TILES_PER_WG
#define MXQ_TILES_PER_WG 1
#endif

constexpr int kRowMirror = 0x140;      // lane i <-> 15-i within each row of 16

// Max over each aligned group of 16 lanes.
__device__ __forceinline__ uint32_t max16(uint32_t v) {
  v = max(v, dpp<kQuadXor1>(v));
  v = max(v, dpp<kQuadXor2>(v));
  v = max(v, dpp<kRowHalfMirror>(v));
  return max(v, dpp<kRowMirror>(v));
}

template <typename T>
struct FoldGeom {
  static constexpr int kEPL = Fmt<T>::kEPL;
  static constexpr int kJ = sizeof(T) == 2 ? MXQ_TILES_PER_WG : (MXQ_TILES_PER_WG > 2 ? 2 : MXQ_TILES_PER_WG);
  static constexpr int kCPT = 128 / kEPL;                  // lanes across one tile row (16 / 32)
  static constexpr int kLPR = kCPT * kJ;                   // lanes across the band row (<= 64)
  static constexpr int kThreads = sizeof(T) == 2 ? MXQ_FOLD_THREADS_BF16 : MXQ_FOLD_THREADS_FP32;
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kRun = sizeof(T) == 2 ? MXQ_FOLD_XCD_RUN_BF16 : MXQ_FOLD_XCD_RUN_FP32;
  static constexpr int kRowsPerPass = kThreads / kLPR;
  static constexpr int kPasses = 128 / kRowsPerPass;
  static_assert(kLPR <= 64, "a band row must fit in one wave");
  static_assert(kThreads % 64 == 0 && kThreads <= 1024 && kRowsPerPass * kPasses == 128, "fold geometry");
};

// The fold of one group of J side-by-side tiles (tile row tr, group tg) by the
// whole workgroup (a barrier inside); s_max: G::kWaves * J words of LDS.  A
// non-zero no-op flag leaves every output untouched.  FULL: whole tile groups
// (rows a multiple of 128, K of 128 J, a band's payload under 2 GiB), so no
// bounds checks; payload stores are buffer stores (nt sc1) off the band's start.
template <typename T, bool VEC, bool FULL = false>
__device__ __forceinline__ void fold_tiles(const T* __restrict__ x, int64_t ld_x, int64_t rows, int64_t K,
                                           uint8_t* __restrict__ data, uint8_t* __restrict__ tile_code,
                                           int64_t tile_ld, uint32_t tiles_per_row, uint32_t tr, uint32_t tg,
                                           const int32_t* __restrict__ noop, uint32_t (*s_max)[FoldGeom<T>::kJ]) {
  using G = FoldGeom<T>;
  constexpr int EPL = G::kEPL, J = G::kJ, CPT = G::kCPT, LPR = G::kLPR, P = G::kPasses;
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t j = (tid % LPR) / CPT;                    // this lane's tile within the group
  const int64_t r0 = (int64_t)tr * 128 + tid / LPR;
  const int64_t col0 = (int64_t)tg * (128 * J) + (tid % LPR) * EPL;

  static_assert(VEC || !FULL, "the full form takes the 16-byte path");
  u32x4 w[P];
#pragma unroll
  for (int i = 0; i < P; i++) {
    const int64_t r = r0 + i * G::kRowsPerPass;
    if constexpr (FULL)
      w[i] = stream_load(reinterpret_cast<const u32x4*>(x + r * ld_x + col0));
    else
      w[i] = (r < rows) ? load_chunk<T, VEC>(x + r * ld_x, col0, K) : u32x4{0u, 0u, 0u, 0u};
  }
  if (skipped(noop)) return;   // read once the input loads are in flight (uniform: before the barrier)
  uint32_t f[P], eb[P];
  uint64_t poisoned = 0u;                                  // bit i: chunk i's block is poisoned
  uint32_t m = 1u;
#pragma unroll
  for (int i = 0; i < P; i++) {
    const Block b = chunk_block<T>(w[i]);
    eb[i] = b.eb;
    f[i] = fp4_of(w[i], e8m0(b.eb), T{});
    poisoned |= (uint64_t)b.poison << i;
    if (!b.poison) m = max(m, b.eb);
  }
  m = max16(m);                                            // every lane: its 16-lane row's maximum
  if constexpr (J == 1 && MXQ_FOLD_READLANE) {
    // One tile per workgroup: the whole wave is one tile, so its maximum is the
    // largest of the four rows' maxima, read as scalars (no shuffle through the
    // LDS crossbar, and no wait on one, between the loads and the barrier).
    m = max(max((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 16)),
            max((uint32_t)__builtin_amdgcn_readlane((int)m, 32), (uint32_t)__builtin_amdgcn_readlane((int)m, 48)));
  } else {
    if constexpr (CPT == 32) m = max(m, (uint32_t)__shfl_xor((int)m, 16, 64));
#pragma unroll
    for (int off = LPR; off < 64; off *= 2) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  }
  if (lane < (uint32_t)LPR && lane % CPT == 0) s_max[wave][j] = m;
  __syncthreads();
#pragma unroll
  for (int v = 0; v < G::kWaves; v++) m = max(m, s_max[v][j]);
  const uint32_t code = m > 6u ? m - 6u : 0u;              // S + 127 = max(M - 6, -127) + 127
  const uint32_t tc = tg * J + j;
  if (tid < (uint32_t)LPR && tid % CPT == 0 && tc < tiles_per_row) tile_code[(int64_t)tr * tile_ld + tc] = (uint8_t)code;

#pragma unroll
  for (int i = 0; i < P; i++) {
    const int64_t r = r0 + i * G::kRowsPerPass;
    const Proj16<T> p = project<T>(f[i], e8m0(eb[i]));
    const auto q = payload_chunk<T>(p, code, (poisoned >> i) & 1u);
    if constexpr (FULL)
      stream_store_at(q, data + (int64_t)tr * 128 * K, (uint32_t)((r - (int64_t)tr * 128) * K + col0));
    else if (r < rows)
      store_payload<T, VEC>(data + r * K, col0, K, q);
  }
}

template <typename T, bool VEC, bool FULL>
__global__ __launch_bounds__(FoldGeom<T>::kThreads) void block128_kernel(
    const T* __restrict__ x, int64_t ld_x, int64_t rows, int64_t K, uint8_t* __restrict__ data,
    uint8_t* __restrict__ tile_code, int64_t tile_ld, uint32_t tiles_per_row, MxqDivisor groups_per_row,
    const int32_t* __restrict__ noop) {
  __shared__ uint32_t s_max[FoldGeom<T>::kWaves][FoldGeom<T>::kJ];
  keep_denormals();
  const uint32_t bid = xcd_run<FoldGeom<T>::kRun>(blockIdx.x, gridDim.x);
  const uint32_t tr = mxq_quot(bid, groups_per_row), tg = bid - tr * groups_per_row.d;
  fold_tiles<T, VEC, FULL>(x, ld_x, rows, K, data, tile_code, tile_ld, tiles_per_row, tr, tg, noop, s_max);
}

// Grouped fold: blockIdx.y is the weight and blockIdx.x the tile group within
// it, with the single fold's workgroup and body (fold_tiles).
struct FoldGroupDesc {
  const void* x;
  int64_t ld_x, rows, K;
  uint8_t* data;
  uint8_t* tile_code;
  int64_t tile_ld;
  MxqDivisor groups_per_row;
  uint32_t tiles_per_row, n_groups;
};
struct FoldGroupTable {
  FoldGroupDesc g[kGroupMax];
};
static_assert(sizeof(FoldGroupTable) <= 3840, "the table must fit the kernel-argument segment");

template <typename T>
__global__ __launch_bounds__(FoldGeom<T>::kThreads) void block128_grouped_kernel(const FoldGroupTable tab) {
  __shared__ uint32_t s_max[FoldGeom<T>::kWaves][FoldGeom<T>::kJ];
  const FoldGroupDesc d = tab.g[blockIdx.y];
  if (blockIdx.x >= d.n_groups) return;                      // uniform: past this weight's tiles
  keep_denormals();
  // bf16: the single fold's tile runs per XCD, within the weight (the XCD of a
  // workgroup follows blockIdx.x when the grid's x extent is a multiple of 8):
  // 48 weights of 1024 x 2048 in 51.0 -> 48.7 us; fp32 keeps the plain order
  // (80.2 -> 81.5 us with its runs of 4)
  const uint32_t bid = xcd_run<sizeof(T) == 2 ? FoldGeom<T>::kRun : 1>(blockIdx.x, d.n_groups);
  const uint32_t tr = mxq_quot(bid, d.groups_per_row), tg = bid - tr * d.groups_per_row.d;
  fold_tiles<T, true>(static_cast<const T*>(d.x), d.ld_x, d.rows, d.K, d.data, d.tile_code, d.tile_ld,
                      d.tiles_per_row, tr, tg, nullptr, s_max);
}

// ------------------------------------------------------------------------------------
// Decode: FP8 payload * 2^(code - 127).  The conversions return a negative quiet
// NaN for NaN payloads and code 255; those (rare) chunks are rewritten to the
// canonical positive quiet NaN.
// ------------------------------------------------------------------------------------
template <bool kE5M2>
__device__ __forceinline__ u32x4 decode8_bf16(u32x2 q, float s) {
  u32x4 o;
  if constexpr (kE5M2) {
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(q[0], s, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(q[0], s, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(q[1], s, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(q[1], s, true));
  } else {
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[0], s, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[0], s, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[1], s, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[1], s, true));
  }
  return o;
}
// One f32 from byte SEL of q.  (The packed two-result f32 forms of these
// conversions are not used: the compiler's model of their second result is not
// reliable.)
template <bool kE5M2, int SEL>
__device__ __forceinline__ uint32_t decode1_f32(uint32_t q, float s) {
  if constexpr (kE5M2) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_f32_bf8(q, s, SEL));
  else return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_f32_fp8(q, s, SEL));
}
// Any NaN payload byte among the 8 (E4M3: magnitude 0x7F; E5M2: above 0x7C).
template <bool kE5M2>
__device__ __forceinline__ bool has_nan_byte(u32x2 q) {
  constexpr uint32_t add = kE5M2 ? 0x03030303u : 0x01010101u;
  return ((((q[0] & 0x7F7F7F7Fu) + add) | ((q[1] & 0x7F7F7F7Fu) + add)) & 0x80808080u) != 0u;
}

// Scale layouts of the decode: one code per 1x32 row block, per 128x128 tile,
// or per 32x1 column block (then each of a lane's 8 columns has its own code).
enum { kLayRow = 0, kLayTile = 1, kLayCol = 2 };

// 8 FP8 bytes -> 8 bf16 with one scale per element: each byte pair is decoded
// at both elements' scales and the halves are picked.
template <bool kE5M2, bool HI>
__device__ __forceinline__ uint32_t bf16_pair_of_fp8(uint32_t q, float s) {
  if constexpr (kE5M2) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(q, s, HI));
  else return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, s, HI));
}
template <bool kE5M2, bool HI>
__device__ __forceinline__ uint32_t bf16_pair_of_fp8_each(uint32_t q, float s_lo, float s_hi) {
  return (bf16_pair_of_fp8<kE5M2, HI>(q, s_lo) & 0x0000FFFFu) | (bf16_pair_of_fp8<kE5M2, HI>(q, s_hi) & 0xFFFF0000u);
}
template <bool kE5M2>
__device__ __forceinline__ u32x4 decode8_bf16_each(u32x2 q, const float (&s)[8]) {
  return u32x4{bf16_pair_of_fp8_each<kE5M2, false>(q[0], s[0], s[1]), bf16_pair_of_fp8_each<kE5M2, true>(q[0], s[2], s[3]),
               bf16_pair_of_fp8_each<kE5M2, false>(q[1], s[4], s[5]), bf16_pair_of_fp8_each<kE5M2, true>(q[1], s[6], s[7])};
}


// The decode's body: workgroup wg's kDequantSteps steps of one weight.  The
// single and grouped kernels both run it.
template <typename TO, bool kE5M2, int kLay, bool VEC, int kDequantSteps>
__device__ __forceinline__ void dequant_steps(const uint8_t* __restrict__ data, const uint8_t* __restrict__ scale,
                                              int64_t scale_ld, int64_t K, TO* __restrict__ out, int64_t ld_out,
                                              MxqDivisor steps_per_row, uint32_t total_steps, uint32_t wg) {
  // 8 payload bytes per lane per step; a step is kDequantThreads * 8 elements of one row.
  constexpr int kDequantThreads = DequantShape<TO>::kThreads;
  // Lane geometry: bf16 output takes 8 consecutive elements per lane (one 16-byte
  // store).  fp32 output (kSplit) takes two groups of 4, half a step apart, so
  // that each of the lane's two 16-byte stores is part of one contiguous
  // 64 x 16-byte store of the wave: two adjacent 16-byte stores per lane cover
  // only half lines per instruction and run far slower.
  constexpr bool kSplit = sizeof(TO) == 4;
  constexpr int64_t kHalf = (int64_t)kDequantThreads * 4;
  const uint32_t tid = threadIdx.x;
  const int64_t lane_col = (int64_t)tid * (kSplit ? 4 : 8);
  // All of the workgroup's loads are issued before any decode or store.
  u32x2 qs[kDequantSteps];                                  // kSplit: [0] the first group's 4 bytes, [1] the second's
  uint32_t cs[kDequantSteps];                               // the step's code (row, tile layouts)
  uint32_t cs_b[kSplit ? kDequantSteps : 1];                // kSplit: the second group's code
  u32x2 ccs[kLay == kLayCol ? kDequantSteps : 1];           // the 8 columns' codes (column layout)
#pragma unroll
  for (int u = 0; u < kDequantSteps; u++) {
    qs[u] = u32x2{0u, 0u};
    cs[u] = 0u;
    if constexpr (kSplit) cs_b[u] = 0u;
    if constexpr (kLay == kLayCol) ccs[u] = u32x2{0u, 0u};
    const uint32_t step = wg * kDequantSteps + u;
    if (step >= total_steps) continue;
    const uint32_t row = mxq_quot(step, steps_per_row), seg = step - row * steps_per_row.d;
    const int64_t col0 = (int64_t)seg * (kDequantThreads * 8) + lane_col;
    if (col0 >= K) continue;
    const uint8_t* drow = data + (int64_t)row * K;
    if constexpr (kSplit) {
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int64_t c = col0 + h * kHalf;
        if (c >= K) continue;
        if (VEC) {
          qs[u][h] = stream_load(reinterpret_cast<const uint32_t*>(drow + c));
        } else {
          for (int i = 0; i < 4; i++)
            if (c + i < K) qs[u][h] |= (uint32_t)drow[c + i] << (8 * i);
        }
        if constexpr (kLay == kLayCol) {
          const uint8_t* srow = scale + (int64_t)(row / 32) * scale_ld;
          if (VEC) {
            ccs[u][h] = *reinterpret_cast<const uint32_t*>(srow + c);
          } else {
            for (int i = 0; i < 4; i++)
              if (c + i < K) ccs[u][h] |= (uint32_t)srow[c + i] << (8 * i);
          }
        } else {
          const uint32_t code = kLay == kLayTile ? scale[(int64_t)(row / 128) * scale_ld + c / 128]
                                                 : scale[(int64_t)row * scale_ld + c / 32];
          if (h == 0) cs[u] = code;
          else cs_b[u] = code;
        }
      }
      continue;
    }
    if (VEC) {
      qs[u] = stream_load(reinterpret_cast<const u32x2*>(drow + col0));
    } else {
      for (int i = 0; i < 8; i++)
        if (col0 + i < K) qs[u][i / 4] |= (uint32_t)drow[col0 + i] << (8 * (i % 4));
    }
    if constexpr (kLay == kLayCol) {
      const uint8_t* srow = scale + (int64_t)(row / 32) * scale_ld;
      if (VEC) {
        ccs[u] = *reinterpret_cast<const u32x2*>(srow + col0);
      } else {
        for (int i = 0; i < 8; i++)
          if (col0 + i < K) ccs[u][i / 4] |= (uint32_t)srow[col0 + i] << (8 * (i % 4));
      }
    } else {
      cs[u] = kLay == kLayTile ? scale[(int64_t)(row / 128) * scale_ld + col0 / 128]
                               : scale[(int64_t)row * scale_ld + col0 / 32];
    }
  }
#pragma unroll
  for (int u = 0; u < kDequantSteps; u++) {
    const uint32_t step = wg * kDequantSteps + u;
    if (step >= total_steps) break;
    const uint32_t row = mxq_quot(step, steps_per_row), seg = step - row * steps_per_row.d;
    const int64_t col0 = (int64_t)seg * (kDequantThreads * 8) + lane_col;
    if (col0 >= K) continue;
    const u32x2 q = qs[u];
    float s8[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      if constexpr (kLay == kLayCol) s8[i] = e8m0((ccs[u][i / 4] >> (8 * (i % 4))) & 0xFFu);
      else if constexpr (kSplit) s8[i] = e8m0(i < 4 ? cs[u] : cs_b[u]);
      else s8[i] = e8m0(cs[u]);
    }
    const float s = s8[0];
    bool fix_nan = kLay == kLayCol || cs[u] == 255u || has_nan_byte<kE5M2>(q);
    if constexpr (kSplit) fix_nan = fix_nan || cs_b[u] == 255u;
    TO* orow = out + (int64_t)row * ld_out;
    if constexpr (sizeof(TO) == 2) {
      u32x4 o = kLay == kLayCol ? decode8_bf16_each<kE5M2>(q, s8) : decode8_bf16<kE5M2>(q, s);
      if (fix_nan) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const uint32_t h = (o[i / 2] >> (16 * (i % 2))) & 0xFFFFu;
          if ((h & 0x7FFFu) > 0x7F80u) o[i / 2] = (o[i / 2] & ~(0xFFFFu << (16 * (i % 2)))) | (0x7FC0u << (16 * (i % 2)));
        }
      }
      if (VEC) {
        stream_store(o, reinterpret_cast<u32x4*>(orow + col0));
      } else {
        for (int i = 0; i < 8; i++)
          if (col0 + i < K) orow[col0 + i] = (uint16_t)(o[i / 2] >> (16 * (i % 2)));
      }
    } else {
      uint32_t f[8] = {decode1_f32<kE5M2, 0>(q[0], s8[0]), decode1_f32<kE5M2, 1>(q[0], s8[1]),
                       decode1_f32<kE5M2, 2>(q[0], s8[2]), decode1_f32<kE5M2, 3>(q[0], s8[3]),
                       decode1_f32<kE5M2, 0>(q[1], s8[4]), decode1_f32<kE5M2, 1>(q[1], s8[5]),
                       decode1_f32<kE5M2, 2>(q[1], s8[6]), decode1_f32<kE5M2, 3>(q[1], s8[7])};
      if (fix_nan) {
#pragma unroll
        for (int i = 0; i < 8; i++)
          if ((f[i] & 0x7FFFFFFFu) > 0x7F800000u) f[i] = 0x7FC00000u;
      }
      // the two groups: elements col0 .. col0+3 and col0+kHalf .. col0+kHalf+3
      if (VEC) {
        stream_store(u32x4{f[0], f[1], f[2], f[3]}, reinterpret_cast<u32x4*>(orow + col0));
        if (col0 + kHalf < K) stream_store(u32x4{f[4], f[5], f[6], f[7]}, reinterpret_cast<u32x4*>(orow + col0 + kHalf));
      } else {
        for (int i = 0; i < 8; i++) {
          const int64_t c = col0 + (i < 4 ? i : kHalf + i - 4);
          if (c < K) orow[c] = f[i];
        }
      }
    }
  }
}

template <typename TO, bool kE5M2, int kLay, bool VEC>
__global__ __launch_bounds__(DequantShape<TO>::kThreads) void dequant_kernel(const uint8_t* __restrict__ data,
                                                           const uint8_t* __restrict__ scale, int64_t scale_ld,
                                                           int64_t K, TO* __restrict__ out, int64_t ld_out,
                                                           MxqDivisor steps_per_row, uint32_t total_steps) {
  keep_denormals();
  dequant_steps<TO, kE5M2, kLay, VEC, DequantShape<TO>::kSteps>(
      data, scale, scale_ld, K, out, ld_out, steps_per_row, total_steps,
      xcd_run<kLay == kLayRow ? kDequantXcdRun : 1>(blockIdx.x, gridDim.x));
}

// Grouped decode, on the grouped row lift's pattern: blockIdx.y is the weight,
// blockIdx.x the workgroup within it; one payload format, scale layout and
// output dtype per launch.  Aligned (VEC) weights only.
struct DequantGroupDesc {
  const uint8_t* data;
  const uint8_t* scale;
  int64_t scale_ld, K;
  void* out;
  int64_t ld_out;
  MxqDivisor steps_per_row;
  uint32_t total_steps;
};
struct DequantGroupTable {
  DequantGroupDesc g[kGroupMax];
};
static_assert(sizeof(DequantGroupTable) <= 3584, "the table must fit the kernel-argument segment");

template <typename TO, bool kE5M2, int kLay>
__global__ __launch_bounds__(DequantShape<TO>::kThreads) void dequant_grouped_kernel(const DequantGroupTable tab) {
  const DequantGroupDesc d = tab.g[blockIdx.y];
  if (blockIdx.x * kDequantGroupedSteps >= d.total_steps) return;   // uniform: past this weight's steps
  keep_denormals();
  dequant_steps<TO, kE5M2, kLay, true, kDequantGroupedSteps>(d.data, d.scale, d.scale_ld, d.K,
                                                                    static_cast<TO*>(d.out), d.ld_out,
                                                                    d.steps_per_row, d.total_steps, blockIdx.x);
}

// ------------------------------------------------------------------------------------
// Packed MXFP4 (the deployment format): E2M1 nibble pairs, element 2i in the low
// nibble of byte i, rows of ceil(K/2) bytes, plus one E8M0 code per 1x32 block.
// ([QAT] Description: the deployment weight is E2M1 payloads with 1x32
// power-of-two UE8M0 scales; Known limitations: above 6 * 2^125 the packed form
// takes scale 2^126 where the projection saturates.)  The packed side uses the
// bf16 chunk geometry: 8 elements (4 packed bytes) per lane, 4 lanes per block.
// ------------------------------------------------------------------------------------
template <typename T>
struct Nibbles;
template <>
struct Nibbles<uint16_t> { typedef uint32_t type; };   // 8 nibbles per bf16 chunk
template <>
struct Nibbles<uint32_t> { typedef uint16_t type; };   // 4 nibbles per fp32 chunk

// The packed encode's body: workgroup wg's kQ4Steps steps of one weight.  The
// single and grouped kernels both run it.
template <typename T, bool VEC, bool FULL = false>
__device__ __forceinline__ void quantize_mxfp4_steps(const T* __restrict__ x, int64_t ld_x, int64_t K,
                                                     uint8_t* __restrict__ packed, uint8_t* __restrict__ scale,
                                                     int64_t scale_ld, MxqDivisor steps_per_row, uint32_t total_steps,
                                                     uint32_t wg) {
  using G = StepGeom<T, kQ4Threads>;
  using N = typename Nibbles<T>::type;
  const uint32_t tid = threadIdx.x;
  const int64_t lane_col = (int64_t)(tid / G::kLPB) * 32 + (tid % G::kLPB) * G::kEPL;
  const int64_t pw = (K + 1) / 2;
  u32x4 w[kQ4Steps];
#pragma unroll
  for (int u = 0; u < kQ4Steps; u++) {
    const uint32_t step = wg * kQ4Steps + u;
    w[u] = u32x4{0u, 0u, 0u, 0u};
    if (FULL || step < total_steps) {
      const uint32_t row = mxq_quot(step, steps_per_row), seg = step - row * steps_per_row.d;
      if constexpr (FULL)
        w[u] = stream_load(reinterpret_cast<const u32x4*>(x + (int64_t)row * ld_x + seg * G::kElemsPerStep + lane_col));
      else
        w[u] = load_chunk<T, VEC>(x + (int64_t)row * ld_x, seg * G::kElemsPerStep + lane_col, K);
    }
  }
  using CG = CodeGather<G::kLPB>;
  constexpr bool kLast =
      FULL && MXQ_Q4_CODE_WORDS && (sizeof(T) == 2 ? MXQ_Q4_CODES_LAST_BF16 : MXQ_Q4_CODES_LAST_FP32);
  uint32_t cw[kQ4Steps];                                   // kLast: each step's gathered codes and row
  uint8_t* cr[kQ4Steps];
#pragma unroll
  for (int u = 0; u < kQ4Steps; u++) {
    const uint32_t step = wg * kQ4Steps + u;
    if (FULL || step < total_steps) {
      const uint32_t row = mxq_quot(step, steps_per_row), seg = step - row * steps_per_row.d;
      const int64_t col0 = seg * G::kElemsPerStep + lane_col;
      const Block b = chunk_block<T, 253>(w[u]);
      const uint32_t f = b.poison ? 0u : fp4_of(w[u], e8m0(b.eb), T{});
      if constexpr (FULL) {
        stream_store_at((N)f, packed + (int64_t)row * pw, (uint32_t)(col0 / 2));
        uint8_t* const crow = scale + (int64_t)row * scale_ld + seg * G::kBlocksPerStep;
        const uint32_t code = b.poison ? 255u : b.eb;
        if constexpr (kLast) {
          cw[u] = CG::gather(code);
          cr[u] = crow;
        } else if constexpr (MXQ_Q4_CODE_WORDS) {
          const uint32_t codes = CG::gather(code);
          if (tid % CG::kLanes == 0) CG::store(crow, tid / G::kLPB, codes);
        } else {
          if (tid % G::kLPB == 0) store_code(crow, tid / G::kLPB, code);
        }
        continue;
      }
      if (col0 < K) {
        uint8_t* prow = packed + (int64_t)row * pw;
        if constexpr (VEC) {
          stream_store((N)f, reinterpret_cast<N*>(prow + col0 / 2));
        } else {
          for (int i = 0; i < G::kEPL; i += 2)
            if (col0 + i < K)
              prow[(col0 + i) / 2] = (uint8_t)((f >> (4 * i)) & (col0 + i + 1 < K ? 0xFFu : 0x0Fu));
        }
        if (tid % G::kLPB == 0) scale[(int64_t)row * scale_ld + col0 / 32] = (uint8_t)(b.poison ? 255u : b.eb);
      }
    }
  }
  if constexpr (kLast) {
    // the block codes go out after every packed-payload store of the workgroup
#pragma unroll
    for (int u = 0; u < kQ4Steps; u++)
      if (tid % CG::kLanes == 0) CG::store(cr[u], tid / G::kLPB, cw[u]);
  }
}

template <typename T, bool VEC, bool FULL>
__global__ __launch_bounds__(kQ4Threads) void quantize_mxfp4_kernel(const T* __restrict__ x, int64_t ld_x, int64_t K,
                                                                  uint8_t* __restrict__ packed,
                                                                  uint8_t* __restrict__ scale, int64_t scale_ld,
                                                                  MxqDivisor steps_per_row, uint32_t total_steps) {
  keep_denormals();
  quantize_mxfp4_steps<T, VEC, FULL>(x, ld_x, K, packed, scale, scale_ld, steps_per_row, total_steps, blockIdx.x);
}

// Grouped packed encode, on the grouped row lift's pattern and with its
// descriptor (data = the packed nibble pairs).  Aligned (VEC) weights only.
template <typename T>
__global__ __launch_bounds__(kQ4Threads) void quantize_mxfp4_grouped_kernel(const RowGroupTable tab) {
  const RowGroupDesc d = tab.g[blockIdx.y];
  if (blockIdx.x * kQ4Steps >= d.total_steps) return;       // uniform: past this weight's steps
  keep_denormals();
  quantize_mxfp4_steps<T, true, false>(static_cast<const T*>(d.x), d.ld_x, d.K, d.data, d.scale, d.scale_ld,
                                       d.steps_per_row, d.total_steps, blockIdx.x);
}

// Eight packed nibbles at E8M0 code c -> four bf16 pairs of p * 2^(c-127), with
// Inf where that exceeds bf16 (codes 253 and 254) and canonical NaN for c = 255.
__device__ __forceinline__ u32x4 decode8_fp4(uint32_t f, uint32_t c) {
  // Codes 253/254 are decoded two binades lower (exact) and moved back up with
  // an exponent add that saturates to Inf.
  const bool high = c >= 253u && c != 255u;
  const float s = e8m0(high ? c - 2u : c);
  u32x4 o{bf16_pair<0>(f, s), bf16_pair<1>(f, s), bf16_pair<2>(f, s), bf16_pair<3>(f, s)};
  if (c == 255u) return u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  if (high) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const uint32_t h = (o[i / 2] >> (16 * (i % 2))) & 0xFFFFu;
      uint32_t r = h;
      if ((h & 0x7FFFu) != 0u) {
        const uint32_t E = ((h >> 7) & 0xFFu) + 2u;
        r = E >= 255u ? ((h & 0x8000u) | 0x7F80u) : h + (2u << 7);
      }
      o[i / 2] = (o[i / 2] & ~(0xFFFFu << (16 * (i % 2)))) | (r << (16 * (i % 2)));
    }
  }
  return o;
}

template <typename TO, bool VEC>
__global__ __launch_bounds__(kDq4Threads) void dequantize_mxfp4_kernel(const uint8_t* __restrict__ packed,
                                                                    const uint8_t* __restrict__ scale,
                                                                    int64_t scale_ld, int64_t K,
                                                                    TO* __restrict__ out, int64_t ld_out,
                                                                    MxqDivisor steps_per_row, uint32_t total_steps) {
  // Lane geometry as in the FP8 decode: bf16 output takes 8 consecutive
  // elements (4 packed bytes) per lane; fp32 output (kSplit) takes two groups of
  // 4 (2 packed bytes each) half a step apart, so each 16-byte store of the lane
  // is part of one contiguous store of the wave.
  constexpr bool kSplit = sizeof(TO) == 4;
  constexpr int64_t kHalf = (int64_t)kDq4Threads * 4;
  keep_denormals();
  const uint32_t tid = threadIdx.x;
  const int64_t lane_col = (int64_t)tid * (kSplit ? 4 : 8), pw = (K + 1) / 2;
  // All of the workgroup's loads are issued before any decode or store.
  uint32_t fs[kDq4Steps], cs[kDq4Steps];
  uint32_t fs_b[kSplit ? kDq4Steps : 1], cs_b[kSplit ? kDq4Steps : 1];   // kSplit: the second group
#pragma unroll
  for (int u = 0; u < kDq4Steps; u++) {
    fs[u] = 0u;
    cs[u] = 0u;
    if constexpr (kSplit) fs_b[u] = 0u, cs_b[u] = 0u;
    const uint32_t step = blockIdx.x * kDq4Steps + u;
    if (step >= total_steps) continue;
    const uint32_t row = mxq_quot(step, steps_per_row), seg = step - row * steps_per_row.d;
    const int64_t col0 = (int64_t)seg * (kDq4Threads * 8) + lane_col;
    if (col0 >= K) continue;
    const uint8_t* prow = packed + (int64_t)row * pw;
    if constexpr (kSplit) {
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int64_t c = col0 + h * kHalf;
        if (c >= K) continue;
        uint32_t f = 0u;
        if (VEC) {
          f = stream_load(reinterpret_cast<const uint16_t*>(prow + c / 2));
        } else {
          for (int i = 0; i < 4; i += 2)
            if (c + i < K) f |= (uint32_t)prow[(c + i) / 2] << (4 * i);
        }
        const uint32_t code = scale[(int64_t)row * scale_ld + c / 32];
        if (h == 0) fs[u] = f, cs[u] = code;
        else fs_b[u] = f, cs_b[u] = code;
      }
      continue;
    }
    if (VEC) {
      fs[u] = stream_load(reinterpret_cast<const uint32_t*>(prow + col0 / 2));
    } else {
      for (int i = 0; i < 8; i += 2)
        if (col0 + i < K) fs[u] |= (uint32_t)prow[(col0 + i) / 2] << (4 * i);
    }
    cs[u] = scale[(int64_t)row * scale_ld + col0 / 32];
  }
#pragma unroll
  for (int u = 0; u < kDq4Steps; u++) {
    const uint32_t step = blockIdx.x * kDq4Steps + u;
    if (step >= total_steps) break;
    const uint32_t row = mxq_quot(step, steps_per_row), seg = step - row * steps_per_row.d;
    const int64_t col0 = (int64_t)seg * (kDq4Threads * 8) + lane_col;
    if (col0 >= K) continue;
    TO* orow = out + (int64_t)row * ld_out;
    if constexpr (kSplit) {
      // each group's 4 nibbles decode through the bf16 path (exact), then widen
      const u32x4 oa = decode8_fp4(fs[u], cs[u]), ob = decode8_fp4(fs_b[u], cs_b[u]);
      const uint32_t h4[8] = {oa[0] & 0xFFFFu, oa[0] >> 16, oa[1] & 0xFFFFu, oa[1] >> 16,
                              ob[0] & 0xFFFFu, ob[0] >> 16, ob[1] & 0xFFFFu, ob[1] >> 16};
      uint32_t fo[8];
#pragma unroll
      for (int i = 0; i < 8; i++) fo[i] = (h4[i] & 0x7FFFu) > 0x7F80u ? 0x7FC00000u : h4[i] << 16;   // exact
      if (VEC) {
        stream_store(u32x4{fo[0], fo[1], fo[2], fo[3]}, reinterpret_cast<u32x4*>(orow + col0));
        if (col0 + kHalf < K) stream_store(u32x4{fo[4], fo[5], fo[6], fo[7]}, reinterpret_cast<u32x4*>(orow + col0 + kHalf));
      } else {
        for (int i = 0; i < 8; i++) {
          const int64_t c = col0 + (i < 4 ? i : kHalf + i - 4);
          if (c < K) orow[c] = fo[i];
        }
      }
      continue;
    }
    const u32x4 o = decode8_fp4(fs[u], cs[u]);
    if constexpr (sizeof(TO) == 2) {
      if (VEC) {
        stream_store(o, reinterpret_cast<u32x4*>(orow + col0));
      } else {
        for (int i = 0; i < 8; i++)
          if (col0 + i < K) orow[col0 + i] = (uint16_t)(o[i / 2] >> (16 * (i % 2)));
      }
    } else {
      uint32_t fo[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t h = (o[i / 2] >> (16 * (i % 2))) & 0xFFFFu;
        fo[i] = (h & 0x7FFFu) > 0x7F80u ? 0x7FC00000u : h << 16;      // bf16 -> fp32 is exact
      }
      if (VEC) {
        stream_store(u32x4{fo[0], fo[1], fo[2], fo[3]}, reinterpret_cast<u32x4*>(orow + col0));
        stream_store(u32x4{fo[4], fo[5], fo[6], fo[7]}, reinterpret_cast<u32x4*>(orow + col0 + 4));
      } else {
        for (int i = 0; i < 8; i++)
          if (col0 + i < K) orow[col0 + i] = fo[i];
      }
    }
  }
}

// RTNE_E4M3(p * 2^ds) of eight packed nibbles, ds <= 6.  p * 2^ds is made exact
// in bf16 first (scale 2^max(ds, -126)); any remaining shift is applied by the
// E4M3 conversion's own scale, so there is a single rounding.
__device__ __forceinline__ u32x2 e4m3x8_of_fp4(uint32_t f, int ds) {
  const int k = ds >= -126 ? 0 : -126 - ds;
  const float sd = e8m0((uint32_t)(127 + ds + k)), se = e8m0((uint32_t)(127 + k));
  return u32x2{e4m3x4(bf16_pair<0>(f, sd), bf16_pair<1>(f, sd), se), e4m3x4(bf16_pair<2>(f, sd), bf16_pair<3>(f, sd), se)};
}

// MXFP8 row lift from packed MXFP4: each lane takes 16 elements (8 packed bytes
// in, 16 payload bytes out), so a block of 32 spans two lanes; even lanes write
// the block's code.  A step is kPackedThreads * 16 elements of one row.
template <bool VEC, bool FULL>
__global__ __launch_bounds__(kPackedThreads) void packed_convert_kernel(const uint8_t* __restrict__ packed,
                                                                  const uint8_t* __restrict__ scale,
                                                                  int64_t scale_ld, int64_t K,
                                                                  uint8_t* __restrict__ data,
                                                                  uint8_t* __restrict__ code_out, int64_t code_ld,
                                                                  MxqDivisor steps_per_row, uint32_t total_steps) {
  keep_denormals();
  const uint32_t tid = threadIdx.x, wg = xcd_run<kPackedXcdRun>(blockIdx.x, gridDim.x);
  const int64_t lane_col = (int64_t)tid * 16, pw = (K + 1) / 2;
  // All of the workgroup's loads are issued before any conversion or store.
  u32x2 f[kPackedSteps];
  uint32_t c[kPackedSteps];
#pragma unroll
  for (int u = 0; u < kPackedSteps; u++) {
    f[u] = u32x2{0u, 0u};
    c[u] = 0u;
    const uint32_t step = wg * kPackedSteps + u;
    if (!FULL && step >= total_steps) continue;
    const uint32_t row = mxq_quot(step, steps_per_row), seg = step - row * steps_per_row.d;
    const int64_t col0 = (int64_t)seg * (kPackedThreads * 16) + lane_col;
    if (!FULL && col0 >= K) continue;
    const uint8_t* prow = packed + (int64_t)row * pw;
    if (VEC) {
      f[u] = stream_load(reinterpret_cast<const u32x2*>(prow + col0 / 2));
    } else {
      for (int i = 0; i < 16; i += 2)
        if (col0 + i < K) f[u][i / 8] |= (uint32_t)prow[(col0 + i) / 2] << (4 * (i % 8));
    }
    c[u] = scale[(int64_t)row * scale_ld + col0 / 32];
  }
#pragma unroll
  for (int u = 0; u < kPackedSteps; u++) {
    const uint32_t step = wg * kPackedSteps + u;
    if (!FULL && step >= total_steps) break;
    const uint32_t row = mxq_quot(step, steps_per_row), seg = step - row * steps_per_row.d;
    const int64_t col0 = (int64_t)seg * (kPackedThreads * 16) + lane_col;
    if (!FULL && col0 >= K) continue;
    // branch-free (convert, then select the poisoned form), so that no load
    // is sunk below a test of the other
    const bool poison = c[u] == 255u;
    const int ds = (int)min(c[u], 6u);
    const u32x2 lo = e4m3x8_of_fp4(f[u][0], ds), hi = e4m3x8_of_fp4(f[u][1], ds);
    const u32x4 q = poison ? u32x4{0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu} : u32x4{lo[0], lo[1], hi[0], hi[1]};
    const uint32_t code = poison ? 255u : (c[u] > 6u ? c[u] - 6u : 0u);   // S = max(e - 6, -127)
    uint8_t* drow = data + (int64_t)row * K;
    if constexpr (FULL) {
      stream_store_at(q, drow, (uint32_t)col0);
      uint8_t* const crow = code_out + (int64_t)row * code_ld + seg * (kPackedThreads / 2);
      if constexpr (MXQ_PACKED_CODE_WORDS) {
        using CG = CodeGather<2>;
        const uint32_t codes = CG::gather(code);
        if (tid % CG::kLanes == 0) CG::store(crow, tid / 2, codes);
      } else {
        if (tid % 2 == 0) store_code(crow, tid / 2, code);
      }
      continue;
    }
    if (VEC) {
      stream_store(q, reinterpret_cast<u32x4*>(drow + col0));
    } else {
      for (int i = 0; i < 16; i++)
        if (col0 + i < K) drow[col0 + i] = (uint8_t)(q[i / 4] >> (8 * (i % 4)));
    }
    if (tid % 2 == 0) code_out[(int64_t)row * code_ld + col0 / 32] = (uint8_t)code;
  }
}

// 128x128 fold from packed MXFP4 in one pass.  A workgroup of 4096 / R lanes
// (R = MXQ_PFOLD_ROWS) takes one 128-row band and four tile columns (512
// elements of each band row):
//  1. Lane t reads 8 block codes (two tiles' worth) of band row t / 2 into LDS
//     and keeps each tile's largest finite code; lanes of the same parity meet
//     by shuffles, the four waves in LDS.  M = that code (1, i.e. e = -126, if
//     the tile has none); tile code max(M - 6, 0), i.e. S = max(M - 6, -127).
//  2. Lane t converts 16 elements (8 packed bytes -> 16 payload bytes) of R
//     band rows, t / 32 + (128 / R) k, at the shift e - S of its block and
//     tile.  Poisoned blocks (code 255) get 0x7F.
// A whole band (all 128 rows and 512 columns in range, aligned storage) runs
// both parts as straight-line code: the code loads, then all R payload loads,
// then the code pass, so the payload is in flight through the code pass and
// the barrier (loads complete in order, and the code pass waits for the code
// loads alone).  Its rows are addressed from the band's base pointers with
// 32-bit lane offsets, so no load or store needs a guard.  An edge band (a
// partial band or column group) converts one row at a time, so that this rare
// path does not set the kernel's register count.
// Workgroup order for the fold from packed.  The hardware deals workgroups
// round-robin over the 8 XCDs (b runs on XCD b % 8), each with its own L2.
// Neighbouring workgroups of a band read neighbouring 16-byte pieces of the
// same 128-byte lines of block codes, so within every window of 64 workgroups
// XCD x takes work items 8x .. 8x+7: the eight that share those lines meet in
// one L2.  A transpose of each 8 x 8 window, so a bijection; a last partial
// window keeps the plain order.
__device__ __forceinline__ uint32_t xcd_window_order(uint32_t b, uint32_t n) {
  if (b >= (n & ~63u)) return b;
  return (b & ~63u) | ((b & 7u) << 3) | ((b >> 3) & 7u);
}

constexpr int kPFoldRG = 128 / kPFoldRows;                  // row groups of the band

struct PFoldLds {
  uint32_t codes[128][4];   // the band rows' 16 block codes
  uint32_t max[4][4];       // wave x tile
};

// Part 1 from lane t's 8 codes w (band row t / 2, half t % 2): the codes go to
// LDS and the four tile codes of the group come back (after a barrier).
__device__ __forceinline__ void pfold_tile_codes(const uint32_t w[2], uint32_t tid, PFoldLds& L, uint32_t tcode[4]) {
  const uint32_t lane = tid & 63u, wave = tid >> 6, rl = tid >> 1, h = tid & 1u;
  if (tid < 256u) {  // the first four waves
    L.codes[rl][2 * h] = w[0];
    L.codes[rl][2 * h + 1] = w[1];
    uint32_t m[2] = {1u, 1u};
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const uint32_t c = (w[t] >> (8 * k)) & 0xFFu;
        if (c != 255u) m[t] = max(m[t], c);
      }
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int off = 2; off < 64; off <<= 1) m[t] = max(m[t], (uint32_t)__shfl_xor((int)m[t], off));
    if (lane < 2u) L.max[wave][2 * lane] = m[0], L.max[wave][2 * lane + 1] = m[1];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const uint32_t M = max(max(L.max[0][t], L.max[1][t]), max(L.max[2][t], L.max[3][t]));
    tcode[t] = M > 6u ? M - 6u : 0u;
  }
}

// 16 payload bytes of one lane's 8 packed bytes f, block code c, tile code ts.
__device__ __forceinline__ u32x4 pfold_payload(u32x2 f, uint32_t c, uint32_t ts) {
  const int ds = min((int)c - (int)ts, 6);                   // e - S <= 6 (code 255: not used)
  const u32x2 lo = e4m3x8_of_fp4(f[0], ds), hi = e4m3x8_of_fp4(f[1], ds);
  return c == 255u ? u32x4{0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu} : u32x4{lo[0], lo[1], hi[0], hi[1]};
}

template <bool VEC>
__global__ __launch_bounds__(kPFoldThreads) void packed_fold_kernel(const uint8_t* __restrict__ packed,
                                                          const uint8_t* __restrict__ scale, int64_t scale_ld,
                                                          int64_t rows, int64_t K, uint8_t* __restrict__ data,
                                                          uint8_t* __restrict__ tile_code, int64_t tile_ld,
                                                          MxqDivisor groups, bool codes_vec) {
  __shared__ PFoldLds L;
  keep_denormals();
  const uint32_t tid = threadIdx.x;
  const uint32_t wb = xcd_window_order(blockIdx.x, gridDim.x);
  const uint32_t tr = mxq_quot(wb, groups), tg = wb - tr * groups.d;
  const int64_t r0 = (int64_t)tr * 128, nb = (K + 31) / 32, pw = (K + 1) / 2, ntc = (K + 127) / 128;
  const uint32_t rl = tid >> 1, h = tid & 1u;                // part 1: band row and half
  const uint32_t cc = tid & 31u, rg = tid >> 5;             // part 2: 16-element column chunk, row group
  const int64_t col0 = (int64_t)tg * 512 + cc * 16;
  const int64_t j = (int64_t)tg * 16 + 8 * h;               // first of the lane's 8 block codes
  uint32_t w[2] = {0xFFFFFFFFu, 0xFFFFFFFFu};                // 255: no finite code
  uint32_t tcode[4];

  if (VEC && codes_vec && r0 + 128 <= rows && (int64_t)tg * 512 + 512 <= K && K <= ((int64_t)1 << 27)) {
    // whole band (uniform branch)
    if (tid < 256u) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(scale + (r0 + rl) * scale_ld + j);
      w[0] = v[0], w[1] = v[1];
    }
    const uint8_t* pband = packed + r0 * pw;
    const uint32_t lp = rg * (uint32_t)pw + (uint32_t)(col0 / 2);
    u32x2 f[kPFoldRows];
#pragma unroll
    for (int k = 0; k < kPFoldRows; k++)
      f[k] = stream_load(reinterpret_cast<const u32x2*>(pband + (int64_t)(kPFoldRG * k) * pw + lp));
    pfold_tile_codes(w, tid, L, tcode);
    if (tid < 4u) tile_code[(int64_t)tr * tile_ld + tg * 4 + tid] = (uint8_t)tcode[tid & 3u];
    const uint32_t tt = cc >> 3, ts = tt == 0 ? tcode[0] : tt == 1 ? tcode[1] : tt == 2 ? tcode[2] : tcode[3];
    uint8_t* dband = data + r0 * K;
    const uint32_t ld = rg * (uint32_t)K + (uint32_t)col0;
#pragma unroll
    for (int k = 0; k < kPFoldRows; k++) {
      const uint32_t c = (L.codes[rg + kPFoldRG * k][cc >> 3] >> (8 * ((cc >> 1) & 3u))) & 0xFFu;
      stream_store(pfold_payload(f[k], c, ts), reinterpret_cast<u32x4*>(dband + (int64_t)(kPFoldRG * k) * K + ld));
    }
    return;
  }

  // edge band
  if (tid < 256u && r0 + rl < rows) {
    const uint8_t* src = scale + (r0 + rl) * scale_ld + j;
    if (codes_vec && j + 8 <= nb) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(src);
      w[0] = v[0], w[1] = v[1];
    } else {
      for (int k = 0; k < 8; k++)
        if (j + k < nb) w[k / 4] = (w[k / 4] & ~(0xFFu << (8 * (k % 4)))) | ((uint32_t)src[k] << (8 * (k % 4)));
    }
  }
  pfold_tile_codes(w, tid, L, tcode);
  if (tid < 4u && (int64_t)tg * 4 + tid < ntc) tile_code[(int64_t)tr * tile_ld + tg * 4 + tid] = (uint8_t)tcode[tid & 3u];
  const uint32_t tt = cc >> 3, ts = tt == 0 ? tcode[0] : tt == 1 ? tcode[1] : tt == 2 ? tcode[2] : tcode[3];
#pragma unroll 1
  for (int k = 0; k < kPFoldRows; k++) {
    const int64_t r = r0 + rg + kPFoldRG * k;
    if (r >= rows || col0 >= K) continue;
    const uint8_t* prow = packed + r * pw;
    u32x2 f = {0u, 0u};
    if (VEC) {
      f = stream_load(reinterpret_cast<const u32x2*>(prow + col0 / 2));
    } else {
      for (int i = 0; i < 16; i += 2)
        if (col0 + i < K) f[i / 8] |= (uint32_t)prow[(col0 + i) / 2] << (4 * (i % 8));
    }
    const uint32_t c = (L.codes[rg + kPFoldRG * k][cc >> 3] >> (8 * ((cc >> 1) & 3u))) & 0xFFu;
    const u32x4 q = pfold_payload(f, c, ts);
    uint8_t* drow = data + r * K;
    if (VEC) {
      stream_store(q, reinterpret_cast<u32x4*>(drow + col0));
    } else {
      for (int i = 0; i < 16; i++)
        if (col0 + i < K) drow[col0 + i] = (uint8_t)(q[i / 4] >> (8 * (i % 4)));
    }
  }
}

// ------------------------------------------------------------------------------------
// Export: strided copy of the first ncols columns of each row, in units of V
// (16, 4 or 1 bytes, whichever the pointers, strides and width allow).  Rows
// are flattened (one unit per lane), so short rows still fill whole waves.
// Workgroup order: the dispatcher deals workgroup b to XCD b % 8, each XCD
// with its own L2, and a padded storage row is not a whole number of 128-byte
// lines, so neighbouring workgroups share the lines at their boundary.  Chunk c
// of the grid (rounded up to a multiple of 8) goes to workgroup
// (c % per) * 8 + c / per with per = grid / 8: XCD x copies the contiguous
// chunks x * per .. x * per + per - 1, and only the 7 lines between those runs
// are fetched by two L2s.
// ------------------------------------------------------------------------------------
template <typename V>
__global__ __launch_bounds__(kThreads) void export_kernel(const uint8_t* __restrict__ src, int64_t src_ld,
                                                          uint8_t* __restrict__ dst, MxqDivisor units_per_row,
                                                          uint32_t total_units) {
  const uint32_t per = gridDim.x / 8, chunk = (blockIdx.x % 8) * per + blockIdx.x / 8;
  const uint64_t i64 = (uint64_t)chunk * kThreads + threadIdx.x;   // the last chunk may pass 2^32
  if (i64 >= total_units) return;
  const uint32_t i = (uint32_t)i64;
  const uint32_t r = mxq_quot(i, units_per_row), j = i - r * units_per_row.d;
  reinterpret_cast<V*>(dst)[i] = reinterpret_cast<const V*>(src + (int64_t)r * src_ld)[j];
}

// The export of 4-byte-aligned source rows into 16-byte-aligned destination
// rows (a padded stride such as ceil(K/32) + 4): each lane loads four
// consecutive 4-byte units of one row and stores them as one 16-byte unit.
// units_per_row and total_units count 16-byte destination units.
__global__ __launch_bounds__(kThreads) void export4_kernel(const uint8_t* __restrict__ src, int64_t src_ld,
                                                           uint8_t* __restrict__ dst, MxqDivisor units_per_row,
                                                           uint32_t total_units) {
  const uint32_t per = gridDim.x / 8, chunk = (blockIdx.x % 8) * per + blockIdx.x / 8;
  const uint64_t i64 = (uint64_t)chunk * kThreads + threadIdx.x;
  if (i64 >= total_units) return;
  const uint32_t i = (uint32_t)i64;
  const uint32_t r = mxq_quot(i, units_per_row), j = i - r * units_per_row.d;
  const uint32_t* s = reinterpret_cast<const uint32_t*>(src + (int64_t)r * src_ld) + 4 * j;
  reinterpret_cast<u32x4*>(dst)[i] = u32x4{s[0], s[1], s[2], s[3]};
}

// ------------------------------------------------------------------------------------
// Host side: validation and launch
// ------------------------------------------------------------------------------------
constexpr int64_t kMaxSteps = (int64_t)1 << 31;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
// The projection's vectorised stores address a row with 32-bit byte offsets;
// longer rows take the element-wise path.
bool fits32(int64_t bytes) { return bytes < ((int64_t)1 << 31); }

// Byte range [lo, hi) of a [rows, cols] matrix (rows, cols >= 1) with row
// stride ld elements of esize bytes.  ok is false when that span cannot be a
// real allocation -- 2^56 bytes or more, or running past the end of the address
// space -- so that no later size arithmetic can overflow; the entry points
// reject such shapes with MXQ_ERR_SHAPE before any other use of the range.
struct Range {
  uintptr_t lo, hi;
  bool ok;
};
Range matrix_range(const void* p, int64_t rows, int64_t cols, int64_t ld, size_t esize) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  const __int128 span = ((__int128)(rows - 1) * ld + cols) * (__int128)esize;
  const bool ok = span > 0 && span < ((__int128)1 << 56) && (unsigned __int128)lo + span <= UINTPTR_MAX;
  return Range{lo, ok ? lo + (uintptr_t)span : lo, ok};
}
bool spans_ok(std::initializer_list<Range> rs) {
  for (const Range& r : rs)
    if (!r.ok) return false;
  return true;
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int launch_status() {
  return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

int steps_for(int64_t rows, int64_t K, int64_t elems_per_step, MxqDivisor* per_row, uint32_t* total) {
  const int64_t spr = (K + elems_per_step - 1) / elems_per_step;
  if (rows > kMaxSteps / spr) return MXQ_ERR_SHAPE;
  *per_row = mxq_divisor((uint32_t)spr);
  *total = (uint32_t)(rows * spr);
  return MXQ_OK;
}

uint32_t grid_for(uint32_t total_steps, int per_wg) { return (total_steps + per_wg - 1) / per_wg; }

int check_dtype(mxq_dtype dt) {
  return (dt == MXQ_BF16 || dt == MXQ_FP32) ? MXQ_OK : MXQ_ERR_DTYPE;
}
size_t dtype_size(mxq_dtype dt) { return dt == MXQ_BF16 ? 2 : 4; }

template <typename T>
int launch_proj(const void* x, int64_t ld_x, void* y, int64_t ld_y, int64_t rows, int64_t K, hipStream_t s) {
  MxqDivisor spr;
  uint32_t total;
  if (steps_for(rows, K, StepGeom<T, kProjThreads>::kElemsPerStep, &spr, &total)) return MXQ_ERR_SHAPE;
  constexpr int EPL = Fmt<T>::kEPL;
  const bool vec = aligned(x, 16) && aligned(y, 16) && ld_x % EPL == 0 && ld_y % EPL == 0 && K % EPL == 0 &&
                   fits32(K * (int64_t)sizeof(T));
  const dim3 grid(grid_for(total, kProjSteps)), block(kProjThreads);
  if (vec)
    hipLaunchKernelGGL((proj_kernel<T, true>), grid, block, 0, s, (const T*)x, ld_x, (T*)y, ld_y, K, spr, total);
  else
    hipLaunchKernelGGL((proj_kernel<T, false>), grid, block, 0, s, (const T*)x, ld_x, (T*)y, ld_y, K, spr, total);
  return launch_status();
}

template <typename T>
int launch_row(const void* x, int64_t ld_x, int64_t rows, int64_t K, uint8_t* data, uint8_t* scale,
               int64_t scale_ld, void* y, int64_t ld_y, const int32_t* noop, hipStream_t s) {
  const bool fused = y != nullptr;
  const int tpb = fused ? kFusedThreads : kRowThreads, steps = fused ? kFusedSteps : kRowSteps;
  MxqDivisor spr;
  uint32_t total;
  if (steps_for(rows, K, (int64_t)(tpb / Fmt<T>::kLPB) * 32, &spr, &total)) return MXQ_ERR_SHAPE;
  constexpr int EPL = Fmt<T>::kEPL;
  const bool vec = aligned(x, 16) && ld_x % EPL == 0 && K % EPL == 0 && aligned(data, EPL) &&
                   (!fused || (aligned(y, 16) && ld_y % EPL == 0 && fits32(K * (int64_t)sizeof(T))));
  // every step whole and every workgroup's steps inside the grid: no bounds checks
  // (and, for the gathered code stores, scale rows aligned to their width: 16 / kLPB bytes)
  const int code_width = MXQ_ROW_CODE_WORDS && !fused ? CodeGather<Fmt<T>::kLPB>::kCodes : 1;
  const bool full = vec && spr.d * (int64_t)((tpb / Fmt<T>::kLPB) * 32) == K && total % steps == 0 &&
                    fits32(K * (int64_t)sizeof(T)) && aligned(scale, code_width) && scale_ld % code_width == 0;
  const dim3 grid(grid_for(total, steps)), block(tpb);
#define MXQ_ROW_LAUNCH(V, P, F)                                                                                  \
  hipLaunchKernelGGL((row_kernel<T, V, P, F>), grid, block, 0, s, (const T*)x, ld_x, K, data, scale, scale_ld, \
                     (T*)y, ld_y, spr, total, noop)
  if (fused) {
    if (full) MXQ_ROW_LAUNCH(true, true, true); else if (vec) MXQ_ROW_LAUNCH(true, true, false);
    else MXQ_ROW_LAUNCH(false, true, false);
  } else {
    if (full) MXQ_ROW_LAUNCH(true, false, true); else if (vec) MXQ_ROW_LAUNCH(true, false, false);
    else MXQ_ROW_LAUNCH(false, false, false);
  }
#undef MXQ_ROW_LAUNCH
  return launch_status();
}

template <typename T>
int launch_col(const void* x, int64_t ld_x, int64_t rows, int64_t K, uint8_t* cdata, uint8_t* cscale,
               int64_t cscale_ld, uint8_t* rdata, uint8_t* rscale, int64_t rscale_ld, const int32_t* noop,
               hipStream_t s) {
  constexpr int64_t kCols = (int64_t)kColThreads * Fmt<T>::kEPL;   // columns per workgroup
  const int64_t groups = (K + kCols - 1) / kCols, bands = (rows + 31) / 32;
  if (bands > kMaxSteps / groups) return MXQ_ERR_SHAPE;
  constexpr int EPL = Fmt<T>::kEPL;
  const bool vec = aligned(x, 16) && ld_x % EPL == 0 && K % EPL == 0 && aligned(cdata, EPL) &&
                   (rdata == nullptr || aligned(rdata, EPL));
  const dim3 grid((uint32_t)(bands * groups)), block(kColThreads * kColGroups);
#define MXQ_COL_LAUNCH(V, R)                                                                                    \
  hipLaunchKernelGGL((col_kernel<T, V, R>), grid, block, 0, s, (const T*)x, ld_x, rows, K, cdata, cscale, cscale_ld, \
                     rdata, rscale, rscale_ld, mxq_divisor((uint32_t)groups), noop)
  if (rdata != nullptr) {
    if (vec) MXQ_COL_LAUNCH(true, true); else MXQ_COL_LAUNCH(false, true);
  } else {
    if (vec) MXQ_COL_LAUNCH(true, false); else MXQ_COL_LAUNCH(false, false);
  }
#undef MXQ_COL_LAUNCH
  return launch_status();
}

template <typename T>
int launch_block128(const void* x, int64_t ld_x, int64_t rows, int64_t K, uint8_t* data, uint8_t* tile_code,
                    int64_t tile_ld, const int32_t* noop, hipStream_t s) {
  constexpr int J = FoldGeom<T>::kJ;
  const int64_t tpr = (K + 127) / 128, gpr = (tpr + J - 1) / J, groups = gpr * ((rows + 127) / 128);
  if (groups >= kMaxSteps) return MXQ_ERR_SHAPE;
  constexpr int EPL = Fmt<T>::kEPL;
  const bool vec = aligned(x, 16) && ld_x % EPL == 0 && K % EPL == 0 && aligned(data, EPL);
  const dim3 grid((uint32_t)groups), block(FoldGeom<T>::kThreads);
  if constexpr (sizeof(T) == 4 && MXQ_FOLD_FULL) {
    if (vec && rows % 128 == 0 && K % (128 * J) == 0 && fits32(128 * K)) {
      hipLaunchKernelGGL((block128_kernel<T, true, true>), grid, block, 0, s, (const T*)x, ld_x, rows, K, data,
                         tile_code, tile_ld, (uint32_t)tpr, mxq_divisor((uint32_t)gpr), noop);
      return launch_status();
    }
  }
  if (vec)
    hipLaunchKernelGGL((block128_kernel<T, true, false>), grid, block, 0, s, (const T*)x, ld_x, rows, K, data,
                       tile_code, tile_ld, (uint32_t)tpr, mxq_divisor((uint32_t)gpr), noop);
  else
    hipLaunchKernelGGL((block128_kernel<T, false, false>), grid, block, 0, s, (const T*)x, ld_x, rows, K, data,
                       tile_code, tile_ld, (uint32_t)tpr, mxq_divisor((uint32_t)gpr), noop);
  return launch_status();
}

template <typename TO, bool kE5M2, int kLay>
int launch_dequant_t(const uint8_t* data, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K, void* out,
                     int64_t ld_out, hipStream_t s) {
  MxqDivisor spr;
  uint32_t total;
  if (steps_for(rows, K, DequantShape<TO>::kThreads * 8, &spr, &total)) return MXQ_ERR_SHAPE;
  constexpr int OPC = 16 / (int)sizeof(TO);   // output elements per 16-byte store
  const bool vec = aligned(data, 8) && K % 8 == 0 && aligned(out, 16) && ld_out % OPC == 0 &&
                   (kLay != kLayCol || (aligned(scale, 8) && scale_ld % 8 == 0));
  const dim3 grid(grid_for(total, DequantShape<TO>::kSteps)), block(DequantShape<TO>::kThreads);
  if (vec)
    hipLaunchKernelGGL((dequant_kernel<TO, kE5M2, kLay, true>), grid, block, 0, s, data, scale, scale_ld, K,
                       (TO*)out, ld_out, spr, total);
  else
    hipLaunchKernelGGL((dequant_kernel<TO, kE5M2, kLay, false>), grid, block, 0, s, data, scale, scale_ld, K,
                       (TO*)out, ld_out, spr, total);
  return launch_status();
}

template <typename TO, bool kE5M2>
int launch_dequant_f(const uint8_t* data, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K,
                     mxq_scale_layout lay, void* out, int64_t ld_out, hipStream_t s) {
  if (lay == MXQ_SCALE_TILE_128X128)
    return launch_dequant_t<TO, kE5M2, kLayTile>(data, scale, scale_ld, rows, K, out, ld_out, s);
  if (lay == MXQ_SCALE_COL_32X1)
    return launch_dequant_t<TO, kE5M2, kLayCol>(data, scale, scale_ld, rows, K, out, ld_out, s);
  return launch_dequant_t<TO, kE5M2, kLayRow>(data, scale, scale_ld, rows, K, out, ld_out, s);
}

template <typename TO>
int launch_dequant(const uint8_t* data, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K,
                   mxq_fp8 fmt, mxq_scale_layout lay, void* out, int64_t ld_out, hipStream_t s) {
  return fmt == MXQ_E5M2 ? launch_dequant_f<TO, true>(data, scale, scale_ld, rows, K, lay, out, ld_out, s)
                         : launch_dequant_f<TO, false>(data, scale, scale_ld, rows, K, lay, out, ld_out, s);
}

template <typename T>
int launch_quantize_mxfp4(const void* x, int64_t ld_x, int64_t rows, int64_t K, uint8_t* packed, uint8_t* scale,
                          int64_t scale_ld, hipStream_t s) {
  MxqDivisor spr;
  uint32_t total;
  if (steps_for(rows, K, StepGeom<T, kQ4Threads>::kElemsPerStep, &spr, &total)) return MXQ_ERR_SHAPE;
  constexpr int EPL = Fmt<T>::kEPL;
  const bool vec = aligned(x, 16) && ld_x % EPL == 0 && K % EPL == 0 && aligned(packed, EPL / 2);
  // every step whole and every workgroup's steps inside the grid: no bounds checks
  // (and, for the gathered code stores, code rows aligned to their width)
  const int code_width = MXQ_Q4_CODE_WORDS ? CodeGather<Fmt<T>::kLPB>::kCodes : 1;
  const bool full = vec && spr.d * (int64_t)StepGeom<T, kQ4Threads>::kElemsPerStep == K && total % kQ4Steps == 0 &&
                    fits32(K * (int64_t)sizeof(T)) && aligned(scale, code_width) && scale_ld % code_width == 0;
  const dim3 grid(grid_for(total, kQ4Steps)), block(kQ4Threads);
  if (full)
    hipLaunchKernelGGL((quantize_mxfp4_kernel<T, true, true>), grid, block, 0, s, (const T*)x, ld_x, K, packed, scale,
                       scale_ld, spr, total);
  else if (vec)
    hipLaunchKernelGGL((quantize_mxfp4_kernel<T, true, false>), grid, block, 0, s, (const T*)x, ld_x, K, packed, scale,
                       scale_ld, spr, total);
  else
    hipLaunchKernelGGL((quantize_mxfp4_kernel<T, false, false>), grid, block, 0, s, (const T*)x, ld_x, K, packed, scale,
                       scale_ld, spr, total);
  return launch_status();
}

template <typename TO>
int launch_dequantize_mxfp4(const uint8_t* packed, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K,
                            void* out, int64_t ld_out, hipStream_t s) {
  MxqDivisor spr;
  uint32_t total;
  if (steps_for(rows, K, kDq4Threads * 8, &spr, &total)) return MXQ_ERR_SHAPE;
  constexpr int OPC = 16 / (int)sizeof(TO);
  const bool vec = aligned(packed, 4) && K % 8 == 0 && aligned(out, 16) && ld_out % OPC == 0;
  const dim3 grid(grid_for(total, kDq4Steps)), block(kDq4Threads);
  if (vec)
    hipLaunchKernelGGL((dequantize_mxfp4_kernel<TO, true>), grid, block, 0, s, packed, scale, scale_ld, K, (TO*)out,
                       ld_out, spr, total);
  else
    hipLaunchKernelGGL((dequantize_mxfp4_kernel<TO, false>), grid, block, 0, s, packed, scale, scale_ld, K, (TO*)out,
                       ld_out, spr, total);
  return launch_status();
}

// Grouped row lift: aligned weights go into tables of up to kGroupMax, one
// launch per table; the others take the single-weight launch.  A table is cut
// early when a weight's size would pad its grid (weights x the largest
// workgroup count) by more than a quarter of the real workgroups plus 4096
// (workgroups that exit at once).  The caller has checked every group
// (shapes, spans, step counts, aliasing) beforehand.
template <typename T>
int launch_row_grouped(const mxq_row_group* gs, int64_t n, hipStream_t s) {
  constexpr int EPL = Fmt<T>::kEPL;
  RowGroupTable tab{};
  int64_t count = 0, max_w = 0, sum_w = 0;
  auto flush = [&]() -> int {
    if (count == 0) return MXQ_OK;
    hipLaunchKernelGGL((row_grouped_kernel<T>), dim3((uint32_t)max_w, (uint32_t)count), dim3(kRowGroupedThreads), 0, s,
                       tab);
    count = max_w = sum_w = 0;
    return launch_status();
  };
  for (int64_t i = 0; i < n; i++) {
    const mxq_row_group& g = gs[i];
    if (g.rows == 0 || g.K == 0) continue;
    if (!(aligned(g.x, 16) && g.ld_x % EPL == 0 && g.K % EPL == 0 && aligned(g.data, EPL))) {
      const int st = launch_row<T>(g.x, g.ld_x, g.rows, g.K, g.data, g.scale, g.scale_ld, nullptr, 0, nullptr, s);
      if (st != MXQ_OK) return st;
      continue;
    }
    MxqDivisor spr;
    uint32_t total;
    if (steps_for(g.rows, g.K, StepGeom<T, kRowGroupedThreads>::kElemsPerStep, &spr, &total)) return MXQ_ERR_SHAPE;
    const int64_t gw = grid_for(total, kRowGroupedSteps);
    const int64_t padded = (count + 1) * std::max(max_w, gw), real = sum_w + gw;
    if (count == kGroupMax || (count > 0 && padded > real + real / 4 + 4096)) {
      const int st = flush();
      if (st != MXQ_OK) return st;
    }
    tab.g[count] = RowGroupDesc{g.x, g.ld_x, g.K, g.data, g.scale, g.scale_ld, spr, total};
    count++;
    max_w = std::max(max_w, gw);
    sum_w += gw;
  }
  return flush();
}

// Grouped projection: the grouped row lift's batching, for the projection.
template <typename T>
int launch_proj_grouped(const mxq_proj_group* gs, int64_t n, hipStream_t s) {
  constexpr int EPL = Fmt<T>::kEPL;
  ProjGroupTable tab{};
  int64_t count = 0, max_w = 0, sum_w = 0;
  auto flush = [&]() -> int {
    if (count == 0) return MXQ_OK;
    hipLaunchKernelGGL((proj_grouped_kernel<T>), dim3((uint32_t)max_w, (uint32_t)count), dim3(kProjThreads), 0, s,
                       tab);
    count = max_w = sum_w = 0;
    return launch_status();
  };
  for (int64_t i = 0; i < n; i++) {
    const mxq_proj_group& g = gs[i];
    if (g.rows == 0 || g.K == 0) continue;
    if (!(aligned(g.x, 16) && aligned(g.y, 16) && g.ld_x % EPL == 0 && g.ld_y % EPL == 0 && g.K % EPL == 0 &&
          fits32(g.K * (int64_t)sizeof(T)))) {
      const int st = launch_proj<T>(g.x, g.ld_x, g.y, g.ld_y, g.rows, g.K, s);
      if (st != MXQ_OK) return st;
      continue;
    }
    MxqDivisor spr;
    uint32_t total;
    if (steps_for(g.rows, g.K, StepGeom<T, kProjThreads>::kElemsPerStep, &spr, &total)) return MXQ_ERR_SHAPE;
    const int64_t gw = grid_for(total, kProjSteps);
    const int64_t padded = (count + 1) * std::max(max_w, gw), real = sum_w + gw;
    if (count == kGroupMax || (count > 0 && padded > real + real / 4 + 4096)) {
      const int st = flush();
      if (st != MXQ_OK) return st;
    }
    tab.g[count] = ProjGroupDesc{g.x, g.ld_x, g.K, g.y, g.ld_y, spr, total};
    count++;
    max_w = std::max(max_w, gw);
    sum_w += gw;
  }
  return flush();
}

// Grouped fold: the grouped row lift's batching, for the fold (one workgroup
// per group of J tiles, as the single launch).
template <typename T>
int launch_block128_grouped(const mxq_block128_group* gs, int64_t n, hipStream_t s) {
  constexpr int EPL = Fmt<T>::kEPL, J = FoldGeom<T>::kJ;
  FoldGroupTable tab{};
  int64_t count = 0, max_w = 0, sum_w = 0;
  auto flush = [&]() -> int {
    if (count == 0) return MXQ_OK;
    hipLaunchKernelGGL((block128_grouped_kernel<T>), dim3((uint32_t)max_w, (uint32_t)count),
                       dim3(FoldGeom<T>::kThreads), 0, s, tab);
    count = max_w = sum_w = 0;
    return launch_status();
  };
  for (int64_t i = 0; i < n; i++) {
    const mxq_block128_group& g = gs[i];
    if (g.rows == 0 || g.K == 0) continue;
    if (!(aligned(g.x, 16) && g.ld_x % EPL == 0 && g.K % EPL == 0 && aligned(g.data, EPL))) {
      const int st = launch_block128<T>(g.x, g.ld_x, g.rows, g.K, g.data, g.tile_code, g.tile_ld, nullptr, s);
      if (st != MXQ_OK) return st;
      continue;
    }
    const int64_t tpr = (g.K + 127) / 128, gpr = (tpr + J - 1) / J, gw = gpr * ((g.rows + 127) / 128);
    if (gw >= kMaxSteps) return MXQ_ERR_SHAPE;
    const int64_t padded = (count + 1) * std::max(max_w, gw), real = sum_w + gw;
    if (count == kGroupMax || (count > 0 && padded > real + real / 4 + 4096)) {
      const int st = flush();
      if (st != MXQ_OK) return st;
    }
    tab.g[count] = FoldGroupDesc{g.x,         g.ld_x,     g.rows, g.K, g.data, g.tile_code, g.tile_ld,
                                 mxq_divisor((uint32_t)gpr), (uint32_t)tpr, (uint32_t)gw};
    count++;
    max_w = std::max(max_w, gw);
    sum_w += gw;
  }
  return flush();
}

// Grouped decode: the grouped row lift's batching, for the decode of one
// payload format, scale layout and output dtype.
template <typename TO, bool kE5M2, int kLay>
int launch_dequant_grouped_t(const mxq_dequant_group* gs, int64_t n, hipStream_t s) {
  constexpr int OPC = 16 / (int)sizeof(TO);
  DequantGroupTable tab{};
  int64_t count = 0, max_w = 0, sum_w = 0;
  auto flush = [&]() -> int {
    if (count == 0) return MXQ_OK;
    hipLaunchKernelGGL((dequant_grouped_kernel<TO, kE5M2, kLay>), dim3((uint32_t)max_w, (uint32_t)count),
                       dim3(DequantShape<TO>::kThreads), 0, s, tab);
    count = max_w = sum_w = 0;
    return launch_status();
  };
  for (int64_t i = 0; i < n; i++) {
    const mxq_dequant_group& g = gs[i];
    if (g.rows == 0 || g.K == 0) continue;
    if (!(aligned(g.data, 8) && g.K % 8 == 0 && aligned(g.out, 16) && g.ld_out % OPC == 0 &&
          (kLay != kLayCol || (aligned(g.scale, 8) && g.scale_ld % 8 == 0)))) {
      const int st = launch_dequant_t<TO, kE5M2, kLay>(g.data, g.scale, g.scale_ld, g.rows, g.K, g.out, g.ld_out, s);
      if (st != MXQ_OK) return st;
      continue;
    }
    MxqDivisor spr;
    uint32_t total;
    if (steps_for(g.rows, g.K, DequantShape<TO>::kThreads * 8, &spr, &total)) return MXQ_ERR_SHAPE;
    const int64_t gw = grid_for(total, kDequantGroupedSteps);
    const int64_t padded = (count + 1) * std::max(max_w, gw), real = sum_w + gw;
    if (count == kGroupMax || (count > 0 && padded > real + real / 4 + 4096)) {
      const int st = flush();
      if (st != MXQ_OK) return st;
    }
    tab.g[count] = DequantGroupDesc{g.data, g.scale, g.scale_ld, g.K, g.out, g.ld_out, spr, total};
    count++;
    max_w = std::max(max_w, gw);
    sum_w += gw;
  }
  return flush();
}

template <typename TO, bool kE5M2>
int launch_dequant_grouped_f(const mxq_dequant_group* gs, int64_t n, mxq_scale_layout lay, hipStream_t s) {
  if (lay == MXQ_SCALE_TILE_128X128) return launch_dequant_grouped_t<TO, kE5M2, kLayTile>(gs, n, s);
  if (lay == MXQ_SCALE_COL_32X1) return launch_dequant_grouped_t<TO, kE5M2, kLayCol>(gs, n, s);
  return launch_dequant_grouped_t<TO, kE5M2, kLayRow>(gs, n, s);
}

template <typename TO>
int launch_dequant_grouped(const mxq_dequant_group* gs, int64_t n, mxq_fp8 fmt, mxq_scale_layout lay,
                           hipStream_t s) {
  return fmt == MXQ_E5M2 ? launch_dequant_grouped_f<TO, true>(gs, n, lay, s)
                         : launch_dequant_grouped_f<TO, false>(gs, n, lay, s);
}

// Grouped packed encode: the grouped row lift's batching, for the encode.
template <typename T>
int launch_quantize_mxfp4_grouped(const mxq_mxfp4_group* gs, int64_t n, hipStream_t s) {
  constexpr int EPL = Fmt<T>::kEPL;
  RowGroupTable tab{};
  int64_t count = 0, max_w = 0, sum_w = 0;
  auto flush = [&]() -> int {
    if (count == 0) return MXQ_OK;
    hipLaunchKernelGGL((quantize_mxfp4_grouped_kernel<T>), dim3((uint32_t)max_w, (uint32_t)count),
                       dim3(kQ4Threads), 0, s, tab);
    count = max_w = sum_w = 0;
    return launch_status();
  };
  for (int64_t i = 0; i < n; i++) {
    const mxq_mxfp4_group& g = gs[i];
    if (g.rows == 0 || g.K == 0) continue;
    if (!(aligned(g.x, 16) && g.ld_x % EPL == 0 && g.K % EPL == 0 && aligned(g.packed, EPL / 2))) {
      const int st = launch_quantize_mxfp4<T>(g.x, g.ld_x, g.rows, g.K, g.packed, g.scale, g.scale_ld, s);
      if (st != MXQ_OK) return st;
      continue;
    }
    MxqDivisor spr;
    uint32_t total;
    if (steps_for(g.rows, g.K, StepGeom<T, kQ4Threads>::kElemsPerStep, &spr, &total)) return MXQ_ERR_SHAPE;
    const int64_t gw = grid_for(total, kQ4Steps);
    const int64_t padded = (count + 1) * std::max(max_w, gw), real = sum_w + gw;
    if (count == kGroupMax || (count > 0 && padded > real + real / 4 + 4096)) {
      const int st = flush();
      if (st != MXQ_OK) return st;
    }
    tab.g[count] = RowGroupDesc{g.x, g.ld_x, g.K, g.packed, g.scale, g.scale_ld, spr, total};
    count++;
    max_w = std::max(max_w, gw);
    sum_w += gw;
  }
  return flush();
}

// The ranges of a grouped call, each marked as an output or not: true when no
// output overlaps any other range.  A sweep in order of start address: a range
// overlaps an earlier one exactly when it starts before the largest end seen
// so far (of outputs, for an input; of anything, for an output).
bool grouped_ranges_disjoint(std::vector<std::pair<Range, bool>>& iv) {
  std::sort(iv.begin(), iv.end(), [](const std::pair<Range, bool>& a, const std::pair<Range, bool>& b) {
    return a.first.lo < b.first.lo;
  });
  uintptr_t end_out = 0, end_in = 0;
  for (const auto& e : iv) {
    const Range& r = e.first;
    if (e.second ? r.lo < std::max(end_out, end_in) : r.lo < end_out) return false;
    uintptr_t& end = e.second ? end_out : end_in;
    end = std::max(end, r.hi);
  }
  return true;
}

}  // namespace

extern "C" {

const char* mxq_status_string(int status) {
  switch (status) {
    case MXQ_OK: return "ok";
    case MXQ_ERR_NULL: return "a required pointer is NULL";
    case MXQ_ERR_SHAPE: return "invalid shape or stride";
    case MXQ_ERR_DTYPE: return "unsupported dtype, format or layout (fp16 is rejected)";
    case MXQ_ERR_NO_ROWWISE_DATA: return "no row-scaled data to export";
    case MXQ_ERR_ALIAS: return "an output overlaps an input";
    case MXQ_ERR_HIP: return "the HIP runtime refused a launch";
    default: return "unknown status";
  }
}

// Argument checks of the projection.  For a non-empty matrix it returns MXQ_OK
// with *rx / *ry and whether the call is in place; for an empty one MXQ_OK with
// *empty set.
static int proj_check(const void* x, int64_t ld_x, const void* y, int64_t ld_y, int64_t rows, int64_t K,
                      mxq_dtype dt, Range* rx, Range* ry, bool* in_place, bool* empty) {
  *empty = false;
  if (check_dtype(dt)) return MXQ_ERR_DTYPE;
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (rows == 0 || K == 0) {
    *empty = true;
    return MXQ_OK;
  }
  if (!x || !y) return MXQ_ERR_NULL;
  if (ld_x < K || ld_y < K) return MXQ_ERR_SHAPE;
  const size_t es = dtype_size(dt);
  *in_place = (x == y) && (ld_x == ld_y);
  *rx = matrix_range(x, rows, K, ld_x, es);
  *ry = matrix_range(y, rows, K, ld_y, es);
  if (!spans_ok({*rx, *ry})) return MXQ_ERR_SHAPE;
  if (!*in_place && overlap(*rx, *ry)) return MXQ_ERR_ALIAS;
  return MXQ_OK;
}

int mxq_fake_quantize_mxfp4(const void* x, int64_t ld_x, void* y, int64_t ld_y, int64_t rows, int64_t K,
                            mxq_dtype dt, hipStream_t stream) {
  Range rx, ry;
  bool in_place, empty;
  const int st = proj_check(x, ld_x, y, ld_y, rows, K, dt, &rx, &ry, &in_place, &empty);
  if (st != MXQ_OK || empty) return st;
  return dt == MXQ_BF16 ? launch_proj<uint16_t>(x, ld_x, y, ld_y, rows, K, stream)
                        : launch_proj<uint32_t>(x, ld_x, y, ld_y, rows, K, stream);
}

int mxq_fake_quantize_mxfp4_grouped(const mxq_proj_group* groups, int64_t n_groups, mxq_dtype dt,
                                    hipStream_t stream) {
  if (check_dtype(dt)) return MXQ_ERR_DTYPE;
  if (n_groups < 0) return MXQ_ERR_SHAPE;
  if (n_groups == 0) return MXQ_OK;
  if (!groups) return MXQ_ERR_NULL;
  const int64_t eps = dt == MXQ_BF16 ? StepGeom<uint16_t, kProjThreads>::kElemsPerStep
                                     : StepGeom<uint32_t, kProjThreads>::kElemsPerStep;
  std::vector<std::pair<Range, bool>> iv;                   // (range, is an output)
  iv.reserve((size_t)std::min<int64_t>(n_groups, 1 << 20) * 2);
  for (int64_t i = 0; i < n_groups; i++) {
    const mxq_proj_group& g = groups[i];
    Range rx, ry;
    bool in_place, empty;
    const int st = proj_check(g.x, g.ld_x, g.y, g.ld_y, g.rows, g.K, dt, &rx, &ry, &in_place, &empty);
    if (st != MXQ_OK) return st;
    if (empty) continue;
    MxqDivisor spr;
    uint32_t total;
    if (steps_for(g.rows, g.K, eps, &spr, &total)) return MXQ_ERR_SHAPE;
    if (!in_place) iv.push_back({rx, false});               // in place: the range is an output only
    iv.push_back({ry, true});
  }
  if (!grouped_ranges_disjoint(iv)) return MXQ_ERR_ALIAS;
  return dt == MXQ_BF16 ? launch_proj_grouped<uint16_t>(groups, n_groups, stream)
                        : launch_proj_grouped<uint32_t>(groups, n_groups, stream);
}

// Argument checks of the row lift (and its fused and gated forms).  For a
// non-empty matrix it returns MXQ_OK with *ranges = {x, data, scale}; for an
// empty one MXQ_OK with *empty set.
static int row_check(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt, uint8_t* data,
                     uint8_t* scale, int64_t scale_ld, void* y, int64_t ld_y, bool need_y, const int32_t* noop,
                     bool need_noop, Range* ranges, bool* empty) {
  *empty = false;
  if (check_dtype(dt)) return MXQ_ERR_DTYPE;
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (rows == 0 || K == 0) {
    *empty = true;
    return MXQ_OK;
  }
  if (!x || !data || !scale || (need_noop && !noop) || (need_y && !y)) return MXQ_ERR_NULL;
  const int64_t nb = (K + 31) / 32;
  if (ld_x < K || scale_ld < nb || (y && ld_y < K)) return MXQ_ERR_SHAPE;
  const size_t es = dtype_size(dt);
  const Range rx = matrix_range(x, rows, K, ld_x, es), rd = matrix_range(data, rows, K, K, 1),
              rs = matrix_range(scale, rows, nb, scale_ld, 1);
  if (!spans_ok({rx, rd, rs})) return MXQ_ERR_SHAPE;
  if (overlap(rx, rd) || overlap(rx, rs) || overlap(rd, rs)) return MXQ_ERR_ALIAS;
  if (y) {
    const Range ry = matrix_range(y, rows, K, ld_y, es);
    if (!ry.ok) return MXQ_ERR_SHAPE;
    const bool in_place = (x == y) && (ld_x == ld_y);
    if ((!in_place && overlap(rx, ry)) || overlap(ry, rd) || overlap(ry, rs)) return MXQ_ERR_ALIAS;
  }
  ranges[0] = rx, ranges[1] = rd, ranges[2] = rs;
  return MXQ_OK;
}

static int row_entry(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt, uint8_t* data,
                     uint8_t* scale, int64_t scale_ld, void* y, int64_t ld_y, bool need_y, const int32_t* noop,
                     bool need_noop, hipStream_t stream) {
  Range r[3];
  bool empty;
  const int st = row_check(x, ld_x, rows, K, dt, data, scale, scale_ld, y, ld_y, need_y, noop, need_noop, r, &empty);
  if (st != MXQ_OK || empty) return st;
  return dt == MXQ_BF16 ? launch_row<uint16_t>(x, ld_x, rows, K, data, scale, scale_ld, y, ld_y, noop, stream)
                        : launch_row<uint32_t>(x, ld_x, rows, K, data, scale, scale_ld, y, ld_y, noop, stream);
}

// Argument checks of the fold.  For a non-empty matrix it returns MXQ_OK with
// *ranges = {x, data, tile_code}; for an empty one MXQ_OK with *empty set.
static int block128_check(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt, uint8_t* data,
                          uint8_t* tile_code, int64_t tile_ld, const int32_t* noop, bool need_noop, Range* ranges,
                          bool* empty) {
  *empty = false;
  if (check_dtype(dt)) return MXQ_ERR_DTYPE;
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (rows == 0 || K == 0) {
    *empty = true;
    return MXQ_OK;
  }
  if (!x || !data || !tile_code || (need_noop && !noop)) return MXQ_ERR_NULL;
  const int64_t ntc = (K + 127) / 128, ntr = (rows + 127) / 128;
  if (ld_x < K || tile_ld < ntc) return MXQ_ERR_SHAPE;
  const Range rx = matrix_range(x, rows, K, ld_x, dtype_size(dt)), rd = matrix_range(data, rows, K, K, 1),
              rt = matrix_range(tile_code, ntr, ntc, tile_ld, 1);
  if (!spans_ok({rx, rd, rt})) return MXQ_ERR_SHAPE;
  if (overlap(rx, rd) || overlap(rx, rt) || overlap(rd, rt)) return MXQ_ERR_ALIAS;
  ranges[0] = rx, ranges[1] = rd, ranges[2] = rt;
  return MXQ_OK;
}

static int block128_entry(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt, uint8_t* data,
                          uint8_t* tile_code, int64_t tile_ld, const int32_t* noop, bool need_noop,
                          hipStream_t stream) {
  Range r[3];
  bool empty;
  const int st = block128_check(x, ld_x, rows, K, dt, data, tile_code, tile_ld, noop, need_noop, r, &empty);
  if (st != MXQ_OK || empty) return st;
  return dt == MXQ_BF16 ? launch_block128<uint16_t>(x, ld_x, rows, K, data, tile_code, tile_ld, noop, stream)
                        : launch_block128<uint32_t>(x, ld_x, rows, K, data, tile_code, tile_ld, noop, stream);
}

int mxq_mxfp4_to_mxfp8_row(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt, uint8_t* data,
                           uint8_t* scale, int64_t scale_ld, hipStream_t stream) {
  return row_entry(x, ld_x, rows, K, dt, data, scale, scale_ld, nullptr, 0, false, nullptr, false, stream);
}

int mxq_mxfp4_to_mxfp8_row_guarded(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt,
                                   uint8_t* data, uint8_t* scale, int64_t scale_ld, const int32_t* noop,
                                   hipStream_t stream) {
  return row_entry(x, ld_x, rows, K, dt, data, scale, scale_ld, nullptr, 0, false, noop, true, stream);
}

int mxq_fake_quantize_mxfp4_with_mxfp8_row(const void* x, int64_t ld_x, void* y, int64_t ld_y, int64_t rows,
                                           int64_t K, mxq_dtype dt, uint8_t* data, uint8_t* scale,
                                           int64_t scale_ld, hipStream_t stream) {
  return row_entry(x, ld_x, rows, K, dt, data, scale, scale_ld, y, ld_y, true, nullptr, false, stream);
}

int mxq_mxfp4_to_fp8_block128(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt, uint8_t* data,
                              uint8_t* tile_code, int64_t tile_ld, hipStream_t stream) {
  return block128_entry(x, ld_x, rows, K, dt, data, tile_code, tile_ld, nullptr, false, stream);
}

int mxq_mxfp4_to_fp8_block128_guarded(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt,
                                      uint8_t* data, uint8_t* tile_code, int64_t tile_ld, const int32_t* noop,
                                      hipStream_t stream) {
  return block128_entry(x, ld_x, rows, K, dt, data, tile_code, tile_ld, noop, true, stream);
}

int mxq_mxfp4_to_fp8_block128_grouped(const mxq_block128_group* groups, int64_t n_groups, mxq_dtype dt,
                                      hipStream_t stream) {
  if (check_dtype(dt)) return MXQ_ERR_DTYPE;
  if (n_groups < 0) return MXQ_ERR_SHAPE;
  if (n_groups == 0) return MXQ_OK;
  if (!groups) return MXQ_ERR_NULL;
  const int J = dt == MXQ_BF16 ? FoldGeom<uint16_t>::kJ : FoldGeom<uint32_t>::kJ;
  std::vector<std::pair<Range, bool>> iv;                   // (range, is an output)
  iv.reserve((size_t)std::min<int64_t>(n_groups, 1 << 20) * 3);
  for (int64_t i = 0; i < n_groups; i++) {
    const mxq_block128_group& g = groups[i];
    Range r[3];
    bool empty;
    const int st = block128_check(g.x, g.ld_x, g.rows, g.K, dt, g.data, g.tile_code, g.tile_ld, nullptr, false, r,
                                  &empty);
    if (st != MXQ_OK) return st;
    if (empty) continue;
    const int64_t tpr = (g.K + 127) / 128, gpr = (tpr + J - 1) / J;
    if (gpr * ((g.rows + 127) / 128) >= kMaxSteps) return MXQ_ERR_SHAPE;
    iv.push_back({r[0], false});
    iv.push_back({r[1], true});
    iv.push_back({r[2], true});
  }
  if (!grouped_ranges_disjoint(iv)) return MXQ_ERR_ALIAS;
  return dt == MXQ_BF16 ? launch_block128_grouped<uint16_t>(groups, n_groups, stream)
                        : launch_block128_grouped<uint32_t>(groups, n_groups, stream);
}

int mxq_mxfp4_to_mxfp8_row_grouped(const mxq_row_group* groups, int64_t n_groups, mxq_dtype dt,
                                   hipStream_t stream) {
  if (check_dtype(dt)) return MXQ_ERR_DTYPE;
  if (n_groups < 0) return MXQ_ERR_SHAPE;
  if (n_groups == 0) return MXQ_OK;
  if (!groups) return MXQ_ERR_NULL;
  // the smaller step of the grouped kernel and of the single launch an unaligned weight takes: the most steps
  const int64_t eps = dt == MXQ_BF16 ? std::min(StepGeom<uint16_t, kRowThreads>::kElemsPerStep,
                                                StepGeom<uint16_t, kRowGroupedThreads>::kElemsPerStep)
                                     : std::min(StepGeom<uint32_t, kRowThreads>::kElemsPerStep,
                                                StepGeom<uint32_t, kRowGroupedThreads>::kElemsPerStep);
  // every group on its own, then no output may overlap any other range
  std::vector<std::pair<Range, bool>> iv;                   // (range, is an output)
  iv.reserve((size_t)std::min<int64_t>(n_groups, 1 << 20) * 3);
  for (int64_t i = 0; i < n_groups; i++) {
    const mxq_row_group& g = groups[i];
    Range r[3];
    bool empty;
    const int st = row_check(g.x, g.ld_x, g.rows, g.K, dt, g.data, g.scale, g.scale_ld, nullptr, 0, false, nullptr,
                             false, r, &empty);
    if (st != MXQ_OK) return st;
    if (empty) continue;
    MxqDivisor spr;
    uint32_t total;
    if (steps_for(g.rows, g.K, eps, &spr, &total)) return MXQ_ERR_SHAPE;
    iv.push_back({r[0], false});
    iv.push_back({r[1], true});
    iv.push_back({r[2], true});
  }
  if (!grouped_ranges_disjoint(iv)) return MXQ_ERR_ALIAS;
  return dt == MXQ_BF16 ? launch_row_grouped<uint16_t>(groups, n_groups, stream)
                        : launch_row_grouped<uint32_t>(groups, n_groups, stream);
}

static int col_entry(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt, uint8_t* row_data,
                     uint8_t* row_scale, int64_t row_scale_ld, bool with_row, uint8_t* col_data, uint8_t* col_scale,
                     int64_t col_scale_ld, const int32_t* noop, bool need_noop, hipStream_t stream) {
  if (check_dtype(dt)) return MXQ_ERR_DTYPE;
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!x || !col_data || !col_scale || (with_row && (!row_data || !row_scale)) || (need_noop && !noop))
    return MXQ_ERR_NULL;
  const int64_t nb = (K + 31) / 32, bands = (rows + 31) / 32;
  if (ld_x < K || col_scale_ld < K || (with_row && row_scale_ld < nb)) return MXQ_ERR_SHAPE;
  const Range rx = matrix_range(x, rows, K, ld_x, dtype_size(dt)), cd = matrix_range(col_data, rows, K, K, 1),
              cs = matrix_range(col_scale, bands, K, col_scale_ld, 1);
  if (!spans_ok({rx, cd, cs})) return MXQ_ERR_SHAPE;
  if (overlap(rx, cd) || overlap(rx, cs) || overlap(cd, cs)) return MXQ_ERR_ALIAS;
  if (with_row) {
    const Range rd = matrix_range(row_data, rows, K, K, 1), rs = matrix_range(row_scale, rows, nb, row_scale_ld, 1);
    if (!spans_ok({rd, rs})) return MXQ_ERR_SHAPE;
    if (overlap(rx, rd) || overlap(rx, rs) || overlap(rd, rs) || overlap(rd, cd) || overlap(rd, cs) ||
        overlap(rs, cd) || overlap(rs, cs))
      return MXQ_ERR_ALIAS;
  } else {
    row_data = nullptr, row_scale = nullptr, row_scale_ld = 0;
  }
  return dt == MXQ_BF16 ? launch_col<uint16_t>(x, ld_x, rows, K, col_data, col_scale, col_scale_ld, row_data,
                                               row_scale, row_scale_ld, noop, stream)
                        : launch_col<uint32_t>(x, ld_x, rows, K, col_data, col_scale, col_scale_ld, row_data,
                                               row_scale, row_scale_ld, noop, stream);
}

int mxq_mxfp4_to_mxfp8_col(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt, uint8_t* data,
                           uint8_t* scale, int64_t scale_ld, hipStream_t stream) {
  return col_entry(x, ld_x, rows, K, dt, nullptr, nullptr, 0, false, data, scale, scale_ld, nullptr, false, stream);
}

int mxq_mxfp4_to_mxfp8_col_guarded(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt,
                                   uint8_t* data, uint8_t* scale, int64_t scale_ld, const int32_t* noop,
                                   hipStream_t stream) {
  return col_entry(x, ld_x, rows, K, dt, nullptr, nullptr, 0, false, data, scale, scale_ld, noop, true, stream);
}

int mxq_mxfp4_to_mxfp8_row_col(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt,
                               uint8_t* row_data, uint8_t* row_scale, int64_t row_scale_ld, uint8_t* col_data,
                               uint8_t* col_scale, int64_t col_scale_ld, hipStream_t stream) {
  return col_entry(x, ld_x, rows, K, dt, row_data, row_scale, row_scale_ld, true, col_data, col_scale, col_scale_ld,
                   nullptr, false, stream);
}

int mxq_mxfp4_to_mxfp8_row_col_guarded(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt,
                                       uint8_t* row_data, uint8_t* row_scale, int64_t row_scale_ld,
                                       uint8_t* col_data, uint8_t* col_scale, int64_t col_scale_ld,
                                       const int32_t* noop, hipStream_t stream) {
  return col_entry(x, ld_x, rows, K, dt, row_data, row_scale, row_scale_ld, true, col_data, col_scale, col_scale_ld,
                   noop, true, stream);
}

int mxq_export_mxfp8(const uint8_t* data, const uint8_t* scale_storage, int64_t rows, int64_t K, int64_t scale_ld,
                     uint8_t* scale_out, hipStream_t stream) {
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (!data || !scale_storage) return MXQ_ERR_NO_ROWWISE_DATA;
  if (rows == 0 || K == 0) return MXQ_OK;
  const int64_t nb = (K + 31) / 32;
  if (scale_ld < nb) return MXQ_ERR_SHAPE;
  if (!scale_out) return MXQ_ERR_NULL;
  if (scale_out == scale_storage && scale_ld == nb) return MXQ_OK;          // already unpadded: a view
  const Range rs = matrix_range(scale_storage, rows, nb, scale_ld, 1), ro = matrix_range(scale_out, rows, nb, nb, 1);
  if (!spans_ok({rs, ro})) return MXQ_ERR_SHAPE;
  if (overlap(rs, ro)) return MXQ_ERR_ALIAS;
  const uintptr_t a = reinterpret_cast<uintptr_t>(scale_storage) | reinterpret_cast<uintptr_t>(scale_out);
  const int64_t width = (a % 16 == 0 && scale_ld % 16 == 0 && nb % 16 == 0) ? 16
                        : (a % 4 == 0 && scale_ld % 4 == 0 && nb % 4 == 0) ? 4 : 1;
  const int64_t units = rows * (nb / width);
  if (units >= kMaxSteps * 2) return MXQ_ERR_SHAPE;
  // a multiple of 8 workgroups (the kernel gives each XCD a contiguous run of chunks)
  const dim3 grid((uint32_t)(((units + kThreads - 1) / kThreads + 7) / 8 * 8)), block(kThreads);
  const MxqDivisor upr = mxq_divisor((uint32_t)(nb / width));
  const uint32_t total = (uint32_t)units;
  if (MXQ_EXPORT4 && width == 4 && aligned(scale_out, 16) && nb % 16 == 0) {
    // four 4-byte units per lane, one 16-byte store
    const int64_t units16 = rows * (nb / 16);
    const dim3 grid16((uint32_t)(((units16 + kThreads - 1) / kThreads + 7) / 8 * 8));
    hipLaunchKernelGGL(export4_kernel, grid16, block, 0, stream, scale_storage, scale_ld, scale_out,
                       mxq_divisor((uint32_t)(nb / 16)), (uint32_t)units16);
  } else if (width == 16)
    hipLaunchKernelGGL(export_kernel<u32x4>, grid, block, 0, stream, scale_storage, scale_ld, scale_out, upr, total);
  else if (width == 4)
    hipLaunchKernelGGL(export_kernel<uint32_t>, grid, block, 0, stream, scale_storage, scale_ld, scale_out, upr, total);
  else
    hipLaunchKernelGGL(export_kernel<uint8_t>, grid, block, 0, stream, scale_storage, scale_ld, scale_out, upr, total);
  return launch_status();
}

// Argument checks of the decode, format and layout already checked.  For a
// non-empty matrix it returns MXQ_OK with r = {data, scale, out}; for an empty
// one MXQ_OK with *empty set.
static int dequant_check(const uint8_t* data, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K,
                         mxq_scale_layout layout, const void* out, int64_t ld_out, mxq_dtype out_dt, Range* r,
                         bool* empty) {
  *empty = false;
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (rows == 0 || K == 0) {
    *empty = true;
    return MXQ_OK;
  }
  if (!data || !scale || !out) return MXQ_ERR_NULL;
  const bool tile = layout == MXQ_SCALE_TILE_128X128, col = layout == MXQ_SCALE_COL_32X1;
  const int64_t srows = tile ? (rows + 127) / 128 : col ? (rows + 31) / 32 : rows,
                scols = tile ? (K + 127) / 128 : col ? K : (K + 31) / 32;
  if (ld_out < K || scale_ld < scols) return MXQ_ERR_SHAPE;
  r[0] = matrix_range(data, rows, K, K, 1);
  r[1] = matrix_range(scale, srows, scols, scale_ld, 1);
  r[2] = matrix_range(out, rows, K, ld_out, dtype_size(out_dt));
  if (!spans_ok({r[0], r[1], r[2]})) return MXQ_ERR_SHAPE;
  if (overlap(r[2], r[0]) || overlap(r[2], r[1])) return MXQ_ERR_ALIAS;
  return MXQ_OK;
}

int mxq_dequantize(const uint8_t* data, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K,
                   mxq_fp8 fmt, mxq_scale_layout layout, void* out, int64_t ld_out, mxq_dtype out_dt,
                   hipStream_t stream) {
  if (check_dtype(out_dt)) return MXQ_ERR_DTYPE;
  if (fmt != MXQ_E4M3 && fmt != MXQ_E5M2) return MXQ_ERR_DTYPE;
  if (layout != MXQ_SCALE_ROW_1X32 && layout != MXQ_SCALE_TILE_128X128 && layout != MXQ_SCALE_COL_32X1)
    return MXQ_ERR_DTYPE;
  Range r[3];
  bool empty;
  const int st = dequant_check(data, scale, scale_ld, rows, K, layout, out, ld_out, out_dt, r, &empty);
  if (st != MXQ_OK || empty) return st;
  return out_dt == MXQ_BF16 ? launch_dequant<uint16_t>(data, scale, scale_ld, rows, K, fmt, layout, out, ld_out, stream)
                            : launch_dequant<uint32_t>(data, scale, scale_ld, rows, K, fmt, layout, out, ld_out, stream);
}

int mxq_dequantize_grouped(const mxq_dequant_group* groups, int64_t n_groups, mxq_fp8 fmt, mxq_scale_layout layout,
                           mxq_dtype out_dt, hipStream_t stream) {
  if (check_dtype(out_dt)) return MXQ_ERR_DTYPE;
  if (fmt != MXQ_E4M3 && fmt != MXQ_E5M2) return MXQ_ERR_DTYPE;
  if (layout != MXQ_SCALE_ROW_1X32 && layout != MXQ_SCALE_TILE_128X128 && layout != MXQ_SCALE_COL_32X1)
    return MXQ_ERR_DTYPE;
  if (n_groups < 0) return MXQ_ERR_SHAPE;
  if (n_groups == 0) return MXQ_OK;
  if (!groups) return MXQ_ERR_NULL;
  // every group on its own, then no output may overlap any other range
  std::vector<std::pair<Range, bool>> iv;                   // (range, is an output)
  iv.reserve((size_t)std::min<int64_t>(n_groups, 1 << 20) * 3);
  for (int64_t i = 0; i < n_groups; i++) {
    const mxq_dequant_group& g = groups[i];
    Range r[3];
    bool empty;
    const int st = dequant_check(g.data, g.scale, g.scale_ld, g.rows, g.K, layout, g.out, g.ld_out, out_dt, r, &empty);
    if (st != MXQ_OK) return st;
    if (empty) continue;
    MxqDivisor spr;
    uint32_t total;
    const int64_t eps = 8 * (out_dt == MXQ_BF16 ? DequantShape<uint16_t>::kThreads : DequantShape<uint32_t>::kThreads);
    if (steps_for(g.rows, g.K, eps, &spr, &total)) return MXQ_ERR_SHAPE;
    iv.push_back({r[0], false});
    iv.push_back({r[1], false});
    iv.push_back({r[2], true});
  }
  if (!grouped_ranges_disjoint(iv)) return MXQ_ERR_ALIAS;
  return out_dt == MXQ_BF16 ? launch_dequant_grouped<uint16_t>(groups, n_groups, fmt, layout, stream)
                            : launch_dequant_grouped<uint32_t>(groups, n_groups, fmt, layout, stream);
}

// Argument checks of the packed encode.  For a non-empty matrix it returns
// MXQ_OK with r = {x, packed, scale}; for an empty one MXQ_OK with *empty set.
static int quantize_mxfp4_check(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt,
                                const uint8_t* packed, const uint8_t* scale, int64_t scale_ld, Range* r, bool* empty) {
  *empty = false;
  if (check_dtype(dt)) return MXQ_ERR_DTYPE;
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (rows == 0 || K == 0) {
    *empty = true;
    return MXQ_OK;
  }
  if (!x || !packed || !scale) return MXQ_ERR_NULL;
  const int64_t nb = (K + 31) / 32, pw = (K + 1) / 2;
  if (ld_x < K || scale_ld < nb) return MXQ_ERR_SHAPE;
  r[0] = matrix_range(x, rows, K, ld_x, dtype_size(dt));
  r[1] = matrix_range(packed, rows, pw, pw, 1);
  r[2] = matrix_range(scale, rows, nb, scale_ld, 1);
  if (!spans_ok({r[0], r[1], r[2]})) return MXQ_ERR_SHAPE;
  if (overlap(r[0], r[1]) || overlap(r[0], r[2]) || overlap(r[1], r[2])) return MXQ_ERR_ALIAS;
  return MXQ_OK;
}

int mxq_quantize_mxfp4(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt, uint8_t* packed,
                       uint8_t* scale, int64_t scale_ld, hipStream_t stream) {
  Range r[3];
  bool empty;
  const int st = quantize_mxfp4_check(x, ld_x, rows, K, dt, packed, scale, scale_ld, r, &empty);
  if (st != MXQ_OK || empty) return st;
  return dt == MXQ_BF16 ? launch_quantize_mxfp4<uint16_t>(x, ld_x, rows, K, packed, scale, scale_ld, stream)
                        : launch_quantize_mxfp4<uint32_t>(x, ld_x, rows, K, packed, scale, scale_ld, stream);
}

int mxq_quantize_mxfp4_grouped(const mxq_mxfp4_group* groups, int64_t n_groups, mxq_dtype dt, hipStream_t stream) {
  if (check_dtype(dt)) return MXQ_ERR_DTYPE;
  if (n_groups < 0) return MXQ_ERR_SHAPE;
  if (n_groups == 0) return MXQ_OK;
  if (!groups) return MXQ_ERR_NULL;
  const int64_t eps = dt == MXQ_BF16 ? StepGeom<uint16_t, kQ4Threads>::kElemsPerStep
                                     : StepGeom<uint32_t, kQ4Threads>::kElemsPerStep;
  // every group on its own, then no output may overlap any other range
  std::vector<std::pair<Range, bool>> iv;                   // (range, is an output)
  iv.reserve((size_t)std::min<int64_t>(n_groups, 1 << 20) * 3);
  for (int64_t i = 0; i < n_groups; i++) {
    const mxq_mxfp4_group& g = groups[i];
    Range r[3];
    bool empty;
    const int st = quantize_mxfp4_check(g.x, g.ld_x, g.rows, g.K, dt, g.packed, g.scale, g.scale_ld, r, &empty);
    if (st != MXQ_OK) return st;
    if (empty) continue;
    MxqDivisor spr;
    uint32_t total;
    if (steps_for(g.rows, g.K, eps, &spr, &total)) return MXQ_ERR_SHAPE;
    iv.push_back({r[0], false});
    iv.push_back({r[1], true});
    iv.push_back({r[2], true});
  }
  if (!grouped_ranges_disjoint(iv)) return MXQ_ERR_ALIAS;
  return dt == MXQ_BF16 ? launch_quantize_mxfp4_grouped<uint16_t>(groups, n_groups, stream)
                        : launch_quantize_mxfp4_grouped<uint32_t>(groups, n_groups, stream);
}

int mxq_dequantize_mxfp4(const uint8_t* packed, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K,
                         void* out, int64_t ld_out, mxq_dtype out_dt, hipStream_t stream) {
  if (check_dtype(out_dt)) return MXQ_ERR_DTYPE;
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!packed || !scale || !out) return MXQ_ERR_NULL;
  const int64_t nb = (K + 31) / 32, pw = (K + 1) / 2;
  if (ld_out < K || scale_ld < nb) return MXQ_ERR_SHAPE;
  const Range ro = matrix_range(out, rows, K, ld_out, dtype_size(out_dt)), rp = matrix_range(packed, rows, pw, pw, 1),
              rs = matrix_range(scale, rows, nb, scale_ld, 1);
  if (!spans_ok({ro, rp, rs})) return MXQ_ERR_SHAPE;
  if (overlap(ro, rp) || overlap(ro, rs)) return MXQ_ERR_ALIAS;
  return out_dt == MXQ_BF16 ? launch_dequantize_mxfp4<uint16_t>(packed, scale, scale_ld, rows, K, out, ld_out, stream)
                            : launch_dequantize_mxfp4<uint32_t>(packed, scale, scale_ld, rows, K, out, ld_out, stream);
}

int mxq_mxfp4_packed_to_mxfp8_row(const uint8_t* packed, const uint8_t* scale, int64_t scale_ld, int64_t rows,
                                  int64_t K, uint8_t* data, uint8_t* scale_out, int64_t scale_out_ld,
                                  hipStream_t stream) {
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!packed || !scale || !data || !scale_out) return MXQ_ERR_NULL;
  const int64_t nb = (K + 31) / 32, pw = (K + 1) / 2;
  if (scale_ld < nb || scale_out_ld < nb) return MXQ_ERR_SHAPE;
  const Range rp = matrix_range(packed, rows, pw, pw, 1), rs = matrix_range(scale, rows, nb, scale_ld, 1),
              rd = matrix_range(data, rows, K, K, 1), ro = matrix_range(scale_out, rows, nb, scale_out_ld, 1);
  if (!spans_ok({rp, rs, rd, ro})) return MXQ_ERR_SHAPE;
  if (overlap(rd, rp) || overlap(rd, rs) || overlap(ro, rp) || overlap(ro, rs) || overlap(rd, ro)) return MXQ_ERR_ALIAS;
  MxqDivisor spr;
  uint32_t total;
  if (steps_for(rows, K, kPackedThreads * 16, &spr, &total)) return MXQ_ERR_SHAPE;
  const bool vec = aligned(packed, 8) && aligned(data, 16) && K % 16 == 0;
  // every step whole and every workgroup's steps inside the grid: no bounds checks
  // (and, for the gathered code stores, code rows aligned to their width: 4 bytes)
  const int code_width = MXQ_PACKED_CODE_WORDS ? CodeGather<2>::kCodes : 1;
  const bool full = vec && spr.d * (int64_t)(kPackedThreads * 16) == K && total % kPackedSteps == 0 && fits32(K) &&
                    aligned(scale_out, code_width) && scale_out_ld % code_width == 0;
  const dim3 grid(grid_for(total, kPackedSteps)), block(kPackedThreads);
  if (full)
    hipLaunchKernelGGL((packed_convert_kernel<true, true>), grid, block, 0, stream, packed, scale, scale_ld, K, data,
                       scale_out, scale_out_ld, spr, total);
  else if (vec)
    hipLaunchKernelGGL((packed_convert_kernel<true, false>), grid, block, 0, stream, packed, scale, scale_ld, K, data,
                       scale_out, scale_out_ld, spr, total);
  else
    hipLaunchKernelGGL((packed_convert_kernel<false, false>), grid, block, 0, stream, packed, scale, scale_ld, K, data,
                       scale_out, scale_out_ld, spr, total);
  return launch_status();
}

int mxq_mxfp4_packed_to_fp8_block128(const uint8_t* packed, const uint8_t* scale, int64_t scale_ld, int64_t rows,
                                     int64_t K, uint8_t* data, uint8_t* tile_code, int64_t tile_ld,
                                     hipStream_t stream) {
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!packed || !scale || !data || !tile_code) return MXQ_ERR_NULL;
  const int64_t nb = (K + 31) / 32, pw = (K + 1) / 2, ntc = (K + 127) / 128, ntr = (rows + 127) / 128;
  if (scale_ld < nb || tile_ld < ntc) return MXQ_ERR_SHAPE;
  const Range rp = matrix_range(packed, rows, pw, pw, 1), rs = matrix_range(scale, rows, nb, scale_ld, 1),
              rd = matrix_range(data, rows, K, K, 1), rt = matrix_range(tile_code, ntr, ntc, tile_ld, 1);
  if (!spans_ok({rp, rs, rd, rt})) return MXQ_ERR_SHAPE;
  if (overlap(rd, rp) || overlap(rd, rs) || overlap(rt, rp) || overlap(rt, rs) || overlap(rd, rt)) return MXQ_ERR_ALIAS;
  if (ntc * ntr >= kMaxSteps) return MXQ_ERR_SHAPE;
  const int64_t groups = (ntc + 3) / 4;
  if (ntr * groups >= kMaxSteps) return MXQ_ERR_SHAPE;
  const bool vec = aligned(packed, 8) && aligned(data, 16) && K % 16 == 0;
  const bool codes_vec = aligned(scale, 8) && scale_ld % 8 == 0;
  const dim3 grid((uint32_t)(ntr * groups)), block(kPFoldThreads);
  if (vec)
    hipLaunchKernelGGL((packed_fold_kernel<true>), grid, block, 0, stream, packed, scale, scale_ld, rows, K, data,
                       tile_code, tile_ld, mxq_divisor((uint32_t)groups), codes_vec);
  else
    hipLaunchKernelGGL((packed_fold_kernel<false>), grid, block, 0, stream, packed, scale, scale_ld, rows, K, data,
                       tile_code, tile_ld, mxq_divisor((uint32_t)groups), codes_vec);
  return launch_status();
}

}  // extern "C"
