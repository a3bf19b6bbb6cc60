// mxq.hip -- gfx950 kernels and the C ABI of include/mxq.h.
//
// Block-scaled weight quantization: MXFP4 projection, the direct MXFP8 rowwise
// lift, 128x128 tile-exponent folding into E4M3, the unpadded scale export and
// the E8M0 decode.  Sources (page title, section):
//   [QAT] "[PyTorch] MXFP4 weight QAT on MXFP8 and FP8 block-scaling recipes":
//         Description (both conversion modes, the E8M0 decode), Test results,
//         Known limitations.
//   [EXP] "MXFP8TensorStorage.export_components()": Description.
//
// Design (CDNA4, wave64).  Every kernel streams HBM once; nothing here is a
// contraction, so there is no MFMA.  A lane owns one 16-byte chunk of a row per
// step (8 bf16 or 4 fp32), so a 1x32 block spans 4 (bf16) or 8 (fp32)
// neighbouring lanes and its amax is reduced with two or three DPP moves.  All
// arithmetic is integer: the scale exponent comes from the amax bit pattern,
// E2M1 rounding is done on bit patterns relative to the block scale, and bf16
// pairs are processed as packed 16-bit lanes (v_pk_* integer ops).  Results do
// not depend on denormal or fast-math settings.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "mxq.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));

// Launch-shape tunables (compile-time).
#ifndef MXQ_STEPS_PER_WG
#define MXQ_STEPS_PER_WG 4        // 16-byte chunks in flight per lane in the streaming kernels
#endif
#ifndef MXQ_NT_LOADS
#define MXQ_NT_LOADS 1            // streaming loads carry the non-temporal hint
#endif
#ifndef MXQ_NT_STORES
#define MXQ_NT_STORES 1           // streaming stores carry the non-temporal hint
#endif

constexpr int kThreads = 256;     // 4 waves per workgroup
constexpr int kStepsPerWG = MXQ_STEPS_PER_WG;

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

// ------------------------------------------------------------------------------------
// Packed 16-bit integer helpers (two bf16 patterns per 32-bit register)
// ------------------------------------------------------------------------------------
__device__ __forceinline__ u16x2 U2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ i16x2 I2(uint32_t v) { return __builtin_bit_cast(i16x2, v); }
__device__ __forceinline__ uint32_t W(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ uint32_t W(i16x2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) { return W(__builtin_elementwise_max(U2(a), U2(b))); }
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) { return W(__builtin_elementwise_min(U2(a), U2(b))); }
__device__ __forceinline__ uint32_t pk_max_i16(uint32_t a, uint32_t b) { return W(__builtin_elementwise_max(I2(a), I2(b))); }
__device__ __forceinline__ uint32_t pk_mad_u16(uint32_t a, uint16_t m, uint32_t c) {
  return W(U2(a) * (u16x2)(m) + U2(c));
}
__device__ __forceinline__ uint32_t pk_add_u16(uint32_t a, uint32_t b) { return W(U2(a) + U2(b)); }
__device__ __forceinline__ uint32_t pk_sub_u16(uint32_t a, uint32_t b) { return W(U2(a) - U2(b)); }
__device__ __forceinline__ uint32_t splat16(uint32_t v) { return (v & 0xFFFFu) * 0x00010001u; }

// Byte permute: result byte i = byte sel_i of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// DPP lane moves inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
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
  static constexpr uint32_t kNaN = 0x7FC0u;
};
template <>
struct Fmt<uint32_t> {   // fp32 bit patterns
  static constexpr int kEPL = 4;
  static constexpr int kLPB = 8;
  static constexpr uint32_t kNaN = 0x7FC00000u;
};

// ------------------------------------------------------------------------------------
// The MXFP4 decomposition of one block ([QAT] Description, conversion mode 1)
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

__device__ __forceinline__ Block block_from_amax_bf16(uint32_t amax) {
  int eb = (int)((amax + 0x3Fu) >> 7) - 2;
  eb = min(max(eb, 1), 252);
  return Block{(uint32_t)eb, amax >= 0x7F80u};
}
__device__ __forceinline__ Block block_from_amax_fp32(uint32_t amax) {
  int eb = (int)((amax + 0x3FFFFFu) >> 23) - 2;
  eb = min(max(eb, 1), 252);
  return Block{(uint32_t)eb, amax >= 0x7F800000u};
}

// E2M1 code c (0..7 for 0, .5, 1, 1.5, 2, 3, 4, 6) of RTNE(|x| / 2^e), returned
// as C = c + 2.
//
// Let d = |x| - 2^e measured in bit-pattern units (one binade = 2^mbits).  The
// value t = |x| / 2^e, mapped to D = 2^(mbits+2) * (t - 1), is the rounding
// variable: E2M1 steps of 0.5 below t = 2 are steps of 2^(mbits+1) in D, and
// above t = 1 bit patterns are linear within each binade with two E2M1 values
// per binade, so there D = 4d.  Below t = 1 the binades shrink: D = 2d in the
// binade just below 2^e and D = d - 2^mbits in the next one (further down t <
// 1/4 rounds to 0 whatever D is).  D = max(4d, 2d, d - 2^mbits) covers all of
// that at once; when eb <= 2 the subnormal patterns continue binade 1 linearly,
// so the pieces that assume a narrower binade are switched off.  Ties are
// broken to the even code by the usual "add half - 1 + lsb" step.  The
// clamp of |x| to [2^e / 16, 6 * 2^e] keeps D in range and makes values above
// 6 * 2^e (only possible at the e = 125 cap) saturate to 6.
struct CodeConsts16 {   // bf16, broadcast to both 16-bit halves
  uint32_t lo, hi, k4, k2, k1;
};
__device__ __forceinline__ CodeConsts16 code_consts_bf16(uint32_t eb) {
  const uint32_t A1 = eb << 7;                      // pattern of 2^e
  CodeConsts16 k;
  k.lo = splat16(A1 > 512u ? A1 - 512u : 0u);       // 2^(e-4)
  k.hi = splat16(A1 + 320u);                        // 6 * 2^e
  // D + 1024 for each piece (1024 keeps D positive and the tie parity intact)
  k.k4 = splat16(1024u - 4u * A1);
  k.k2 = splat16(1024u - 2u * A1 - (eb == 1 ? 4096u : 0u));
  k.k1 = splat16(896u - A1 - (eb <= 2 ? 4096u : 0u));
  return k;
}

// Codes of two bf16 elements (one 32-bit word of magnitudes a): two C values.
__device__ __forceinline__ uint32_t codes_bf16(uint32_t a, const CodeConsts16& k) {
  uint32_t ac = pk_min_u16(pk_max_u16(a, k.lo), k.hi);
  uint32_t p4 = pk_mad_u16(ac, 4, k.k4);
  uint32_t p2 = pk_mad_u16(ac, 2, k.k2);
  uint32_t p1 = pk_add_u16(ac, k.k1);
  uint32_t D = pk_max_i16(pk_max_i16(p4, p2), p1);            // 384 .. 2304 per half
  uint32_t lsb = (D >> 8) & 0x00010001u;
  uint32_t S = D + 0x007F007Fu + lsb;                           // no carry between halves
  return (S >> 8) & 0x00FF00FFu;                                // C = c + 2 in 2..9
}

struct CodeConsts32 {
  uint32_t A1, lo, hi;
  int32_t k2, k1;
};
__device__ __forceinline__ CodeConsts32 code_consts_fp32(uint32_t eb) {
  CodeConsts32 k;
  k.A1 = eb << 23;
  k.lo = k.A1 > (4u << 23) ? k.A1 - (4u << 23) : 0u;
  k.hi = k.A1 + (5u << 22);
  k.k2 = eb == 1 ? -(1 << 28) : 0;
  k.k1 = (eb <= 2 ? -(1 << 28) : 0) - (1 << 23);
  return k;
}
__device__ __forceinline__ uint32_t code_fp32(uint32_t a, const CodeConsts32& k) {
  uint32_t ac = min(max(a, k.lo), k.hi);
  int32_t d = (int32_t)(ac - k.A1);
  int32_t D = max(max(4 * d, 2 * d + k.k2), d + k.k1) + (1 << 26);
  uint32_t Du = (uint32_t)D;
  return (Du + (1u << 23) - 1u + ((Du >> 24) & 1u)) >> 24;      // C = c + 2 in 2..9
}

// ------------------------------------------------------------------------------------
// Output encodings from C = c + 2
// ------------------------------------------------------------------------------------
// Projection, bf16: p * 2^e for c >= 2 has pattern (eb-1)*128 + 64c, i.e.
// (eb-2)*128 + 64C; c = 1 (0.5 * 2^e) is (eb-1)*128, except at eb = 1 where it
// is the subnormal 0x0040, which the first formula already gives; c = 0 is 0.
// min() of three affine pieces picks the right one for every C.
struct ProjConsts16 {
  uint32_t kq, k3, floor, smask;
};
__device__ __forceinline__ ProjConsts16 proj_consts_bf16(Block b) {
  ProjConsts16 p;
  p.kq = splat16((b.eb - 2u) << 7);
  p.k3 = splat16(b.eb == 1 ? 0x7C00u : (b.eb - 4u) << 7);
  p.floor = b.poison ? 0x7FC07FC0u : 0u;
  p.smask = b.poison ? 0u : 0x80008000u;
  return p;
}
__device__ __forceinline__ uint32_t proj_word_bf16(uint32_t w, uint32_t C, const ProjConsts16& p) {
  uint32_t q = pk_mad_u16(C, 64, p.kq);
  uint32_t q3 = pk_mad_u16(C, 128, p.k3);
  uint32_t q5 = pk_sub_u16(0x00020002u, C);                     // 0 for c = 0, huge otherwise
  uint32_t m = pk_max_u16(pk_min_u16(pk_min_u16(q, q3), q5), p.floor);
  return (w & p.smask) | m;
}

__device__ __forceinline__ uint32_t proj_fp32(uint32_t w, uint32_t C, Block b) {
  if (b.poison) return Fmt<uint32_t>::kNaN;
  uint32_t m;
  if (C <= 2u) m = 0u;
  else if (C == 3u && b.eb >= 2u) m = (b.eb - 1u) << 23;
  else m = ((b.eb - 2u) << 23) + (C << 22);
  return (w & 0x80000000u) | m;
}

// Row lift payload: E4M3 of p * 2^s with s = min(6, e + 127) >= 1.  For c >= 1
// the exponent field is s + 6 + E(c) and the mantissa the E2M1 mantissa bit,
// giving bytes b, b+8, b+12, b+16, b+20, b+24, b+28 with b = (s + 6) * 8
// (b = 0x60 at s = 6: 0x60, 0x68, 0x6C, ..., 0x7C).  Eight entries = a v_perm LUT.
struct Lut8 {
  uint32_t lo, hi;    // bytes for codes 0..3 and 4..7
};
__device__ __forceinline__ Lut8 row_lut(Block b) {
  if (b.poison) return Lut8{0x7F7F7F7Fu, 0x7F7F7F7Fu};
  uint32_t s = min(b.eb, 6u);
  uint32_t base = (s + 6u) << 3;
  return Lut8{base * 0x01010100u + 0x0C080000u, base * 0x01010101u + 0x1C181410u};
}
__device__ __forceinline__ uint32_t row_code(Block b) {
  return b.poison ? 255u : (b.eb > 6u ? b.eb - 6u : 0u);         // max(e + 121, 0)
}

// 128x128 fold payload: RTNE_E4M3(p * 2^sh) for sh = e - S in [-16, 6] (anything
// lower rounds to zero like -16).  In units of the E4M3 subnormal step 2^-9 the
// value is N = 2p * 2^(sh + 8); below 16 steps the encoding is N itself
// (subnormals and the first normal binade share the step), above it the grid
// values are exact with at most two significant bits.
constexpr int kFoldMin = -16, kFoldMax = 6, kFoldEntries = kFoldMax - kFoldMin + 1;

constexpr uint32_t e4m3_grid_byte(int c, int sh) {
  const uint32_t twice_p[8] = {0, 1, 2, 3, 4, 6, 8, 12};
  const int s = sh + 8;
  uint32_t N = 0;
  if (s >= 0) {
    N = twice_p[c] << s;
  } else {
    const int r = -s;
    const uint32_t q = twice_p[c] >> r, rem = twice_p[c] & ((1u << r) - 1u), half = 1u << (r - 1);
    N = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
  }
  if (N < 16u) return N;
  int j = 0;
  while ((N >> (j + 1)) != 0u) j++;
  return ((uint32_t)(j - 2) << 3) | ((N >> (j - 3)) - 8u);
}

struct FoldTable {
  uint32_t w[2 * kFoldEntries];
};
constexpr FoldTable make_fold_table() {
  FoldTable t{};
  for (int i = 0; i < kFoldEntries; i++) {
    const int sh = kFoldMin + i;
    for (int c = 0; c < 8; c++) t.w[2 * i + c / 4] |= e4m3_grid_byte(c, sh) << (8 * (c % 4));
  }
  return t;
}
__constant__ FoldTable kFold = make_fold_table();
static_assert(e4m3_grid_byte(7, 6) == 0x7C && e4m3_grid_byte(1, 6) == 0x60, "fold table");
static_assert(e4m3_grid_byte(1, -6) == 0x04 && e4m3_grid_byte(7, -6) == 0x1C, "fold table");
static_assert(e4m3_grid_byte(1, -9) == 0x00 && e4m3_grid_byte(3, -9) == 0x02, "fold table");

// Payload bytes of four elements from their C = c + 2 values (one byte each in
// `sel_plus2`) and their sign bytes.
__device__ __forceinline__ uint32_t payload4(uint32_t sel_plus2, Lut8 lut, uint32_t sign_bytes, uint32_t smask8) {
  uint32_t q = perm(lut.hi, lut.lo, sel_plus2 - 0x02020202u);
  return q | (sign_bytes & smask8);
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

template <typename T, bool VEC>
__device__ __forceinline__ void store_chunk(T* __restrict__ row, int64_t col0, int64_t K, u32x4 w) {
  constexpr int EPL = Fmt<T>::kEPL;
  if (col0 >= K) return;
  if constexpr (VEC) {
    stream_store(w, reinterpret_cast<u32x4*>(row + col0));
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

// Payload bytes of one chunk: 8 (bf16 chunk) or 4 (fp32 chunk).
template <typename T>
struct PayloadChunk;
template <>
struct PayloadChunk<uint16_t> { typedef u32x2 type; };
template <>
struct PayloadChunk<uint32_t> { typedef uint32_t type; };

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
// Per-chunk pipelines
// ------------------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ uint32_t chunk_amax(u32x4 w) {
  if constexpr (sizeof(T) == 2) {
    uint32_t m = pk_max_u16(pk_max_u16(w[0] & 0x7FFF7FFFu, w[1] & 0x7FFF7FFFu),
                            pk_max_u16(w[2] & 0x7FFF7FFFu, w[3] & 0x7FFF7FFFu));
    return max(m & 0xFFFFu, m >> 16);
  } else {
    return max(max(w[0] & 0x7FFFFFFFu, w[1] & 0x7FFFFFFFu), max(w[2] & 0x7FFFFFFFu, w[3] & 0x7FFFFFFFu));
  }
}

template <typename T>
__device__ __forceinline__ Block chunk_block(u32x4 w) {
  uint32_t amax = block_max<Fmt<T>::kLPB>(chunk_amax<T>(w));
  if constexpr (sizeof(T) == 2) return block_from_amax_bf16(amax);
  else return block_from_amax_fp32(amax);
}

// C = c + 2 of every element of the chunk: bf16 -> 4 words of two 16-bit
// values; fp32 -> 4 words of one value each.
template <typename T>
__device__ __forceinline__ u32x4 chunk_codes(u32x4 w, Block b) {
  u32x4 C;
  if constexpr (sizeof(T) == 2) {
    const CodeConsts16 k = code_consts_bf16(b.eb);
#pragma unroll
    for (int i = 0; i < 4; i++) C[i] = codes_bf16(w[i] & 0x7FFF7FFFu, k);
  } else {
    const CodeConsts32 k = code_consts_fp32(b.eb);
#pragma unroll
    for (int i = 0; i < 4; i++) C[i] = code_fp32(w[i] & 0x7FFFFFFFu, k);
  }
  return C;
}

template <typename T>
__device__ __forceinline__ u32x4 chunk_proj(u32x4 w, Block b) {
  const u32x4 C = chunk_codes<T>(w, b);
  u32x4 y;
  if constexpr (sizeof(T) == 2) {
    const ProjConsts16 p = proj_consts_bf16(b);
#pragma unroll
    for (int i = 0; i < 4; i++) y[i] = proj_word_bf16(w[i], C[i], p);
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) y[i] = proj_fp32(w[i], C[i], b);
  }
  return y;
}

// E4M3 payload of the chunk through an 8-entry byte LUT indexed by code.
template <typename T>
__device__ __forceinline__ typename PayloadChunk<T>::type chunk_payload(u32x4 w, u32x4 C, Lut8 lut, bool poison) {
  const uint32_t smask8 = poison ? 0u : 0x80808080u;
  if constexpr (sizeof(T) == 2) {
    // bytes 0 and 2 of two words = the four low bytes of four 16-bit C values
    const uint32_t sel01 = perm(C[1], C[0], 0x06040200u), sel23 = perm(C[3], C[2], 0x06040200u);
    const uint32_t sg01 = perm(w[1], w[0], 0x07050301u), sg23 = perm(w[3], w[2], 0x07050301u);
    u32x2 p;
    p[0] = payload4(sel01, lut, sg01, smask8);
    p[1] = payload4(sel23, lut, sg23, smask8);
    return p;
  } else {
    const uint32_t sel = C[0] | (C[1] << 8) | (C[2] << 16) | (C[3] << 24);
    const uint32_t sg = perm(perm(w[3], w[2], 0x0C0C0703u), perm(w[1], w[0], 0x0C0C0703u), 0x05040100u);
    return payload4(sel, lut, sg, smask8);
  }
}

// ------------------------------------------------------------------------------------
// Streaming kernels: projection and row lift.  A "step" is 256 lanes x one
// 16-byte chunk = 2048 bf16 / 1024 fp32 elements of ONE row (64 / 32 blocks);
// rows are padded to whole steps, so the row / segment split is per-step
// uniform (scalar) arithmetic and no block straddles two lanes' rows.
// ------------------------------------------------------------------------------------
template <typename T>
struct StepGeom {
  static constexpr int kEPL = Fmt<T>::kEPL, kLPB = Fmt<T>::kLPB;
  static constexpr int kBlocksPerStep = kThreads / kLPB;
  static constexpr int64_t kElemsPerStep = (int64_t)kBlocksPerStep * 32;
};

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void proj_kernel(const T* __restrict__ x, int64_t ld_x, T* __restrict__ y,
                                                        int64_t ld_y, int64_t K, uint32_t steps_per_row,
                                                        uint32_t total_steps) {
  using G = StepGeom<T>;
  const uint32_t tid = threadIdx.x;
  const int64_t lane_col = (int64_t)(tid / G::kLPB) * 32 + (tid % G::kLPB) * G::kEPL;
  u32x4 w[kStepsPerWG];
#pragma unroll
  for (int u = 0; u < kStepsPerWG; u++) {
    const uint32_t step = blockIdx.x * kStepsPerWG + u;
    w[u] = u32x4{0u, 0u, 0u, 0u};
    if (step < total_steps) {
      const uint32_t row = step / steps_per_row, seg = step - row * steps_per_row;
      w[u] = load_chunk<T, VEC>(x + (int64_t)row * ld_x, seg * G::kElemsPerStep + lane_col, K);
    }
  }
#pragma unroll
  for (int u = 0; u < kStepsPerWG; u++) {
    const uint32_t step = blockIdx.x * kStepsPerWG + u;
    if (step < total_steps) {
      const uint32_t row = step / steps_per_row, seg = step - row * steps_per_row;
      const Block b = chunk_block<T>(w[u]);
      store_chunk<T, VEC>(y + (int64_t)row * ld_y, seg * G::kElemsPerStep + lane_col, K, chunk_proj<T>(w[u], b));
    }
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void row_kernel(const T* __restrict__ x, int64_t ld_x, int64_t K,
                                                       uint8_t* __restrict__ data, uint8_t* __restrict__ scale,
                                                       int64_t scale_ld, uint32_t steps_per_row,
                                                       uint32_t total_steps) {
  using G = StepGeom<T>;
  const uint32_t tid = threadIdx.x;
  const int64_t lane_col = (int64_t)(tid / G::kLPB) * 32 + (tid % G::kLPB) * G::kEPL;
  u32x4 w[kStepsPerWG];
#pragma unroll
  for (int u = 0; u < kStepsPerWG; u++) {
    const uint32_t step = blockIdx.x * kStepsPerWG + u;
    w[u] = u32x4{0u, 0u, 0u, 0u};
    if (step < total_steps) {
      const uint32_t row = step / steps_per_row, seg = step - row * steps_per_row;
      w[u] = load_chunk<T, VEC>(x + (int64_t)row * ld_x, seg * G::kElemsPerStep + lane_col, K);
    }
  }
#pragma unroll
  for (int u = 0; u < kStepsPerWG; u++) {
    const uint32_t step = blockIdx.x * kStepsPerWG + u;
    if (step < total_steps) {
      const uint32_t row = step / steps_per_row, seg = step - row * steps_per_row;
      const int64_t col0 = seg * G::kElemsPerStep + lane_col;
      const Block b = chunk_block<T>(w[u]);
      const u32x4 C = chunk_codes<T>(w[u], b);
      store_payload<T, VEC>(data + (int64_t)row * K, col0, K, chunk_payload<T>(w[u], C, row_lut(b), b.poison));
      if (tid % G::kLPB == 0 && col0 < K) scale[(int64_t)row * scale_ld + col0 / 32] = (uint8_t)row_code(b);
    }
  }
}

// ------------------------------------------------------------------------------------
// 128x128 tile fold: one workgroup per tile, one HBM pass.  The 256 lanes hold
// the whole tile in registers (bf16: 8 chunks per lane, fp32: 16), reduce the
// largest finite block exponent through DPP / shuffles and LDS, then write the
// folded payload.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void block128_kernel(const T* __restrict__ x, int64_t ld_x, int64_t rows,
                                                            int64_t K, uint8_t* __restrict__ data,
                                                            uint8_t* __restrict__ tile_code, int64_t tile_ld,
                                                            uint32_t tiles_per_row) {
  constexpr int EPL = Fmt<T>::kEPL, LPB = Fmt<T>::kLPB;
  constexpr int kChunksPerRow = 128 / EPL;             // 16 (bf16) / 32 (fp32)
  constexpr int kRowsPerPass = kThreads / kChunksPerRow;   // 16 / 8
  constexpr int kPasses = 128 / kRowsPerPass;              // 8 / 16
  __shared__ uint32_t s_fold[2 * kFoldEntries];
  __shared__ uint32_t s_wave_max[kThreads / 64];

  const uint32_t tid = threadIdx.x;
  const uint32_t tr = blockIdx.x / tiles_per_row, tc = blockIdx.x - tr * tiles_per_row;
  const int64_t r0 = (int64_t)tr * 128 + tid / kChunksPerRow;
  const int64_t col0 = (int64_t)tc * 128 + (tid % kChunksPerRow) * EPL;

  if (tid < 2 * kFoldEntries) s_fold[tid] = kFold.w[tid];

  u32x4 w[kPasses];
#pragma unroll
  for (int i = 0; i < kPasses; i++) {
    const int64_t r = r0 + i * kRowsPerPass;
    w[i] = (r < rows) ? load_chunk<T, VEC>(x + r * ld_x, col0, K) : u32x4{0u, 0u, 0u, 0u};
  }
  Block b[kPasses];
  uint32_t m = 1u;
#pragma unroll
  for (int i = 0; i < kPasses; i++) {
    b[i] = chunk_block<T>(w[i]);
    if (!b[i].poison) m = max(m, b[i].eb);
  }
  m = wave_max(m);
  if ((tid & 63u) == 0u) s_wave_max[tid >> 6] = m;
  __syncthreads();
  m = max(max(s_wave_max[0], s_wave_max[1]), max(s_wave_max[2], s_wave_max[3]));
  const uint32_t code = m > 6u ? m - 6u : 0u;                    // S + 127 = max(M - 6, -127) + 127
  if (tid == 0) tile_code[(int64_t)tr * tile_ld + tc] = (uint8_t)code;

#pragma unroll
  for (int i = 0; i < kPasses; i++) {
    const int64_t r = r0 + i * kRowsPerPass;
    const int sh = min(max((int)b[i].eb - (int)code, kFoldMin), kFoldMax);   // e - S
    const uint32_t idx = 2u * (uint32_t)(sh - kFoldMin);
    const Lut8 lut = b[i].poison ? Lut8{0x7F7F7F7Fu, 0x7F7F7F7Fu} : Lut8{s_fold[idx], s_fold[idx + 1]};
    const u32x4 C = chunk_codes<T>(w[i], b[i]);
    const auto p = chunk_payload<T>(w[i], C, lut, b[i].poison);
    if (r < rows) store_payload<T, VEC>(data + r * K, col0, K, p);
  }
  (void)LPB;
}

// ------------------------------------------------------------------------------------
// Decode: FP8 payload * 2^(code - 127) -> fp32 bits, exact (or Inf above the fp32
// range); bf16 is the nearest-even rounding of those fp32 bits.
// ------------------------------------------------------------------------------------
template <bool kE5M2>
__device__ __forceinline__ uint32_t decode_fp32(uint32_t q, uint32_t code) {
  constexpr int MB = kE5M2 ? 2 : 3, BIAS = kE5M2 ? 15 : 7;
  const uint32_t sign = (q & 0x80u) << 24, mag = q & 0x7Fu;
  const uint32_t E = mag >> MB, m = mag & ((1u << MB) - 1u);
  const bool nan = (code == 255u) || (kE5M2 ? (E == 31u && m != 0u) : (mag == 0x7Fu));
  if (nan) return 0x7FC00000u;
  if (kE5M2 && E == 31u) return sign | 0x7F800000u;
  const uint32_t sig = E ? ((1u << MB) | m) : m;
  if (sig == 0u) return sign;
  const int ex = E ? (int)E : 1;
  const int L = 31 - __clz((int)sig);
  const int biased = ex + (int)code + L - BIAS - MB;            // fp32 biased exponent
  if (biased >= 255) return sign | 0x7F800000u;
  if (biased >= 1) return sign | ((uint32_t)biased << 23) | ((sig << (23 - L)) & 0x7FFFFFu);
  return sign | (sig << (ex + (int)code + 22 - BIAS - MB));      // fp32 subnormal, exact
}
__device__ __forceinline__ uint32_t fp32_to_bf16_rne(uint32_t f) {
  if ((f & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (f + 0x7FFFu + ((f >> 16) & 1u)) >> 16;
}

template <typename TO, bool kE5M2, bool kTile, bool VEC>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ data,
                                                           const uint8_t* __restrict__ scale, int64_t scale_ld,
                                                           int64_t K, TO* __restrict__ out, int64_t ld_out,
                                                           uint32_t steps_per_row, uint32_t total_steps) {
  // 8 payload bytes per lane per step; 64 x 1x32 blocks per step.
  const uint32_t tid = threadIdx.x;
  const int64_t lane_col = (int64_t)tid * 8;
  for (int u = 0; u < kStepsPerWG; u++) {
    const uint32_t step = blockIdx.x * kStepsPerWG + u;
    if (step >= total_steps) break;
    const uint32_t row = step / steps_per_row, seg = step - row * steps_per_row;
    const int64_t col0 = (int64_t)seg * 2048 + lane_col;
    if (col0 >= K) continue;
    const uint8_t* drow = data + (int64_t)row * K;
    uint32_t q[2] = {0u, 0u};
    if (VEC) {
      const u32x2 v = stream_load(reinterpret_cast<const u32x2*>(drow + col0));
      q[0] = v[0];
      q[1] = v[1];
    } else {
      for (int i = 0; i < 8; i++)
        if (col0 + i < K) q[i / 4] |= (uint32_t)drow[col0 + i] << (8 * (i % 4));
    }
    const uint32_t code = kTile ? scale[(int64_t)(row / 128) * scale_ld + col0 / 128]
                                : scale[(int64_t)row * scale_ld + col0 / 32];
    uint32_t f[8];
#pragma unroll
    for (int i = 0; i < 8; i++) f[i] = decode_fp32<kE5M2>((q[i / 4] >> (8 * (i % 4))) & 0xFFu, code);
    TO* orow = out + (int64_t)row * ld_out;
    if constexpr (sizeof(TO) == 2) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; i++) o[i] = fp32_to_bf16_rne(f[2 * i]) | (fp32_to_bf16_rne(f[2 * i + 1]) << 16);
      if (VEC) {
        stream_store(o, reinterpret_cast<u32x4*>(orow + col0));
      } else {
        for (int i = 0; i < 8; i++)
          if (col0 + i < K) orow[col0 + i] = (uint16_t)(o[i / 2] >> (16 * (i % 2)));
      }
    } else {
      if (VEC) {
        stream_store(u32x4{f[0], f[1], f[2], f[3]}, reinterpret_cast<u32x4*>(orow + col0));
        stream_store(u32x4{f[4], f[5], f[6], f[7]}, reinterpret_cast<u32x4*>(orow + col0 + 4));
      } else {
        for (int i = 0; i < 8; i++)
          if (col0 + i < K) orow[col0 + i] = f[i];
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// Export: strided copy of the first ncols columns of each row.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void export_kernel(const uint8_t* __restrict__ src, int64_t src_ld,
                                                          uint8_t* __restrict__ dst, int64_t rows, int64_t ncols) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < ncols; j += (int64_t)gridDim.x * kThreads)
      dst[r * ncols + j] = src[r * src_ld + j];
  }
}

// ------------------------------------------------------------------------------------
// Host side: validation and launch
// ------------------------------------------------------------------------------------
constexpr int64_t kMaxSteps = (int64_t)1 << 31;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte range [lo, hi) of a [rows, cols] matrix with row stride ld elements of esize.
struct Range {
  uintptr_t lo, hi;
};
Range matrix_range(const void* p, int64_t rows, int64_t cols, int64_t ld, size_t esize) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)(((rows - 1) * ld + cols) * (int64_t)esize)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int launch_status() {
  return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

int steps_for(int64_t rows, int64_t K, int64_t elems_per_step, uint32_t* per_row, uint32_t* total) {
  const int64_t spr = (K + elems_per_step - 1) / elems_per_step;
  if (rows > kMaxSteps / spr) return MXQ_ERR_SHAPE;
  *per_row = (uint32_t)spr;
  *total = (uint32_t)(rows * spr);
  return MXQ_OK;
}

uint32_t grid_for(uint32_t total_steps) { return (total_steps + kStepsPerWG - 1) / kStepsPerWG; }

int check_dtype(mxq_dtype dt) {
  return (dt == MXQ_BF16 || dt == MXQ_FP32) ? MXQ_OK : MXQ_ERR_DTYPE;
}
size_t dtype_size(mxq_dtype dt) { return dt == MXQ_BF16 ? 2 : 4; }

template <typename T>
int launch_proj(const void* x, int64_t ld_x, void* y, int64_t ld_y, int64_t rows, int64_t K, hipStream_t s) {
  uint32_t spr, total;
  if (steps_for(rows, K, StepGeom<T>::kElemsPerStep, &spr, &total)) return MXQ_ERR_SHAPE;
  constexpr int EPL = Fmt<T>::kEPL;
  const bool vec = aligned(x, 16) && aligned(y, 16) && ld_x % EPL == 0 && ld_y % EPL == 0 && K % EPL == 0;
  const dim3 grid(grid_for(total)), block(kThreads);
  if (vec)
    hipLaunchKernelGGL((proj_kernel<T, true>), grid, block, 0, s, (const T*)x, ld_x, (T*)y, ld_y, K, spr, total);
  else
    hipLaunchKernelGGL((proj_kernel<T, false>), grid, block, 0, s, (const T*)x, ld_x, (T*)y, ld_y, K, spr, total);
  return launch_status();
}

template <typename T>
int launch_row(const void* x, int64_t ld_x, int64_t rows, int64_t K, uint8_t* data, uint8_t* scale,
               int64_t scale_ld, hipStream_t s) {
  uint32_t spr, total;
  if (steps_for(rows, K, StepGeom<T>::kElemsPerStep, &spr, &total)) return MXQ_ERR_SHAPE;
  constexpr int EPL = Fmt<T>::kEPL;
  const bool vec = aligned(x, 16) && ld_x % EPL == 0 && K % EPL == 0 && aligned(data, EPL);
  const dim3 grid(grid_for(total)), block(kThreads);
  if (vec)
    hipLaunchKernelGGL((row_kernel<T, true>), grid, block, 0, s, (const T*)x, ld_x, K, data, scale, scale_ld, spr,
                       total);
  else
    hipLaunchKernelGGL((row_kernel<T, false>), grid, block, 0, s, (const T*)x, ld_x, K, data, scale, scale_ld, spr,
                       total);
  return launch_status();
}

template <typename T>
int launch_block128(const void* x, int64_t ld_x, int64_t rows, int64_t K, uint8_t* data, uint8_t* tile_code,
                    int64_t tile_ld, hipStream_t s) {
  const int64_t tpr = (K + 127) / 128, tiles = tpr * ((rows + 127) / 128);
  if (tiles >= kMaxSteps) return MXQ_ERR_SHAPE;
  constexpr int EPL = Fmt<T>::kEPL;
  const bool vec = aligned(x, 16) && ld_x % EPL == 0 && K % EPL == 0 && aligned(data, EPL);
  const dim3 grid((uint32_t)tiles), block(kThreads);
  if (vec)
    hipLaunchKernelGGL((block128_kernel<T, true>), grid, block, 0, s, (const T*)x, ld_x, rows, K, data, tile_code,
                       tile_ld, (uint32_t)tpr);
  else
    hipLaunchKernelGGL((block128_kernel<T, false>), grid, block, 0, s, (const T*)x, ld_x, rows, K, data, tile_code,
                       tile_ld, (uint32_t)tpr);
  return launch_status();
}

template <typename TO, bool kE5M2, bool kTile>
int launch_dequant_t(const uint8_t* data, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K, void* out,
                     int64_t ld_out, hipStream_t s) {
  uint32_t spr, total;
  if (steps_for(rows, K, 2048, &spr, &total)) return MXQ_ERR_SHAPE;
  constexpr int OPC = 16 / (int)sizeof(TO);   // output elements per 16-byte store
  const bool vec = aligned(data, 8) && K % 8 == 0 && aligned(out, 16) && ld_out % OPC == 0;
  const dim3 grid(grid_for(total)), block(kThreads);
  if (vec)
    hipLaunchKernelGGL((dequant_kernel<TO, kE5M2, kTile, true>), grid, block, 0, s, data, scale, scale_ld, K,
                       (TO*)out, ld_out, spr, total);
  else
    hipLaunchKernelGGL((dequant_kernel<TO, kE5M2, kTile, false>), grid, block, 0, s, data, scale, scale_ld, K,
                       (TO*)out, ld_out, spr, total);
  return launch_status();
}

template <typename TO>
int launch_dequant(const uint8_t* data, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K,
                   mxq_fp8 fmt, mxq_scale_layout lay, void* out, int64_t ld_out, hipStream_t s) {
  const bool e5 = fmt == MXQ_E5M2, tile = lay == MXQ_SCALE_TILE_128X128;
  if (e5 && tile) return launch_dequant_t<TO, true, true>(data, scale, scale_ld, rows, K, out, ld_out, s);
  if (e5) return launch_dequant_t<TO, true, false>(data, scale, scale_ld, rows, K, out, ld_out, s);
  if (tile) return launch_dequant_t<TO, false, true>(data, scale, scale_ld, rows, K, out, ld_out, s);
  return launch_dequant_t<TO, false, false>(data, scale, scale_ld, rows, K, out, ld_out, s);
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

int mxq_fake_quantize_mxfp4(const void* x, int64_t ld_x, void* y, int64_t ld_y, int64_t rows, int64_t K,
                            mxq_dtype dt, hipStream_t stream) {
  if (check_dtype(dt)) return MXQ_ERR_DTYPE;
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!x || !y) return MXQ_ERR_NULL;
  if (ld_x < K || ld_y < K) return MXQ_ERR_SHAPE;
  const size_t es = dtype_size(dt);
  const bool in_place = (x == y) && (ld_x == ld_y);
  if (!in_place && overlap(matrix_range(x, rows, K, ld_x, es), matrix_range(y, rows, K, ld_y, es)))
    return MXQ_ERR_ALIAS;
  return dt == MXQ_BF16 ? launch_proj<uint16_t>(x, ld_x, y, ld_y, rows, K, stream)
                        : launch_proj<uint32_t>(x, ld_x, y, ld_y, rows, K, stream);
}

int mxq_mxfp4_to_mxfp8_row(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt, uint8_t* data,
                           uint8_t* scale, int64_t scale_ld, hipStream_t stream) {
  if (check_dtype(dt)) return MXQ_ERR_DTYPE;
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!x || !data || !scale) return MXQ_ERR_NULL;
  const int64_t nb = (K + 31) / 32;
  if (ld_x < K || scale_ld < nb) return MXQ_ERR_SHAPE;
  const Range rx = matrix_range(x, rows, K, ld_x, dtype_size(dt)), rd = matrix_range(data, rows, K, K, 1),
              rs = matrix_range(scale, rows, nb, scale_ld, 1);
  if (overlap(rx, rd) || overlap(rx, rs) || overlap(rd, rs)) return MXQ_ERR_ALIAS;
  return dt == MXQ_BF16 ? launch_row<uint16_t>(x, ld_x, rows, K, data, scale, scale_ld, stream)
                        : launch_row<uint32_t>(x, ld_x, rows, K, data, scale, scale_ld, stream);
}

int mxq_mxfp4_to_fp8_block128(const void* x, int64_t ld_x, int64_t rows, int64_t K, mxq_dtype dt, uint8_t* data,
                              uint8_t* tile_code, int64_t tile_ld, hipStream_t stream) {
  if (check_dtype(dt)) return MXQ_ERR_DTYPE;
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!x || !data || !tile_code) return MXQ_ERR_NULL;
  const int64_t ntc = (K + 127) / 128, ntr = (rows + 127) / 128;
  if (ld_x < K || tile_ld < ntc) return MXQ_ERR_SHAPE;
  const Range rx = matrix_range(x, rows, K, ld_x, dtype_size(dt)), rd = matrix_range(data, rows, K, K, 1),
              rt = matrix_range(tile_code, ntr, ntc, tile_ld, 1);
  if (overlap(rx, rd) || overlap(rx, rt) || overlap(rd, rt)) return MXQ_ERR_ALIAS;
  return dt == MXQ_BF16 ? launch_block128<uint16_t>(x, ld_x, rows, K, data, tile_code, tile_ld, stream)
                        : launch_block128<uint32_t>(x, ld_x, rows, K, data, tile_code, tile_ld, stream);
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
  if (overlap(matrix_range(scale_storage, rows, nb, scale_ld, 1), matrix_range(scale_out, rows, nb, nb, 1)))
    return MXQ_ERR_ALIAS;
  const int64_t gx = (nb + kThreads - 1) / kThreads;
  const dim3 grid((uint32_t)(gx < 65535 ? gx : 65535), (uint32_t)(rows < 65535 ? rows : 65535)), block(kThreads);
  hipLaunchKernelGGL(export_kernel, grid, block, 0, stream, scale_storage, scale_ld, scale_out, rows, nb);
  return launch_status();
}

int mxq_dequantize(const uint8_t* data, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K,
                   mxq_fp8 fmt, mxq_scale_layout layout, void* out, int64_t ld_out, mxq_dtype out_dt,
                   hipStream_t stream) {
  if (check_dtype(out_dt)) return MXQ_ERR_DTYPE;
  if (fmt != MXQ_E4M3 && fmt != MXQ_E5M2) return MXQ_ERR_DTYPE;
  if (layout != MXQ_SCALE_ROW_1X32 && layout != MXQ_SCALE_TILE_128X128) return MXQ_ERR_DTYPE;
  if (rows < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!data || !scale || !out) return MXQ_ERR_NULL;
  const bool tile = layout == MXQ_SCALE_TILE_128X128;
  const int64_t srows = tile ? (rows + 127) / 128 : rows, scols = tile ? (K + 127) / 128 : (K + 31) / 32;
  if (ld_out < K || scale_ld < scols) return MXQ_ERR_SHAPE;
  const Range ro = matrix_range(out, rows, K, ld_out, dtype_size(out_dt));
  if (overlap(ro, matrix_range(data, rows, K, K, 1)) || overlap(ro, matrix_range(scale, srows, scols, scale_ld, 1)))
    return MXQ_ERR_ALIAS;
  return out_dt == MXQ_BF16 ? launch_dequant<uint16_t>(data, scale, scale_ld, rows, K, fmt, layout, out, ld_out, stream)
                            : launch_dequant<uint32_t>(data, scale, scale_ld, rows, K, fmt, layout, out, ld_out, stream);
}

}  // extern "C"
