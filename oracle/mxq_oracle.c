/*
 * mxq_oracle.c -- plain CPU oracle for block-scaled MXFP4 weight quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only the
 * test suite, the smoke check and the bench's CPU-baseline leg may load it.  It
 * shares no code, header, table or constant with the HIP library and includes no
 * HIP header.
 *
 * Every value handled here is a dyadic rational (-1)^neg * M * 2^k with an
 * integer M, so every step below is exact integer arithmetic: no floating point
 * is used anywhere, and the results cannot depend on compiler flags or on the
 * host's denormal mode.
 *
 * Sources (the pages' text; cited by page title and section):
 *  [QAT]  "[PyTorch] MXFP4 weight QAT on MXFP8 and FP8 block-scaling recipes"
 *         (TransformerEngine PR 3264), sections Description (the two conversion
 *         modes), Test results (B200) and Known limitations.
 *  [EXP]  "MXFP8TensorStorage.export_components()" (TransformerEngine PR 3790),
 *         section Description.
 *
 * Where the pages leave a step open, the plainest reading is taken; each such
 * place says "Reading:" below.
 */
#include <stdint.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Dyadic numbers                                                            */
/* ------------------------------------------------------------------------ */

enum { CLS_FINITE = 0, CLS_INF = 1, CLS_NAN = 2 };

typedef struct {
  int neg;      /* sign bit */
  int cls;      /* CLS_FINITE / CLS_INF / CLS_NAN */
  uint64_t M;   /* magnitude significand (finite only) */
  int k;        /* magnitude = M * 2^k */
} dyadic;

static int bitlen(uint64_t M) {
  int n = 0;
  while (M) { n++; M >>= 1; }
  return n;
}

/* Exact comparison of |a| and |b| (both finite): -1, 0, +1. */
static int cmp_mag(dyadic a, dyadic b) {
  if (a.M == 0 || b.M == 0) return (a.M != 0) - (b.M != 0);
  int la = bitlen(a.M) + a.k, lb = bitlen(b.M) + b.k; /* value in [2^(l-1), 2^l) */
  if (la != lb) return la < lb ? -1 : 1;
  /* Same binade: bring both to the smaller exponent.  Equal top-bit positions
   * guarantee the shifted significand has at most 64 bits. */
  uint64_t A = a.M, B = b.M;
  if (a.k > b.k) A <<= (a.k - b.k); else B <<= (b.k - a.k);
  return (A > B) - (A < B);
}

/* IEEE binary formats used for inputs and outputs. */
typedef struct {
  int ebits, mbits, bias;
  int fn;   /* 1: "FN" finite-only format (E4M3FN: no Inf, NaN = all-ones) */
} fmt_t;

static const fmt_t FMT_BF16 = {8, 7, 127, 0};
static const fmt_t FMT_FP32 = {8, 23, 127, 0};
static const fmt_t FMT_E4M3 = {4, 3, 7, 1};
static const fmt_t FMT_E5M2 = {5, 2, 15, 0};

/* Bits -> dyadic, straight from the IEEE-754 layout. */
static dyadic unpack(uint32_t bits, fmt_t f) {
  dyadic d;
  uint32_t emask = (1u << f.ebits) - 1, mmask = (1u << f.mbits) - 1;
  uint32_t E = (bits >> f.mbits) & emask, m = bits & mmask;
  d.neg = (bits >> (f.ebits + f.mbits)) & 1;
  d.cls = CLS_FINITE;
  if (f.fn) {
    if (E == emask && m == mmask) { d.cls = CLS_NAN; d.M = 0; d.k = 0; return d; }
  } else if (E == emask) {
    d.cls = m ? CLS_NAN : CLS_INF; d.M = 0; d.k = 0; return d;
  }
  int emin = 1 - f.bias;
  if (E == 0) { d.M = m; d.k = emin - f.mbits; }
  else { d.M = ((uint64_t)1 << f.mbits) | m; d.k = (int)E - f.bias - f.mbits; }
  return d;
}

/*
 * Round (-1)^neg * M * 2^k to the nearest value of format f, ties to the even
 * significand (IEEE round-to-nearest-even), with gradual underflow.  Overflow:
 * IEEE formats give Inf; FN formats report it through *overflow (the callers
 * here never overflow an FN format and assert so).  *inexact tells whether
 * rounding changed the value.
 */
static uint32_t round_to_format(int neg, uint64_t M, int k, fmt_t f, int* inexact, int* overflow) {
  uint32_t sign = (uint32_t)(neg & 1) << (f.ebits + f.mbits);
  *inexact = 0; *overflow = 0;
  if (M == 0) return sign;
  int emin = 1 - f.bias;
  int L = bitlen(M) - 1 + k;                          /* value in [2^L, 2^(L+1)) */
  int qexp = (L < emin ? emin : L) - f.mbits;         /* exponent of one ulp there */
  int sh = qexp - k;
  uint64_t N;
  if (sh <= 0) {
    N = M << (-sh);                                   /* exact, |sh| <= mbits */
  } else if (sh >= 64) {
    N = 0; *inexact = 1;                              /* M < 2^63 < half an ulp */
  } else {
    uint64_t q = M >> sh, r = M - (q << sh), half = (uint64_t)1 << (sh - 1);
    if (r > half || (r == half && (q & 1))) q++;
    N = q; *inexact = (r != 0);
  }
  if (N >> (f.mbits + 1)) { N >>= 1; qexp++; }        /* carry into the next binade */
  uint32_t fe, fm;
  if (N >> f.mbits) { fe = (uint32_t)(qexp + f.mbits + f.bias); fm = (uint32_t)(N - ((uint64_t)1 << f.mbits)); }
  else { fe = 0; fm = (uint32_t)N; }                  /* subnormal (or zero) */
  uint32_t emask = (1u << f.ebits) - 1, mmask = (1u << f.mbits) - 1;
  if (f.fn) {
    if ((int)fe > (int)emask || (fe == emask && fm == mmask)) { *overflow = 1; return sign | (emask << f.mbits) | mmask; }
  } else if ((int)fe >= (int)emask) {
    *overflow = 1; return sign | (emask << f.mbits);  /* Inf */
  }
  return sign | (fe << f.mbits) | fm;
}

static void die(const char* what) {
  fprintf(stderr, "mxq oracle: internal invariant violated: %s\n", what);
  abort();
}

/* ------------------------------------------------------------------------ */
/* The MXFP4 decomposition ([QAT] Description, conversion mode 1)            */
/* ------------------------------------------------------------------------ */

/* E2M1 magnitudes, doubled so they are integers: {0, .5, 1, 1.5, 2, 3, 4, 6}.
 * The index is the 3-bit E2M1 code. */
static const int E2M1_X2[8] = {0, 1, 2, 3, 4, 6, 8, 12};

/* Scale exponent of one 1x32 block: e = clamp(ceil(log2(amax/6)), -126, 125),
 * i.e. the smallest integer e with 6 * 2^e >= amax, then clamped.
 * Reading: amax = 0 has log2 = -inf and clamps to -126. */
static int scale_exponent_clamped(dyadic amax, int lo, int hi);
static int orc_scale_exponent(dyadic amax) { return scale_exponent_clamped(amax, -126, 125); }

static int scale_exponent_clamped(dyadic amax, int lo, int hi) {
  int e;
  if (amax.M == 0) {
    e = -126;
  } else {
    /* amax >= 2^(l-1) with l = bitlen(M)+k, and 6*2^(l-4) < 2^(l-1), so the
     * answer is above l-4: walk up from there. */
    e = bitlen(amax.M) + amax.k - 4;
    for (;;) {
      dyadic six = {0, CLS_FINITE, 6, e};
      if (cmp_mag(six, amax) >= 0) break;
      e++;
    }
  }
  if (e < lo) e = lo;
  if (e > hi) e = hi;
  return e;
}

/* E2M1 code of |x| / 2^e rounded to the nearest grid point, ties to the even
 * code ([QAT] Description: round to nearest, ties to even, on E2M1).  Values above 6 have 6 as their
 * nearest grid point (the top scale saturates: [QAT] Known limitations). */
static int orc_e2m1_code(dyadic ax, int e) {
  if (ax.M == 0) return 0;
  int j = ax.k - e;                                     /* t = M * 2^j */
  int l = bitlen(ax.M) + j;                             /* t in [2^(l-1), 2^l) */
  if (l >= 4) return 7;                                 /* t >= 8: nearest is 6 */
  if (l <= -3) return 0;                                /* t < 1/8: nearest is 0 */
  /* t in [1/8, 8): T = t * 2^27 is an integer below 2^30. */
  int s = j + 27;
  uint64_t T = s >= 0 ? ax.M << s : ax.M >> (-s);
  if (s < 0 && ((ax.M >> (-s)) << (-s)) != ax.M) die("e2m1 scaling lost bits");
  int best = 0;
  uint64_t bestd = UINT64_MAX;
  for (int c = 0; c < 8; c++) {
    uint64_t g = (uint64_t)E2M1_X2[c] << 26;            /* grid value * 2^27 */
    uint64_t d = T > g ? T - g : g - T;
    if (d < bestd || (d == bestd && (c % 2 == 0))) { bestd = d; best = c; }
  }
  return best;
}

/* One 1x32 block (or a shorter last block) of a row: its amax, its poison flag
 * (any Inf or NaN in the block, [QAT] Test results: non-finite block poisoning),
 * and its scale exponent e. */
typedef struct { int poisoned; int e; } block_info;

static block_info analyse_block(const dyadic* v, int n) {
  block_info b = {0, -126};
  dyadic amax = {0, CLS_FINITE, 0, 0};
  for (int i = 0; i < n; i++) {
    if (v[i].cls != CLS_FINITE) { b.poisoned = 1; continue; }
    if (cmp_mag(v[i], amax) > 0) amax = v[i];
  }
  b.e = orc_scale_exponent(amax);
  return b;
}

static fmt_t dtype_fmt(int dtype) { return dtype == 0 ? FMT_BF16 : FMT_FP32; }

static uint32_t load_bits(const void* base, int dtype, size_t idx) {
  if (dtype == 0) return ((const uint16_t*)base)[idx];
  return ((const uint32_t*)base)[idx];
}
static void store_bits(void* base, int dtype, size_t idx, uint32_t v) {
  if (dtype == 0) ((uint16_t*)base)[idx] = (uint16_t)v;
  else ((uint32_t*)base)[idx] = v;
}
/* Reading: a poisoned block is written as the canonical positive quiet NaN. */
static uint32_t canonical_nan(int dtype) { return dtype == 0 ? 0x7FC0u : 0x7FC00000u; }

/* Status codes of the oracle's array functions. */
enum { ORC_OK = 0, ORC_BAD_ARG = 1 };

static int check_common(int64_t rows, int64_t K, int64_t ld, int dtype, int64_t r0, int64_t r1) {
  if (rows < 0 || K < 0 || ld < K || (dtype != 0 && dtype != 1)) return ORC_BAD_ARG;
  if (r0 < 0 || r1 > rows || r0 > r1) return ORC_BAD_ARG;
  return ORC_OK;
}

/* Read row r's block starting at column c0 (width n <= 32) into v. */
static void read_block(const void* x, int64_t ld, int dtype, int64_t r, int64_t c0, int n, dyadic* v) {
  fmt_t f = dtype_fmt(dtype);
  for (int i = 0; i < n; i++) v[i] = unpack(load_bits(x, dtype, (size_t)(r * ld + c0 + i)), f);
}

/*
 * Projection ([QAT] Description, mode 1): y = RTNE_E2M1(x / 2^e) * 2^e per 1x32
 * block, written in the input's dtype.  The last block of a row may be shorter
 * than 32 and keeps its own scale ([EXP] Description).  Rows [r0, r1) only.
 */
int orc_fake_quantize_mxfp4(const void* x, int64_t ld_x, void* y, int64_t ld_y,
                            int64_t rows, int64_t K, int dtype, int64_t r0, int64_t r1) {
  if (check_common(rows, K, ld_x, dtype, r0, r1) || ld_y < K) return ORC_BAD_ARG;
  fmt_t f = dtype_fmt(dtype);
  dyadic v[32];
  for (int64_t r = r0; r < r1; r++) {
    for (int64_t c0 = 0; c0 < K; c0 += 32) {
      int n = (int)(K - c0 < 32 ? K - c0 : 32);
      read_block(x, ld_x, dtype, r, c0, n, v);
      block_info b = analyse_block(v, n);
      for (int i = 0; i < n; i++) {
        uint32_t out;
        if (b.poisoned) {
          out = canonical_nan(dtype);
        } else {
          int c = orc_e2m1_code(v[i], b.e);
          int inexact, ovf;
          /* p * 2^e with p = E2M1_X2[c] / 2 */
          out = round_to_format(v[i].neg, (uint64_t)E2M1_X2[c], b.e - 1, f, &inexact, &ovf);
          if (inexact || ovf) die("projected value not representable in the input dtype");
        }
        store_bits(y, dtype, (size_t)(r * ld_y + c0 + i), out);
      }
    }
  }
  return ORC_OK;
}

/*
 * Direct MXFP8 rowwise lift ([QAT] Description, mode 2): the MXFP4
 * decomposition (p, e) of each block is written as E4M3 payload p * 2^6 with
 * scale 2^(e-6).  Where e-6 is below the smallest E8M0 scale 2^-127 the scale
 * is clamped to code 0 and the shift is absorbed exactly into the payload.
 * Reading: a poisoned block gets scale code 255 and payload 0x7F (both NaN).
 * Scale columns j >= ceil(K/32) of the padded storage are not written.
 */
int orc_mxfp4_to_mxfp8_row(const void* x, int64_t ld_x, int64_t rows, int64_t K, int dtype,
                           uint8_t* data, uint8_t* scale, int64_t scale_ld, int64_t r0, int64_t r1) {
  int64_t nb = (K + 31) / 32;
  if (check_common(rows, K, ld_x, dtype, r0, r1) || scale_ld < nb) return ORC_BAD_ARG;
  dyadic v[32];
  for (int64_t r = r0; r < r1; r++) {
    for (int64_t j = 0; j < nb; j++) {
      int64_t c0 = j * 32;
      int n = (int)(K - c0 < 32 ? K - c0 : 32);
      read_block(x, ld_x, dtype, r, c0, n, v);
      block_info b = analyse_block(v, n);
      if (b.poisoned) {
        scale[r * scale_ld + j] = 255;
        for (int i = 0; i < n; i++) data[r * K + c0 + i] = 0x7F;
        continue;
      }
      int S = b.e - 6;                 /* fixed shift 6 */
      if (S < -127) S = -127;          /* E8M0 code 0; the rest goes into the payload */
      scale[r * scale_ld + j] = (uint8_t)(S + 127);
      for (int i = 0; i < n; i++) {
        int c = orc_e2m1_code(v[i], b.e);
        int inexact, ovf;
        uint32_t q = round_to_format(v[i].neg, (uint64_t)E2M1_X2[c], b.e - 1 - S, FMT_E4M3, &inexact, &ovf);
        if (inexact || ovf) die("row lift is not exact");
        data[r * K + c0 + i] = (uint8_t)q;
      }
    }
  }
  return ORC_OK;
}

/*
 * Direct 128x128 blockwise FP8 ([QAT] Description, mode 2): per 128x128 tile,
 * M = the largest block exponent e among the tile's 1x32 blocks, tile scale
 * 2^S with S = max(M - 6, -127), and payload RTNE_E4M3(p * 2^(e - S)) including
 * E4M3 subnormals.
 * Readings: tiles are anchored at (0,0) and truncated at the edges; the tile
 * scale is stored as the E8M0 code S + 127; poisoned blocks do not take part in
 * M and their payload is 0x7F; a tile with no finite block has M = -126.
 * Processes the 128-row tile bands that start in [r0, r1) (r0 a multiple of 128).
 */
int orc_mxfp4_to_fp8_block128(const void* x, int64_t ld_x, int64_t rows, int64_t K, int dtype,
                              uint8_t* data, uint8_t* tile_code, int64_t tile_ld, int64_t r0, int64_t r1) {
  int64_t ntc = (K + 127) / 128;
  if (check_common(rows, K, ld_x, dtype, r0, r1) || tile_ld < ntc || (r0 % 128) != 0) return ORC_BAD_ARG;
  dyadic v[32];
  for (int64_t tr0 = r0; tr0 < r1; tr0 += 128) {
    int64_t tr1 = tr0 + 128 < rows ? tr0 + 128 : rows;
    for (int64_t tc = 0; tc < ntc; tc++) {
      int64_t tc0 = tc * 128, tc1 = tc0 + 128 < K ? tc0 + 128 : K;
      /* pass 1: the tile's largest finite block exponent */
      int M = -126;
      for (int64_t r = tr0; r < tr1; r++) {
        for (int64_t c0 = tc0; c0 < tc1; c0 += 32) {
          int n = (int)(K - c0 < 32 ? K - c0 : 32);
          read_block(x, ld_x, dtype, r, c0, n, v);
          block_info b = analyse_block(v, n);
          if (!b.poisoned && b.e > M) M = b.e;
        }
      }
      int S = M - 6;
      if (S < -127) S = -127;
      tile_code[(tr0 / 128) * tile_ld + tc] = (uint8_t)(S + 127);
      /* pass 2: fold every block's exponent into the tile scale */
      for (int64_t r = tr0; r < tr1; r++) {
        for (int64_t c0 = tc0; c0 < tc1; c0 += 32) {
          int n = (int)(K - c0 < 32 ? K - c0 : 32);
          read_block(x, ld_x, dtype, r, c0, n, v);
          block_info b = analyse_block(v, n);
          for (int i = 0; i < n; i++) {
            uint8_t q;
            if (b.poisoned) {
              q = 0x7F;
            } else {
              int c = orc_e2m1_code(v[i], b.e);
              int inexact, ovf;
              q = (uint8_t)round_to_format(v[i].neg, (uint64_t)E2M1_X2[c], b.e - 1 - S, FMT_E4M3, &inexact, &ovf);
              if (ovf) die("tile fold overflowed E4M3");   /* e - S <= 6 keeps p*2^(e-S) <= 384 */
            }
            data[r * K + c0 + i] = q;
          }
        }
      }
    }
  }
  return ORC_OK;
}

/*
 * MXFP8 columnwise from the decomposition ([QAT] Description, mode 2, and its
 * MXFP8 weight dataflow without a backward override): a fresh MXFP8
 * quantization, over 32x1 blocks (32 consecutive rows of one column), of the
 * projected weight y = p * 2^e, with the host quantizer's scale rule, so that
 * the bytes equal those the host quantizer makes from the projection (mode 1).
 *
 * Reading (the pages name the host amax rule but do not write it out): the OCP
 * MX rule, scale 2^S with S = floor(log2(amax)) - 8, 8 being E4M3's largest
 * exponent, raised to -127 where it falls below the E8M0 range; payload
 * RTNE_E4M3(y / 2^S) with subnormals.  On projected values amax has at most
 * two significant bits, so this S equals ceil(log2(amax / 448)) (the rule that
 * divides by E4M3's largest value) and y / 2^S <= 384 never saturates.
 * Readings: amax is over the block's finite values; an element of a poisoned
 * row block (NaN in y) gets payload 0x7F and takes no part in amax; a block with
 * no nonzero finite value gets code 0; blocks start at row 0 and the last one
 * may be short.  The code of row block j, column c, is scale[j*scale_ld + c].
 * Processes the row blocks that start in [r0, r1) (r0 a multiple of 32).
 */
int orc_mxfp4_to_mxfp8_col(const void* x, int64_t ld_x, int64_t rows, int64_t K, int dtype,
                           uint8_t* data, uint8_t* scale, int64_t scale_ld, int64_t r0, int64_t r1) {
  if (check_common(rows, K, ld_x, dtype, r0, r1) || scale_ld < K || (r0 % 32) != 0) return ORC_BAD_ARG;
  if (K == 0) return ORC_OK;
  /* the projected values of one 32-row band: |y| = M * 2^k, nan marks poison */
  typedef struct { int neg, nan; uint64_t M; int k; } yval;
  yval* y = (yval*)malloc(sizeof(yval) * 32 * (size_t)K);
  if (!y) die("out of memory");
  dyadic v[32];
  for (int64_t b0 = r0; b0 < r1; b0 += 32) {
    int64_t b1 = b0 + 32 < rows ? b0 + 32 : rows;
    /* step 1: the MXFP4 decomposition of every 1x32 row block in the band */
    for (int64_t r = b0; r < b1; r++) {
      for (int64_t c0 = 0; c0 < K; c0 += 32) {
        int n = (int)(K - c0 < 32 ? K - c0 : 32);
        read_block(x, ld_x, dtype, r, c0, n, v);
        block_info b = analyse_block(v, n);
        for (int i = 0; i < n; i++) {
          yval* t = &y[(r - b0) * K + c0 + i];
          t->neg = v[i].neg;
          t->nan = b.poisoned;
          t->M = (uint64_t)E2M1_X2[orc_e2m1_code(v[i], b.e)];   /* 2p */
          t->k = b.e - 1;
        }
      }
    }
    /* step 2: per column, the block's amax, its scale and the payloads */
    for (int64_t c = 0; c < K; c++) {
      dyadic amax = {0, CLS_FINITE, 0, 0};
      for (int64_t r = b0; r < b1; r++) {
        const yval* t = &y[(r - b0) * K + c];
        dyadic d = {t->neg, CLS_FINITE, t->M, t->k};
        if (!t->nan && cmp_mag(d, amax) > 0) amax = d;
      }
      int S = -127;
      if (amax.M != 0) {
        int fl = bitlen(amax.M) - 1 + amax.k;                   /* floor(log2(amax)) */
        S = fl - 8 < -127 ? -127 : fl - 8;
      }
      scale[(b0 / 32) * scale_ld + c] = (uint8_t)(S + 127);
      for (int64_t r = b0; r < b1; r++) {
        const yval* t = &y[(r - b0) * K + c];
        uint8_t q = 0x7F;
        if (!t->nan) {
          int inexact, ovf;
          q = (uint8_t)round_to_format(t->neg, t->M, t->k - S, FMT_E4M3, &inexact, &ovf);
          if (ovf) die("columnwise payload overflowed E4M3");
        }
        data[r * K + c] = q;
      }
    }
  }
  free(y);
  return ORC_OK;
}

/*
 * Unpadded export ([EXP] Description): scale_inv has shape (rows, ceil(K/32)),
 * taken from the first ceil(K/32) columns of storage whose row stride is
 * scale_ld; the payload bytes are the data itself.
 */
int orc_export_mxfp8(const uint8_t* scale_storage, int64_t rows, int64_t K, int64_t scale_ld, uint8_t* scale_out) {
  int64_t nb = (K + 31) / 32;
  if (rows < 0 || K < 0 || scale_ld < nb) return ORC_BAD_ARG;
  for (int64_t r = 0; r < rows; r++)
    for (int64_t j = 0; j < nb; j++) scale_out[r * nb + j] = scale_storage[r * scale_ld + j];
  return ORC_OK;
}

/*
 * Decode: value = FP8(q) * 2^(c - 127) rounded (nearest-even) to the output
 * dtype.  E8M0 code 0 is 2^-127 and code 255 is NaN ([QAT] Description, the
 * E8M0 decode fix; Test results: planted extreme scale codes).  A NaN payload
 * also decodes to NaN.  Reading: NaN is written as the canonical quiet NaN.
 * layout 0: one code per 1x32 block of a row (scale[r*scale_ld + col/32]);
 * layout 1: one code per 128x128 tile (scale[(r/128)*scale_ld + col/128]);
 * layout 2: one code per 32x1 block of a column (scale[(r/32)*scale_ld + col]).
 * fp8 0: E4M3 (FN); fp8 1: E5M2 (IEEE, with Inf).
 */
int orc_dequantize(const uint8_t* data, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K,
                   int fp8, int layout, void* out, int64_t ld_out, int dtype, int64_t r0, int64_t r1) {
  if (rows < 0 || K < 0 || ld_out < K || (dtype != 0 && dtype != 1) || (fp8 != 0 && fp8 != 1) ||
      layout < 0 || layout > 2 || r0 < 0 || r1 > rows || r0 > r1) return ORC_BAD_ARG;
  int64_t ncols = layout == 0 ? (K + 31) / 32 : layout == 1 ? (K + 127) / 128 : K;
  if (scale_ld < ncols) return ORC_BAD_ARG;
  fmt_t f = dtype_fmt(dtype), pf = fp8 == 0 ? FMT_E4M3 : FMT_E5M2;
  for (int64_t r = r0; r < r1; r++) {
    for (int64_t col = 0; col < K; col++) {
      uint8_t c = layout == 0   ? scale[r * scale_ld + col / 32]
                  : layout == 1 ? scale[(r / 128) * scale_ld + col / 128]
                                : scale[(r / 32) * scale_ld + col];
      dyadic q = unpack(data[r * K + col], pf);
      uint32_t o;
      if (c == 255 || q.cls == CLS_NAN) {
        o = canonical_nan(dtype);
      } else if (q.cls == CLS_INF) {
        o = ((uint32_t)q.neg << (f.ebits + f.mbits)) | (((1u << f.ebits) - 1) << f.mbits);
      } else {
        int inexact, ovf;
        o = round_to_format(q.neg, q.M, q.k + (int)c - 127, f, &inexact, &ovf);
      }
      store_bits(out, dtype, (size_t)(r * ld_out + col), o);
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Packed MXFP4 (the deployment format)                                      */
/* ------------------------------------------------------------------------ */
/*
 * Quantize for deployment: E2M1 payloads and 1x32 power-of-two E8M0 scales
 * ([QAT] Description: the weight training sees is the deployed one, E2M1
 * payloads with one power-of-two UE8M0 scale per 1x32 block; [ISS]
 * Description, workflow 2).  The MXFP4 decomposition is the projection's,
 * except that above the cap the scale moves to 2^126 ([QAT] Known
 * limitations): e = clamp(ceil(log2(amax/6)), -126, 126).  Code = e + 127.
 * Packing: element 2i in the low nibble of byte i, 2i+1 in the high nibble
 * (0 when K is odd); rows are ceil(K/2) bytes, contiguous.
 * Readings: the lower clamp stays at -126 (so the decoded deployment weight is
 * exactly the projection below the cap); a poisoned block gets code 255 (NaN)
 * and zero nibbles.
 */
int orc_quantize_mxfp4(const void* x, int64_t ld_x, int64_t rows, int64_t K, int dtype,
                       uint8_t* packed, uint8_t* scale, int64_t scale_ld, int64_t r0, int64_t r1) {
  int64_t nb = (K + 31) / 32, pw = (K + 1) / 2;
  if (check_common(rows, K, ld_x, dtype, r0, r1) || scale_ld < nb) return ORC_BAD_ARG;
  fmt_t f = dtype_fmt(dtype);
  for (int64_t r = r0; r < r1; r++) {
    for (int64_t i = 0; i < pw; i++) packed[r * pw + i] = 0;
    for (int64_t j = 0; j < nb; j++) {
      int64_t c0 = j * 32;
      int n = (int)(K - c0 < 32 ? K - c0 : 32);
      dyadic v[32];
      int poisoned = 0;
      dyadic amax = {0, CLS_FINITE, 0, 0};
      for (int i = 0; i < n; i++) {
        v[i] = unpack(load_bits(x, dtype, (size_t)(r * ld_x + c0 + i)), f);
        if (v[i].cls != CLS_FINITE) poisoned = 1;
        else if (cmp_mag(v[i], amax) > 0) amax = v[i];
      }
      if (poisoned) { scale[r * scale_ld + j] = 255; continue; }
      int e = scale_exponent_clamped(amax, -126, 126);
      scale[r * scale_ld + j] = (uint8_t)(e + 127);
      for (int i = 0; i < n; i++) {
        uint8_t nib = (uint8_t)((v[i].neg << 3) | orc_e2m1_code(v[i], e));
        int64_t col = c0 + i;
        packed[r * pw + col / 2] |= (uint8_t)(nib << (4 * (col % 2)));
      }
    }
  }
  return ORC_OK;
}

/* E2M1 nibble of element col of a packed row, as (neg, 2p). */
static void packed_element(const uint8_t* packed, int64_t pw, int64_t r, int64_t col, int* neg, int* twice_p) {
  uint8_t nib = (uint8_t)((packed[r * pw + col / 2] >> (4 * (col % 2))) & 0xF);
  *neg = nib >> 3;
  *twice_p = E2M1_X2[nib & 7];
}

/* Decode packed MXFP4: value = E2M1 * 2^(code - 127), nearest-even into the
 * output dtype (Inf beyond its range); code 255 gives canonical NaN. */
int orc_dequantize_mxfp4(const uint8_t* packed, const uint8_t* scale, int64_t scale_ld, int64_t rows, int64_t K,
                         void* out, int64_t ld_out, int dtype, int64_t r0, int64_t r1) {
  int64_t pw = (K + 1) / 2, nb = (K + 31) / 32;
  if (rows < 0 || K < 0 || ld_out < K || scale_ld < nb || (dtype != 0 && dtype != 1) || r0 < 0 || r1 > rows || r0 > r1)
    return ORC_BAD_ARG;
  fmt_t f = dtype_fmt(dtype);
  for (int64_t r = r0; r < r1; r++) {
    for (int64_t col = 0; col < K; col++) {
      uint8_t c = scale[r * scale_ld + col / 32];
      uint32_t o;
      if (c == 255) {
        o = canonical_nan(dtype);
      } else {
        int neg, tp, inexact, ovf;
        packed_element(packed, pw, r, col, &neg, &tp);
        o = round_to_format(neg, (uint64_t)tp, (int)c - 127 - 1, f, &inexact, &ovf);
      }
      store_bits(out, dtype, (size_t)(r * ld_out + col), o);
    }
  }
  return ORC_OK;
}

/* Direct MXFP8 row lift from packed MXFP4: the same fixed-shift-6 lift as
 * orc_mxfp4_to_mxfp8_row, with (p, e) read from the packed payload and code
 * (e = code - 127).  Code 255 (NaN) gives code 255 and payload 0x7F. */
int orc_mxfp4_packed_to_mxfp8_row(const uint8_t* packed, const uint8_t* scale, int64_t scale_ld, int64_t rows,
                                  int64_t K, uint8_t* data, uint8_t* scale_out, int64_t scale_out_ld,
                                  int64_t r0, int64_t r1) {
  int64_t pw = (K + 1) / 2, nb = (K + 31) / 32;
  if (rows < 0 || K < 0 || scale_ld < nb || scale_out_ld < nb || r0 < 0 || r1 > rows || r0 > r1) return ORC_BAD_ARG;
  for (int64_t r = r0; r < r1; r++) {
    for (int64_t j = 0; j < nb; j++) {
      int64_t c0 = j * 32, c1 = c0 + 32 < K ? c0 + 32 : K;
      uint8_t c = scale[r * scale_ld + j];
      if (c == 255) {
        scale_out[r * scale_out_ld + j] = 255;
        for (int64_t col = c0; col < c1; col++) data[r * K + col] = 0x7F;
        continue;
      }
      int e = (int)c - 127, S = e - 6;
      if (S < -127) S = -127;
      scale_out[r * scale_out_ld + j] = (uint8_t)(S + 127);
      for (int64_t col = c0; col < c1; col++) {
        int neg, tp, inexact, ovf;
        packed_element(packed, pw, r, col, &neg, &tp);
        uint32_t q = round_to_format(neg, (uint64_t)tp, e - 1 - S, FMT_E4M3, &inexact, &ovf);
        if (inexact || ovf) die("packed row lift is not exact");
        data[r * K + col] = (uint8_t)q;
      }
    }
  }
  return ORC_OK;
}

/* Direct 128x128 blockwise FP8 from packed MXFP4: the same tile fold as
 * orc_mxfp4_to_fp8_block128 with (p, e) read from the packed form; blocks with
 * code 255 are the poisoned ones.  Bands starting in [r0, r1), r0 % 128 == 0. */
int orc_mxfp4_packed_to_fp8_block128(const uint8_t* packed, const uint8_t* scale, int64_t scale_ld, int64_t rows,
                                     int64_t K, uint8_t* data, uint8_t* tile_code, int64_t tile_ld,
                                     int64_t r0, int64_t r1) {
  int64_t pw = (K + 1) / 2, nb = (K + 31) / 32, ntc = (K + 127) / 128;
  if (rows < 0 || K < 0 || scale_ld < nb || tile_ld < ntc || r0 < 0 || r1 > rows || r0 > r1 || r0 % 128) return ORC_BAD_ARG;
  for (int64_t tr0 = r0; tr0 < r1; tr0 += 128) {
    int64_t tr1 = tr0 + 128 < rows ? tr0 + 128 : rows;
    for (int64_t tc = 0; tc < ntc; tc++) {
      int64_t jb0 = tc * 4, jb1 = jb0 + 4 < nb ? jb0 + 4 : nb;
      int M = -126;
      for (int64_t r = tr0; r < tr1; r++)
        for (int64_t j = jb0; j < jb1; j++) {
          uint8_t c = scale[r * scale_ld + j];
          if (c != 255 && (int)c - 127 > M) M = (int)c - 127;
        }
      int S = M - 6;
      if (S < -127) S = -127;
      tile_code[(tr0 / 128) * tile_ld + tc] = (uint8_t)(S + 127);
      for (int64_t r = tr0; r < tr1; r++)
        for (int64_t j = jb0; j < jb1; j++) {
          uint8_t c = scale[r * scale_ld + j];
          int64_t c0 = j * 32, c1 = c0 + 32 < K ? c0 + 32 : K;
          for (int64_t col = c0; col < c1; col++) {
            if (c == 255) { data[r * K + col] = 0x7F; continue; }
            int neg, tp, inexact, ovf;
            packed_element(packed, pw, r, col, &neg, &tp);
            uint32_t q = round_to_format(neg, (uint64_t)tp, (int)c - 127 - 1 - S, FMT_E4M3, &inexact, &ovf);
            if (ovf) die("packed tile fold overflowed E4M3");
            data[r * K + col] = (uint8_t)q;
          }
        }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Element-level entry points, so the pins can test each step on its own.    */
/* ------------------------------------------------------------------------ */

/* Scale exponent of a block whose amax has the given bits (dtype 0 bf16, 1 fp32). */
int orc_scale_exponent_bits(uint32_t amax_bits, int dtype) {
  dyadic a = unpack(amax_bits & (dtype == 0 ? 0x7FFFu : 0x7FFFFFFFu), dtype_fmt(dtype));
  if (a.cls != CLS_FINITE) return 999;
  return orc_scale_exponent(a);
}

/* E2M1 code of RTNE(|x| / 2^e) for the given element bits. */
int orc_e2m1_code_bits(uint32_t x_bits, int dtype, int e) {
  dyadic a = unpack(x_bits, dtype_fmt(dtype));
  if (a.cls != CLS_FINITE) return -1;
  return orc_e2m1_code(a, e);
}

/* Nearest-even rounding of (-1)^neg * M * 2^k to fmt_id (0 bf16, 1 fp32, 2 E4M3, 3 E5M2).
 * flags bit 0: inexact, bit 1: overflow. */
uint32_t orc_round_to_format(int neg, uint64_t M, int k, int fmt_id, int* flags) {
  fmt_t f = fmt_id == 0 ? FMT_BF16 : fmt_id == 1 ? FMT_FP32 : fmt_id == 2 ? FMT_E4M3 : FMT_E5M2;
  int inexact, ovf;
  uint32_t b = round_to_format(neg, M, k, f, &inexact, &ovf);
  if (flags) *flags = inexact | (ovf << 1);
  return b;
}

/* Bits of format fmt_id -> (neg, M, k, cls). */
void orc_unpack(uint32_t bits, int fmt_id, int* neg, uint64_t* M, int* k, int* cls) {
  fmt_t f = fmt_id == 0 ? FMT_BF16 : fmt_id == 1 ? FMT_FP32 : fmt_id == 2 ? FMT_E4M3 : FMT_E5M2;
  dyadic d = unpack(bits, f);
  *neg = d.neg; *M = d.M; *k = d.k; *cls = d.cls;
}
