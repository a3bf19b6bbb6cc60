/*
 * A plain C caller of the library: no PyTorch, only the HIP runtime's C API and
 * include/mxq.h.  It runs the whole path on one bf16 weight read from a file --
 * projection, row lift into padded scale storage, export, 128x128 fold and both
 * decodes -- on a stream of its own, checks every status, and writes the outputs
 * to a file for the test (tests/test_gpu_c_caller.py) to compare with the oracle.
 * It also checks that argument errors come back as status codes before any
 * launch, and that the grouped row lift, decode and packed encode of two
 * weights give the single calls' bytes.
 *
 * usage: c_caller ROWS K SCALE_LD IN.bin OUT.bin
 *   IN.bin   ROWS*K bf16 bit patterns (uint16, little endian)
 *   OUT.bin  y (bf16), data, exported codes, tile payload, tile codes,
 *            row decode (bf16), tile decode (bf16), concatenated in that order
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mxq.h"

#define HIP_OK(call)                                                                    \
  do {                                                                                  \
    hipError_t e_ = (call);                                                             \
    if (e_ != hipSuccess) {                                                             \
      fprintf(stderr, "c_caller: %s failed: %s\n", #call, hipGetErrorString(e_));      \
      exit(2);                                                                          \
    }                                                                                   \
  } while (0)

#define MXQ_OK_OR_DIE(call)                                                             \
  do {                                                                                  \
    int s_ = (call);                                                                    \
    if (s_ != MXQ_OK) {                                                                 \
      fprintf(stderr, "c_caller: %s returned %d (%s)\n", #call, s_, mxq_status_string(s_)); \
      exit(3);                                                                          \
    }                                                                                   \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 6) {
    fprintf(stderr, "usage: %s ROWS K SCALE_LD IN.bin OUT.bin\n", argv[0]);
    return 1;
  }
  const int64_t rows = atoll(argv[1]), K = atoll(argv[2]), sld = atoll(argv[3]);
  const int64_t nb = (K + 31) / 32, tr = (rows + 127) / 128, tcn = (K + 127) / 128, n = rows * K;
  if (rows <= 0 || K <= 0 || sld < nb) {
    fprintf(stderr, "c_caller: bad shape\n");
    return 1;
  }

  uint16_t* hx = (uint16_t*)malloc((size_t)n * 2);
  FILE* f = fopen(argv[4], "rb");
  if (!hx || !f || fread(hx, 2, (size_t)n, f) != (size_t)n) {
    fprintf(stderr, "c_caller: cannot read %s\n", argv[4]);
    return 1;
  }
  fclose(f);

  /* Argument errors: status codes, nothing enqueued. */
  if (mxq_fake_quantize_mxfp4(NULL, K, NULL, K, rows, -1, MXQ_BF16, 0) != MXQ_ERR_SHAPE ||
      mxq_fake_quantize_mxfp4(hx, K, hx, K, rows, K, MXQ_FP16, 0) != MXQ_ERR_DTYPE ||
      mxq_export_mxfp8(NULL, NULL, rows, K, sld, NULL, 0) != MXQ_ERR_NO_ROWWISE_DATA ||
      strlen(mxq_status_string(MXQ_ERR_ALIAS)) == 0) {
    fprintf(stderr, "c_caller: argument checks did not return the documented codes\n");
    return 4;
  }

  void *x, *y, *dec_r, *dec_t;
  uint8_t *data, *scale, *comp, *bdata, *tc;
  HIP_OK(hipMalloc(&x, (size_t)n * 2));
  HIP_OK(hipMalloc(&y, (size_t)n * 2));
  HIP_OK(hipMalloc(&dec_r, (size_t)n * 2));
  HIP_OK(hipMalloc(&dec_t, (size_t)n * 2));
  HIP_OK(hipMalloc((void**)&data, (size_t)n));
  HIP_OK(hipMalloc((void**)&scale, (size_t)(rows * sld)));
  HIP_OK(hipMalloc((void**)&comp, (size_t)(rows * nb)));
  HIP_OK(hipMalloc((void**)&bdata, (size_t)n));
  HIP_OK(hipMalloc((void**)&tc, (size_t)(tr * tcn)));
  HIP_OK(hipMemcpy(x, hx, (size_t)n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(scale, 0, (size_t)(rows * sld)));

  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  MXQ_OK_OR_DIE(mxq_fake_quantize_mxfp4(x, K, y, K, rows, K, MXQ_BF16, s));
  MXQ_OK_OR_DIE(mxq_mxfp4_to_mxfp8_row(x, K, rows, K, MXQ_BF16, data, scale, sld, s));
  MXQ_OK_OR_DIE(mxq_export_mxfp8(data, scale, rows, K, sld, comp, s));
  MXQ_OK_OR_DIE(mxq_mxfp4_to_fp8_block128(x, K, rows, K, MXQ_BF16, bdata, tc, tcn, s));
  MXQ_OK_OR_DIE(mxq_dequantize(data, comp, nb, rows, K, MXQ_E4M3, MXQ_SCALE_ROW_1X32, dec_r, K, MXQ_BF16, s));
  MXQ_OK_OR_DIE(mxq_dequantize(bdata, tc, tcn, rows, K, MXQ_E4M3, MXQ_SCALE_TILE_128X128, dec_t, K, MXQ_BF16, s));
  /* The grouped row lift of two weights (the whole weight and its first half of
   * rows, read-only overlap is allowed) gives the single call's bytes. */
  const int64_t half = rows / 2 > 0 ? rows / 2 : 1;
  uint8_t *gdata[2], *gscale[2];
  for (int i = 0; i < 2; i++) {
    HIP_OK(hipMalloc((void**)&gdata[i], (size_t)n));
    HIP_OK(hipMalloc((void**)&gscale[i], (size_t)(rows * sld)));
    HIP_OK(hipMemset(gscale[i], 0, (size_t)(rows * sld)));
  }
  const mxq_row_group groups[2] = {{x, K, rows, K, gdata[0], gscale[0], sld}, {x, K, half, K, gdata[1], gscale[1], sld}};
  MXQ_OK_OR_DIE(mxq_mxfp4_to_mxfp8_row_grouped(groups, 2, MXQ_BF16, s));
  /* an overlap is refused: the payload written over the weight */
  if (mxq_mxfp4_to_mxfp8_row(x, K, rows, K, MXQ_BF16, (uint8_t*)x, scale, sld, s) != MXQ_ERR_ALIAS) {
    fprintf(stderr, "c_caller: an aliased output was not refused\n");
    return 4;
  }
  HIP_OK(hipStreamSynchronize(s));
  {
    uint8_t* a = (uint8_t*)malloc((size_t)n);
    uint8_t* b = (uint8_t*)malloc((size_t)n);
    const size_t sizes[2] = {(size_t)n, (size_t)(half * K)};
    for (int i = 0; i < 2; i++) {
      HIP_OK(hipMemcpy(a, data, sizes[i], hipMemcpyDeviceToHost));
      HIP_OK(hipMemcpy(b, gdata[i], sizes[i], hipMemcpyDeviceToHost));
      if (memcmp(a, b, sizes[i]) != 0) {
        fprintf(stderr, "c_caller: grouped row lift differs from the single call (weight %d)\n", i);
        return 5;
      }
      HIP_OK(hipMemcpy(a, scale, (size_t)((i ? half : rows) * sld), hipMemcpyDeviceToHost));
      HIP_OK(hipMemcpy(b, gscale[i], (size_t)((i ? half : rows) * sld), hipMemcpyDeviceToHost));
      if (memcmp(a, b, (size_t)((i ? half : rows) * sld)) != 0) {
        fprintf(stderr, "c_caller: grouped codes differ from the single call (weight %d)\n", i);
        return 5;
      }
    }
    /* grouped decode of the two row lifts, and grouped packed encode of the two weights */
    void *gdec[2], *sdec;
    uint8_t *gpk[2], *gps[2], *spk, *sps;
    const int64_t pw = (K + 1) / 2;
    HIP_OK(hipMalloc(&sdec, (size_t)n * 2));
    HIP_OK(hipMalloc((void**)&spk, (size_t)(rows * pw)));
    HIP_OK(hipMalloc((void**)&sps, (size_t)(rows * nb)));
    for (int i = 0; i < 2; i++) {
      HIP_OK(hipMalloc(&gdec[i], (size_t)n * 2));
      HIP_OK(hipMalloc((void**)&gpk[i], (size_t)(rows * pw)));
      HIP_OK(hipMalloc((void**)&gps[i], (size_t)(rows * nb)));
    }
    const mxq_dequant_group dg[2] = {{gdata[0], gscale[0], sld, rows, K, gdec[0], K},
                                     {gdata[1], gscale[1], sld, half, K, gdec[1], K}};
    const mxq_mxfp4_group qg[2] = {{x, K, rows, K, gpk[0], gps[0], nb}, {x, K, half, K, gpk[1], gps[1], nb}};
    MXQ_OK_OR_DIE(mxq_dequantize(data, scale, sld, rows, K, MXQ_E4M3, MXQ_SCALE_ROW_1X32, sdec, K, MXQ_BF16, s));
    MXQ_OK_OR_DIE(mxq_dequantize_grouped(dg, 2, MXQ_E4M3, MXQ_SCALE_ROW_1X32, MXQ_BF16, s));
    MXQ_OK_OR_DIE(mxq_quantize_mxfp4(x, K, rows, K, MXQ_BF16, spk, sps, nb, s));
    MXQ_OK_OR_DIE(mxq_quantize_mxfp4_grouped(qg, 2, MXQ_BF16, s));
    HIP_OK(hipStreamSynchronize(s));
    uint8_t* c = (uint8_t*)malloc((size_t)n * 2);
    uint8_t* d = (uint8_t*)malloc((size_t)n * 2);
    for (int i = 0; i < 2; i++) {
      const int64_t r = i ? half : rows;
      const void* pairs[3][2] = {{sdec, gdec[i]}, {spk, gpk[i]}, {sps, gps[i]}};
      const size_t len[3] = {(size_t)(r * K * 2), (size_t)(r * pw), (size_t)(r * nb)};
      for (int j = 0; j < 3; j++) {
        HIP_OK(hipMemcpy(c, pairs[j][0], len[j], hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(d, pairs[j][1], len[j], hipMemcpyDeviceToHost));
        if (memcmp(c, d, len[j]) != 0) {
          fprintf(stderr, "c_caller: grouped %s differs from the single call (weight %d)\n",
                  j == 0 ? "decode" : "packed encode", i);
          return 5;
        }
      }
    }
    free(c);
    free(d);
    HIP_OK(hipFree(sdec));
    HIP_OK(hipFree(spk));
    HIP_OK(hipFree(sps));
    for (int i = 0; i < 2; i++) {
      HIP_OK(hipFree(gdec[i]));
      HIP_OK(hipFree(gpk[i]));
      HIP_OK(hipFree(gps[i]));
    }
    free(a);
    free(b);
    for (int i = 0; i < 2; i++) {
      HIP_OK(hipFree(gdata[i]));
      HIP_OK(hipFree(gscale[i]));
    }
  }

  const size_t sizes[7] = {(size_t)n * 2, (size_t)n, (size_t)(rows * nb), (size_t)n, (size_t)(tr * tcn),
                           (size_t)n * 2, (size_t)n * 2};
  const void* bufs[7] = {y, data, comp, bdata, tc, dec_r, dec_t};
  FILE* o = fopen(argv[5], "wb");
  if (!o) {
    fprintf(stderr, "c_caller: cannot write %s\n", argv[5]);
    return 1;
  }
  for (int i = 0; i < 7; i++) {
    void* h = malloc(sizes[i]);
    HIP_OK(hipMemcpy(h, bufs[i], sizes[i], hipMemcpyDeviceToHost));
    if (fwrite(h, 1, sizes[i], o) != sizes[i]) {
      fprintf(stderr, "c_caller: short write\n");
      return 1;
    }
    free(h);
  }
  fclose(o);
  HIP_OK(hipStreamDestroy(s));
  HIP_OK(hipFree(x));
  HIP_OK(hipFree(y));
  HIP_OK(hipFree(dec_r));
  HIP_OK(hipFree(dec_t));
  HIP_OK(hipFree(data));
  HIP_OK(hipFree(scale));
  HIP_OK(hipFree(comp));
  HIP_OK(hipFree(bdata));
  HIP_OK(hipFree(tc));
  free(hx);
  printf("c_caller: ok\n");
  return 0;
}
