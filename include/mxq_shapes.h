/*
 * mxq_shapes.h -- access-shape reference kernels (libmxq_shapes.so), for measurement.
 *
 * Not part of the quantization path.  Each shape moves the bytes of one of
 * libmxq's kernels over a [rows, K] matrix of element_size-byte elements (2:
 * bf16, 4: fp32) in that kernel's access pattern -- lanes per workgroup, chunks
 * per lane, load and store widths, cache-policy bits, barrier -- with a few bit
 * operations in place of the quantization.  A kernel timed beside its shape
 * shows how much of its time its memory pattern accounts for on the machine
 * (the roofline measurement of the MXFP4-QAT page's "Test results (B200)"
 * kernel timings, re-done on MI355X).
 *
 * int mxq_shape_run(shape, element_size, in, out, codes, rows, K, stream)
 *   in     [rows, K] input elements, contiguous (MXQ_SHAPE_DECODE: [rows, K] payload bytes;
 *          MXQ_SHAPE_PACKED_ROW: [rows, K / 2] packed bytes, element_size ignored)
 *   out    at least rows * K * element_size bytes
 *   codes  at least max(rows * K / 32, rows * K / 16384) bytes (code bytes the shape writes or reads)
 *   Returns 0 when launched, 1 when the shape does not fit (sizes, pointers), 2 when the runtime
 *   refused the launch.  Each shape needs whole workgroups of work: COPY16: rows * K *
 *   element_size a multiple of 1024; ROW, ROW_CODES: a multiple of 8192; DECODE: rows * K a
 *   multiple of 64 * 16 / element_size; TILE*: rows and K multiples of 128; LINEAR_FOLD*:
 *   rows * K a multiple of 16384 (a tile's elements); PACKED_ROW: rows * K a multiple of 4096;
 *   READ: rows * K * element_size a multiple of 8192; WRITE: a multiple of 4096;
 *   TILE_LOADS, LINEAR_LOADS, TILE_STORES, LINEAR_STORES: as TILE*.
 *   The fold's workgroup (TILE*, LINEAR_FOLD*) is 512 lanes for element_size 2 and 1024 for 4,
 *   as in libmxq's fold.
 */
#ifndef MXQ_SHAPES_H
#define MXQ_SHAPES_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MXQ_SHAPE_COPY16 = 0,                 /* projection: 64 lanes, 16 B in, 16 B out (nt sc1) per lane */
  MXQ_SHAPE_ROW = 1,                    /* row lift payload: 256 lanes, two 16 B chunks in, 16/es B out (nt sc1) each */
  MXQ_SHAPE_ROW_CODES = 2,              /* ROW plus one code byte per 32 elements (sc1) */
  MXQ_SHAPE_DECODE = 3,                 /* row decode: 64 lanes, 16/es B + a code byte in, 16 B out (nt) */
  MXQ_SHAPE_TILE = 4,                   /* 128x128 fold: its workgroup per tile in its tile order, all loads,
                                           LDS max, barrier, stores */
  MXQ_SHAPE_TILE_NO_BARRIER = 5,        /* TILE without the workgroup-wide maximum (wave-wide only) */
  MXQ_SHAPE_LINEAR_FOLD = 6,            /* the fold's workgroup (lanes, chunks per lane) over a contiguous stream */
  MXQ_SHAPE_LINEAR_FOLD_NO_BARRIER = 7, /* LINEAR_FOLD without the barrier */
  MXQ_SHAPE_PACKED_ROW = 8,             /* row lift from packed MXFP4: 64 lanes x 4 steps, 8 B + a code byte in, 16 B
                                           out (nt sc1), gathered 4-byte code stores back over the codes read */
  MXQ_SHAPE_READ = 9,                   /* the machine's read-only stream: 64 lanes x 8 chunks of 16 B in (nt), none out */
  MXQ_SHAPE_WRITE = 10,                 /* the machine's write-only stream: 64 lanes x 4 chunks of 16 B out (nt sc1) */
  MXQ_SHAPE_TILE_LOADS = 11,            /* TILE's loads alone (its workgroup and tile order) */
  MXQ_SHAPE_LINEAR_LOADS = 12,          /* LINEAR_FOLD's loads alone */
  MXQ_SHAPE_TILE_STORES = 13,           /* TILE's stores alone */
  MXQ_SHAPE_LINEAR_STORES = 14          /* LINEAR_FOLD's stores alone */
};

int mxq_shape_run(int shape, int element_size, const void* in, void* out, void* codes, int64_t rows, int64_t K,
                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_SHAPES_H */
