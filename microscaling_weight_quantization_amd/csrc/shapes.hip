// shapes.hip -- access-shape reference kernels (measurement only; see include/mxq_shapes.h).
//
// Each kernel moves the bytes of one of libmxq's kernels over a [rows, K] matrix
// in the same access pattern -- the same lanes per workgroup, chunks per lane,
// load and store widths and cache-policy bits, the same barrier -- with a few
// bit operations in place of the quantization (every output byte depends on the
// loaded bytes, so no load can be dropped).  Timing a kernel beside its shape
// separates what the kernel's own instructions cost from what its memory
// pattern costs on the machine.  Nothing here is on the quantization path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_shapes.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// The fold's wave-wide maximum: DPP within each 16-lane row (pair swap, quad
// swap, half-row mirror, row mirror), then the four rows' maxima as scalars.
__device__ __forceinline__ uint32_t wave_max(uint32_t m) {
  m = max(m, dpp<0xB1>(m));
  m = max(m, dpp<0x4E>(m));
  m = max(m, dpp<0x141>(m));
  m = max(m, dpp<0x140>(m));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)m, 32), (uint32_t)__builtin_amdgcn_readlane((int)m, 48)));
}

// A 16-byte chunk folded to 16 / ES bytes (ES = 2: 8 bytes, ES = 4: 4 bytes).
template <int ES>
struct Narrow;
template <>
struct Narrow<2> {
  typedef u32x2 type;
  static __device__ __forceinline__ type of(u32x4 w, uint32_t m) { return u32x2{(w[0] ^ (w[1] << 1)) + m, w[2] ^ (w[3] << 1)}; }
};
template <>
struct Narrow<4> {
  typedef uint32_t type;
  static __device__ __forceinline__ type of(u32x4 w, uint32_t m) { return (w[0] ^ (w[1] << 1) ^ (w[2] << 2) ^ (w[3] << 3)) + m; }
};

template <int AUX = 2, typename V>
__device__ __forceinline__ void store_nt(V v, void* base, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, 0x00020000);
  if constexpr (sizeof(V) == 16) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, AUX);
  else if constexpr (sizeof(V) == 8) __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, AUX);
  else __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, AUX);
}

// The projection's pattern: 64-lane workgroups, one 16-byte chunk per lane in,
// one out (nt sc1 stores).  Workgroup b covers bytes [1024 b, 1024 b + 1024).
__global__ __launch_bounds__(64) void copy16_kernel(const u32x4* __restrict__ in, uint8_t* __restrict__ out) {
  const u32x4 w = __builtin_nontemporal_load(in + (uint64_t)blockIdx.x * 64 + threadIdx.x);
  store_nt<2 | 16>(w ^ 0x01010101u, out + (uint64_t)blockIdx.x * 1024, threadIdx.x * 16);
}

// The row lift's pattern: 256-lane workgroups, two 16-byte chunks per lane
// (chunks l and 256 + l of the workgroup's 8 KB, both loaded before any store),
// 16 / ES bytes out per chunk (nt sc1); with CODES also one byte per 32
// elements (the lane that holds a block's first chunk), stored with the sc1 bit.
template <int ES, bool CODES>
__global__ __launch_bounds__(256) void row_kernel(const u32x4* __restrict__ in, uint8_t* __restrict__ out,
                                                  uint8_t* __restrict__ codes) {
  constexpr int kLanesPerBlock = 32 / (16 / ES);   // lanes holding one 32-element block: 4 (2-byte) or 8 (4-byte)
  const uint32_t t = threadIdx.x;
  u32x4 w[2];
#pragma unroll
  for (int u = 0; u < 2; u++) w[u] = __builtin_nontemporal_load(in + (uint64_t)blockIdx.x * 512 + u * 256 + t);
#pragma unroll
  for (int u = 0; u < 2; u++) {
    uint32_t m = max(max(w[u][0], w[u][1]), max(w[u][2], w[u][3])) >> 24;
    m = max(m, dpp<0xB1>(m));
    m = max(m, dpp<0x4E>(m));
    const uint32_t c = u * 256 + t;                 // the chunk within the workgroup
    store_nt<2 | 16>(Narrow<ES>::of(w[u], m), out + (uint64_t)blockIdx.x * (8192 / ES), c * (16 / ES));
    if (CODES && t % kLanesPerBlock == 0) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          codes + (uint64_t)blockIdx.x * (512 / kLanesPerBlock), 0, 0x7FFFFFFF, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)m, r, c / kLanesPerBlock, 0, 16);
    }
  }
}

// The row decode's pattern: 64-lane workgroups, 16 / ES payload bytes and one
// code byte per lane in, 16 bytes out (nt).
template <int ES>
__global__ __launch_bounds__(64) void decode_kernel(const uint8_t* __restrict__ in, const uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ out) {
  constexpr int kIn = 16 / ES;
  const uint32_t t = threadIdx.x;
  const uint64_t e0 = ((uint64_t)blockIdx.x * 64 + t) * (16 / ES);     // first element of the lane
  uint32_t a = 0, b = 0;
  if constexpr (kIn == 8) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(in + e0));
    a = v[0], b = v[1];
  } else {
    a = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(in + e0));
  }
  const uint32_t c = codes[e0 / 32];
  store_nt(u32x4{a + c, a >> 1, b ^ c, b >> 1}, out + (uint64_t)blockIdx.x * 1024, t * 16);
}

// The 128x128 fold's workgroup by element size: lanes per tile (512 for ES 2,
// 1024 for ES 4; 128 * ES / 16 lanes across a tile row, 16-byte chunks), and
// the tile order: the workgroups are dealt to the 8 XCDs in turn, and each run
// of 8 M workgroups is reordered so that XCD x takes M side-by-side tiles
// (M = 8 for ES 2, 4 for ES 4; the last, partial run keeps the plain order).
template <int ES>
struct FoldShape {
  static constexpr int kThreads = ES == 2 ? 512 : 1024;
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kRun = ES == 2 ? 8 : 4;
  static constexpr int kCPT = 128 * ES / 16;              // lanes across one tile row
  static constexpr int kRPP = kThreads / kCPT;            // tile rows per pass
  static constexpr int kP = 128 / kRPP;                   // chunks per lane
};
template <int M>
__device__ __forceinline__ uint32_t in_runs(uint32_t b, uint32_t n) {
  constexpr uint32_t G = 8u * M;
  if (b >= n - n % G) return b;
  const uint32_t r = b % G;
  return b - r + (r % 8u) * M + r / 8u;
}

// The 128x128 fold's pattern: one FoldShape workgroup per tile, in the fold's
// tile order, every chunk loaded first, the fold's wave maximum, a tile-wide
// maximum through LDS and a barrier (BARRIER), then 16 / ES bytes out per chunk
// and one byte per tile.
template <int ES, bool BARRIER>
__global__ __launch_bounds__(FoldShape<ES>::kThreads) void tile_kernel(const uint8_t* __restrict__ in, int64_t K,
                                                                    uint8_t* __restrict__ out,
                                                                    uint8_t* __restrict__ codes,
                                                                    uint32_t tiles_per_row) {
  using S = FoldShape<ES>;
  constexpr int CPT = S::kCPT, RPP = S::kRPP, P = S::kP;
  __shared__ uint32_t s_max[S::kWaves];
  const uint32_t t = threadIdx.x, bid = in_runs<S::kRun>(blockIdx.x, gridDim.x);
  const uint32_t tr = bid / tiles_per_row, tc = bid % tiles_per_row;
  const uint64_t r0 = (uint64_t)tr * 128 + t / CPT, c0 = (uint64_t)tc * 128 + (t % CPT) * (16 / ES);
  u32x4 w[P];
#pragma unroll
  for (int i = 0; i < P; i++)
    w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(in + ((r0 + i * RPP) * K + c0) * ES));
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < P; i++) m = max(m, max(max(w[i][0], w[i][1]), max(w[i][2], w[i][3])) >> 24);
  m = wave_max(m);
  if constexpr (BARRIER) {
    if ((t & 63u) == 0) s_max[t >> 6] = m;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < S::kWaves; v++) m = max(m, s_max[v]);
  }
#pragma unroll
  for (int i = 0; i < P; i++)   // stores off the band's first row (a base the whole workgroup shares)
    store_nt(Narrow<ES>::of(w[i], m), out + (uint64_t)tr * 128 * K, (uint32_t)((r0 - (uint64_t)tr * 128 + i * RPP) * K + c0));
  if (t == 0) codes[bid] = (uint8_t)m;
}

// The fold's workgroup (FoldShape: its lanes and chunks per lane, chunk l + i *
// lanes of the workgroup's 128 * 128 * ES bytes) over a plain contiguous stream
// in the plain order, with the same wave maximum, with or without the barrier:
// the tile shape's arithmetic and synchronization on linear addresses.
template <int ES, bool BARRIER>
__global__ __launch_bounds__(FoldShape<ES>::kThreads) void linear_kernel(const u32x4* __restrict__ in,
                                                                      uint8_t* __restrict__ out) {
  using S = FoldShape<ES>;
  constexpr int N = S::kThreads, P = S::kP;
  __shared__ uint32_t s_max[S::kWaves];
  const uint32_t t = threadIdx.x;
  const uint64_t c = (uint64_t)blockIdx.x * (N * P) + t;
  u32x4 w[P];
#pragma unroll
  for (int i = 0; i < P; i++) w[i] = __builtin_nontemporal_load(in + c + i * N);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < P; i++) m = max(m, max(max(w[i][0], w[i][1]), max(w[i][2], w[i][3])) >> 24);
  m = wave_max(m);
  if constexpr (BARRIER) {
    if ((t & 63u) == 0) s_max[t >> 6] = m;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < S::kWaves; v++) m = max(m, s_max[v]);
  }
  uint8_t* o = out + (uint64_t)blockIdx.x * (N * P) * (16 / ES);
#pragma unroll
  for (int i = 0; i < P; i++) store_nt(Narrow<ES>::of(w[i], m), o, (i * N + t) * (16 / ES));
}

// The fold's pattern split into its reads and its writes: the fold's workgroup
// and tile order (TILE) or the same workgroup over a contiguous stream, either
// only loading its chunks (their bits feed a test that practically never
// stores) or only storing 16 / ES bytes per chunk.  No reduction, no barrier.
template <int ES, bool TILE, bool LOAD>
__global__ __launch_bounds__(FoldShape<ES>::kThreads) void fold_io_kernel(const uint8_t* __restrict__ in, int64_t K,
                                                                       uint8_t* __restrict__ out,
                                                                       uint32_t tiles_per_row) {
  using S = FoldShape<ES>;
  constexpr int CPT = S::kCPT, RPP = S::kRPP, P = S::kP, N = S::kThreads;
  const uint32_t t = threadIdx.x, bid = TILE ? in_runs<S::kRun>(blockIdx.x, gridDim.x) : blockIdx.x;
  const uint32_t tr = bid / tiles_per_row, tc = bid % tiles_per_row;
  if constexpr (LOAD) {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < P; i++) {
      const uint64_t row = (uint64_t)tr * 128 + t / CPT + i * RPP, col = (uint64_t)tc * 128 + (t % CPT) * (16 / ES);
      const uint64_t off = TILE ? (row * K + col) * ES : ((uint64_t)bid * (N * P) + i * N + t) * 16;
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(in + off));
      x ^= w[0] ^ (w[1] << 1) ^ (w[2] << 2) ^ (w[3] << 3);
    }
    if (x == 0x9E3779B9u) reinterpret_cast<uint32_t*>(out)[bid] = x;
  } else {
    const u32x4 w = u32x4{t, bid, 0x01010101u, 0x02020202u};
#pragma unroll
    for (int i = 0; i < P; i++) {
      if constexpr (TILE)
        store_nt(Narrow<ES>::of(w, (uint32_t)i), out + (uint64_t)tr * 128 * K,
                 (uint32_t)((t / CPT + i * RPP) * K + (uint64_t)tc * 128 + (t % CPT) * (16 / ES)));
      else
        store_nt(Narrow<ES>::of(w, (uint32_t)i), out + (uint64_t)bid * (N * P) * (16 / ES), (i * N + t) * (16 / ES));
    }
  }
}

// The row lift from packed MXFP4's pattern: 64-lane workgroups of 4 steps
// (4096 elements of a row, one 128-byte line of codes), 8 packed bytes and one
// code byte (two lanes per code) in per lane per step, all loaded first; then
// per step 16 payload bytes out (nt sc1) and the codes of each 8 lanes gathered
// into one 4-byte store.  The gathered word is written back over the codes it
// was read from (the same bytes), so the shape needs no second code buffer.
__global__ __launch_bounds__(64) void packed_row_kernel(const u32x2* __restrict__ in, uint8_t* __restrict__ out,
                                                        uint8_t* __restrict__ codes) {
  const uint32_t t = threadIdx.x;
  uint8_t* const wcodes = codes + (uint64_t)blockIdx.x * 128;    // the workgroup's 128 codes
  u32x2 f[4];
  uint32_t c[4];
#pragma unroll
  for (int u = 0; u < 4; u++) {
    f[u] = __builtin_nontemporal_load(in + ((uint64_t)blockIdx.x * 4 + u) * 64 + t);
    c[u] = wcodes[u * 32 + t / 2];
  }
#pragma unroll
  for (int u = 0; u < 4; u++) {
    store_nt<2 | 16>(u32x4{f[u][0] ^ c[u], f[u][0] >> 4, f[u][1] + c[u], f[u][1] >> 4},
                     out + ((uint64_t)blockIdx.x * 4 + u) * 1024, t * 16);
    const uint32_t w = c[u] | (dpp<0x102>(c[u]) << 8) | (dpp<0x104>(c[u]) << 16) | (dpp<0x106>(c[u]) << 24);
    if (t % 8 == 0) store_nt<0>(w, wcodes, u * 32 + t / 2);
  }
}

int status() { return hipGetLastError() == hipSuccess ? 0 : 2; }

// The machine's plain streams, for scale: a read-only stream (64-lane
// workgroups, 8 chunks of 16 B per lane, nt; the loads feed a test that
// practically never stores) and a write-only one (4 chunks per lane, nt sc1).
// With one chunk per lane either is bound by how fast one-wave workgroups are
// dispatched, so they take several.
__global__ __launch_bounds__(64) void read_kernel(const u32x4* __restrict__ in, uint32_t* __restrict__ sink) {
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < 8; u++) {
    const u32x4 w = __builtin_nontemporal_load(in + ((uint64_t)blockIdx.x * 8 + u) * 64 + threadIdx.x);
    x ^= w[0] ^ (w[1] << 1) ^ (w[2] << 2) ^ (w[3] << 3);
  }
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}
__global__ __launch_bounds__(64) void write_kernel(uint8_t* __restrict__ out) {
  const u32x4 v = u32x4{blockIdx.x, threadIdx.x, 0x01010101u, 0x02020202u};
#pragma unroll
  for (int u = 0; u < 4; u++) store_nt<2 | 16>(v, out + ((uint64_t)blockIdx.x * 4 + u) * 1024, threadIdx.x * 16);
}

template <int ES>
int run(int shape, const void* in, void* out, void* codes, int64_t rows, int64_t K, hipStream_t s) {
  const int64_t bytes = rows * K * ES;                       // input bytes
  const uint32_t chunks = (uint32_t)(bytes / 16);
  switch (shape) {
    case MXQ_SHAPE_COPY16:
      if (bytes % 1024) return 1;
      hipLaunchKernelGGL(copy16_kernel, dim3(chunks / 64), dim3(64), 0, s, (const u32x4*)in, (uint8_t*)out);
      return status();
    case MXQ_SHAPE_ROW:
    case MXQ_SHAPE_ROW_CODES:
      if (bytes % 8192) return 1;
      if (shape == MXQ_SHAPE_ROW)
        hipLaunchKernelGGL((row_kernel<ES, false>), dim3(chunks / 512), dim3(256), 0, s, (const u32x4*)in,
                           (uint8_t*)out, (uint8_t*)codes);
      else
        hipLaunchKernelGGL((row_kernel<ES, true>), dim3(chunks / 512), dim3(256), 0, s, (const u32x4*)in,
                           (uint8_t*)out, (uint8_t*)codes);
      return status();
    case MXQ_SHAPE_DECODE:
      if ((rows * K) % (64 * (16 / ES))) return 1;
      hipLaunchKernelGGL((decode_kernel<ES>), dim3((uint32_t)(rows * K / (64 * (16 / ES)))), dim3(64), 0, s,
                         (const uint8_t*)in, (const uint8_t*)codes, (uint8_t*)out);
      return status();
    case MXQ_SHAPE_TILE:
    case MXQ_SHAPE_TILE_NO_BARRIER: {
      if (rows % 128 || K % 128 || 128 * K >= ((int64_t)1 << 31)) return 1;   // a band's payload: 32-bit offsets
      const uint32_t tpr = (uint32_t)(K / 128), tiles = (uint32_t)(rows / 128) * tpr;
      constexpr int N = FoldShape<ES>::kThreads;
      if (shape == MXQ_SHAPE_TILE)
        hipLaunchKernelGGL((tile_kernel<ES, true>), dim3(tiles), dim3(N), 0, s, (const uint8_t*)in, K, (uint8_t*)out,
                           (uint8_t*)codes, tpr);
      else
        hipLaunchKernelGGL((tile_kernel<ES, false>), dim3(tiles), dim3(N), 0, s, (const uint8_t*)in, K,
                           (uint8_t*)out, (uint8_t*)codes, tpr);
      return status();
    }
    case MXQ_SHAPE_LINEAR_FOLD:
    case MXQ_SHAPE_LINEAR_FOLD_NO_BARRIER: {
      constexpr int N = FoldShape<ES>::kThreads, PER = N * FoldShape<ES>::kP;   // chunks per workgroup
      if (chunks % PER) return 1;
      if (shape == MXQ_SHAPE_LINEAR_FOLD)
        hipLaunchKernelGGL((linear_kernel<ES, true>), dim3(chunks / PER), dim3(N), 0, s, (const u32x4*)in,
                           (uint8_t*)out);
      else
        hipLaunchKernelGGL((linear_kernel<ES, false>), dim3(chunks / PER), dim3(N), 0, s, (const u32x4*)in,
                           (uint8_t*)out);
      return status();
    }
    case MXQ_SHAPE_PACKED_ROW:
      if ((rows * K) % 4096) return 1;
      hipLaunchKernelGGL(packed_row_kernel, dim3((uint32_t)(rows * K / 4096)), dim3(64), 0, s, (const u32x2*)in,
                         (uint8_t*)out, (uint8_t*)codes);
      return status();
    case MXQ_SHAPE_TILE_LOADS:
    case MXQ_SHAPE_LINEAR_LOADS:
    case MXQ_SHAPE_TILE_STORES:
    case MXQ_SHAPE_LINEAR_STORES: {
      if (rows % 128 || K % 128 || 128 * K >= ((int64_t)1 << 31)) return 1;
      const uint32_t tpr = (uint32_t)(K / 128), tiles = (uint32_t)(rows / 128) * tpr;
      constexpr int N = FoldShape<ES>::kThreads;
      const uint8_t* i8 = (const uint8_t*)in;
      uint8_t* o8 = (uint8_t*)out;
      if (shape == MXQ_SHAPE_TILE_LOADS)
        hipLaunchKernelGGL((fold_io_kernel<ES, true, true>), dim3(tiles), dim3(N), 0, s, i8, K, o8, tpr);
      else if (shape == MXQ_SHAPE_LINEAR_LOADS)
        hipLaunchKernelGGL((fold_io_kernel<ES, false, true>), dim3(tiles), dim3(N), 0, s, i8, K, o8, tpr);
      else if (shape == MXQ_SHAPE_TILE_STORES)
        hipLaunchKernelGGL((fold_io_kernel<ES, true, false>), dim3(tiles), dim3(N), 0, s, i8, K, o8, tpr);
      else
        hipLaunchKernelGGL((fold_io_kernel<ES, false, false>), dim3(tiles), dim3(N), 0, s, i8, K, o8, tpr);
      return status();
    }
    case MXQ_SHAPE_READ:
      if (bytes % 8192) return 1;
      hipLaunchKernelGGL(read_kernel, dim3(chunks / 512), dim3(64), 0, s, (const u32x4*)in, (uint32_t*)out);
      return status();
    case MXQ_SHAPE_WRITE:
      if (bytes % 4096) return 1;
      hipLaunchKernelGGL(write_kernel, dim3(chunks / 256), dim3(64), 0, s, (uint8_t*)out);
      return status();
    default:
      return 1;
  }
}

}  // namespace

extern "C" int mxq_shape_run(int shape, int element_size, const void* in, void* out, void* codes, int64_t rows,
                             int64_t K, hipStream_t stream) {
  if (!in || !out || !codes || rows <= 0 || K <= 0 || rows * K >= ((int64_t)1 << 34)) return 1;
  if (element_size == 2) return run<2>(shape, in, out, codes, rows, K, stream);
  if (element_size == 4) return run<4>(shape, in, out, codes, rows, K, stream);
  return 1;
}
