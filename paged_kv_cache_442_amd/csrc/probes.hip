// Read-bandwidth probes for gfx950: what the memory system delivers to a kernel that only
// reads, for the access patterns of paged decode.  Measurement infrastructure (bench.py's
// ceilings), built into its own library (libpa_probe.so), not part of the attention path.
//
// A probe reads a list of tiles: tile t is tile_bytes contiguous bytes at
// base + ids[t] * tile_bytes.  With ids = 0, 1, 2, ... it is one contiguous stream; with a
// random permutation it is the paged pattern of the decode kernel (a tile per (block, KV
// head): 4 KiB at block size 16, bf16, head_dim 128) or, with 32 KiB tiles, the pattern of
// reading all 8 KV heads of a block as one run.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // loads in flight per thread per pass

// Thread g of the grid reads 16-byte chunks g, g + n, g + 2n, ... of the tile list (n =
// threads in the grid), kUnroll of them in flight at a time; consecutive threads read
// consecutive chunks of a tile.  The XOR of everything read decides a store that never
// happens in practice, so the loads cannot be dropped and nothing is written.
__global__ __launch_bounds__(kThreads) void read_tiles_kernel(const u32x4* __restrict__ base,
                                                              const int32_t* __restrict__ ids,
                                                              int64_t n_chunks, int32_t tile_shift,
                                                              uint32_t* sink) {
  const int64_t n = static_cast<int64_t>(gridDim.x) * kThreads;
  int64_t c = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t tile_mask = (int64_t{1} << tile_shift) - 1;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; c + (kUnroll - 1) * n < n_chunks; c += kUnroll * n) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t cc = c + u * n;
      const int64_t tile = ids[cc >> tile_shift];
      x[u] = __builtin_nontemporal_load(base + ((tile << tile_shift) | (cc & tile_mask)));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= x[u];
  }
  for (; c < n_chunks; c += n) {
    const int64_t tile = ids[c >> tile_shift];
    acc ^= __builtin_nontemporal_load(base + ((tile << tile_shift) | (c & tile_mask)));
  }
  const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == 0x9e3779b9u) sink[blockIdx.x] = r;
}

// Workgroup b reads whole tiles: U tiles at a time (tiles b * U .. b * U + U - 1, then the
// next U after the grid's), each thread one 16-byte chunk of each of the U tiles per pass,
// so a pass has U loads per thread in flight.  This is the decode kernel's way: a
// workgroup reads a whole tile, and the tiles of concurrent workgroups are far apart.
template <int U>
__global__ __launch_bounds__(kThreads) void read_tiles_wg_kernel(const u32x4* __restrict__ base,
                                                                 const int32_t* __restrict__ ids,
                                                                 int32_t n_tiles, int32_t tile_shift,
                                                                 uint32_t* sink) {
  const int64_t chunks = int64_t{1} << tile_shift;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t t0 = static_cast<int64_t>(blockIdx.x) * U; t0 < n_tiles;
       t0 += static_cast<int64_t>(gridDim.x) * U) {
    int64_t tile[U];
#pragma unroll
    for (int u = 0; u < U; ++u) tile[u] = t0 + u < n_tiles ? ids[t0 + u] : ids[t0];
    for (int64_t c = threadIdx.x; c < chunks; c += kThreads) {
      u32x4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(base + ((tile[u] << tile_shift) | c));
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= x[u];
    }
  }
  const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == 0x9e3779b9u) sink[blockIdx.x] = r;
}

}  // namespace

extern "C" {

// pa_probe_read_tiles with whole tiles per workgroup (read_tiles_wg_kernel): each of the
// `grid` workgroups reads `tiles_in_flight` (1, 2, 4 or 8) tiles at a time; tile_bytes a
// power of two >= 4096.  Same arguments, guarantee and results otherwise.  A tile past the
// list's end in the last group rereads the group's first tile.
int pa_probe_read_tiles_wg(const void* base, const int32_t* ids, int32_t n_tiles, int32_t tile_bytes,
                           int32_t grid, int32_t tiles_in_flight, uint32_t* sink, void* stream) {
  if (!base || !ids || !sink || n_tiles < 0 || grid < 1 || tile_bytes < 4096 ||
      (tile_bytes & (tile_bytes - 1)) != 0)
    return -1;
  if (n_tiles == 0) return 0;
  const int32_t shift = __builtin_ctz(static_cast<unsigned>(tile_bytes / 16));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* b = static_cast<const u32x4*>(base);
  (void)hipGetLastError();
  switch (tiles_in_flight) {
    case 1: hipLaunchKernelGGL(read_tiles_wg_kernel<1>, dim3(grid), dim3(kThreads), 0, s, b, ids, n_tiles, shift, sink); break;
    case 2: hipLaunchKernelGGL(read_tiles_wg_kernel<2>, dim3(grid), dim3(kThreads), 0, s, b, ids, n_tiles, shift, sink); break;
    case 4: hipLaunchKernelGGL(read_tiles_wg_kernel<4>, dim3(grid), dim3(kThreads), 0, s, b, ids, n_tiles, shift, sink); break;
    case 8: hipLaunchKernelGGL(read_tiles_wg_kernel<8>, dim3(grid), dim3(kThreads), 0, s, b, ids, n_tiles, shift, sink); break;
    default: return -1;
  }
  return static_cast<int>(hipGetLastError());
}


// Reads n_tiles tiles of tile_bytes (a power of two >= 16) at base + ids[t] * tile_bytes
// (ids: device int32 [n_tiles]; the caller guarantees every ids[t] * tile_bytes +
// tile_bytes <= the buffer's size) with `grid` workgroups of 256 threads; `sink` is a device
// buffer of at least `grid` uint32 that is written only if the data's XOR equals a fixed
// constant.  Asynchronous on `stream`.  Returns 0, or -1 for bad arguments, or the HIP
// error code of the launch.
int pa_probe_read_tiles(const void* base, const int32_t* ids, int32_t n_tiles, int32_t tile_bytes,
                        int32_t grid, uint32_t* sink, void* stream) {
  if (!base || !ids || !sink || n_tiles < 0 || grid < 1 || tile_bytes < 16 ||
      (tile_bytes & (tile_bytes - 1)) != 0)
    return -1;
  if (n_tiles == 0) return 0;
  const int32_t shift = __builtin_ctz(static_cast<unsigned>(tile_bytes / 16));
  const int64_t n_chunks = static_cast<int64_t>(n_tiles) * (tile_bytes / 16);
  (void)hipGetLastError();
  hipLaunchKernelGGL(read_tiles_kernel, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(base), ids,
                     n_chunks, shift, sink);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
