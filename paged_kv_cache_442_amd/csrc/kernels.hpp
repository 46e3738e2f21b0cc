// Launchers for the gfx950 kernels (defined in kernels.hip).  Host-side only; every
// pointer is device memory owned by the caller, every launch is asynchronous on
// `stream`.  Argument checking happens in the C ABI layer (capi.cpp); these
// functions assume valid, supported arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pa {

constexpr int kHeadDim = 128;        // head_dim the attention kernels are built for
constexpr int kTileTokens = 16;      // tokens per K/V tile streamed by the decode kernel
constexpr int kDecodeWaves = 4;      // waves per decode workgroup
constexpr int kPlanThreads = 1024;
// A wave's tiles of one unit must fit one wave of lanes; a workgroup has four tile
// streams (four waves, each carrying its KV head's whole group of query heads).
constexpr int kMaxPartition = 4 * 64 * kTileTokens;

struct DecodeArgs {
  const void* q;            // [S][Hq][128]
  const void* k_cache;      // one layer: [N][Hkv][bs][128]
  const void* v_cache;
  const int32_t* tables;    // [S][max_blocks]
  const int32_t* ctx;       // [S]
  float* out;               // [S][Hq][128]
  float* part_o;            // [S][Hq][pmax][128]
  float* part_lse;          // [S][Hq][pmax], base-2 log-sum-exp of scaled scores
  int32_t* work_header;     // [0] work counter, [1] number of (item, KV head) work units
  int32_t* work_items;      // [S * pmax][4] (sequence, partition, context length, 0)
  int32_t num_seqs, num_q_heads, num_kv_heads, max_blocks, num_blocks, block_size;
  int32_t max_context, partition_tokens, pmax;
  int32_t window;           // attend to the last `window` tokens only; 0 = all
  float scale_log2;         // scale * log2(e) (times the K scale of an FP8 cache)
  float v_scale;            // V scale of an FP8 cache (1 otherwise)
};

// Bytes of the decode workspace the library holds itself, per GPU, for callers that
// cannot allocate (pa_cache_and_decode_static).
constexpr int64_t kStaticScratchBytes = int64_t{32} << 20;
// The current device's address of that workspace (looked up once per device).  Every call
// on a device shares it.
hipError_t static_scratch(void** ptr);

// The plan kernel lists the work items and zeroes the work counter; the partition
// kernel (persistent) needs a plan on the same workspace before it.
hipError_t launch_decode_plan(const DecodeArgs& a, hipStream_t s);
// dtype: 0 fp32, 1 fp16, 2 bf16, 3 fp8 e4m3 (bf16 queries); group = num_q_heads /
// num_kv_heads in {1, 2, 4, 8}.
hipError_t launch_decode_partitions(const DecodeArgs& a, int dtype, int group, hipStream_t s);
hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t s);

// New K/V rows [n_tokens][num_kv_heads][head_dim] written to their slots of one layer.
// A 16/32-bit pool copies the rows; an FP8 pool takes bf16 rows (head_dim 128) and
// quantizes them with the float32 reciprocals inv_k, inv_v of the layer's scales.
struct CacheWrite {
  const void* k;
  const void* v;
  const int64_t* slots;     // [n_tokens]; -1 (or out of range) skips the token
  void* k_cache;            // one layer: [N][Hkv][bs][head_dim]
  void* v_cache;
  int64_t total_chunks;     // 16-byte chunks of stored rows: n_tokens * Hkv * row_chunks
  int64_t num_slots;        // N * bs
  int32_t num_kv_heads, block_size, row_chunks;
  int32_t fp8;              // 1: quantizing FP8 write
  float inv_k, inv_v;
};

hipError_t launch_reshape_and_cache(const CacheWrite& w, hipStream_t s);
// One launch that does the cache write and the decode plan (launch_decode_plan's work).
hipError_t launch_cache_write_plan(const CacheWrite& w, const DecodeArgs& a, hipStream_t s);

// base: pool base, holding `arrays` (= 2 * num_layers) arrays, each of num_blocks blocks of
// block_bytes bytes (one layer's K or V part of a block).
// Whole-block copies between the device pool and a host swap space (pinned host memory
// addressed through its device mapping); pairs are device int32 [n_pairs][2].
hipError_t launch_swap_blocks(const int32_t* pairs, int32_t n_pairs, const void* src_base,
                              int32_t src_blocks, void* dst_base, int32_t dst_blocks, int32_t arrays,
                              int64_t block_bytes, hipStream_t s);
hipError_t launch_copy_blocks(const int32_t* pairs, int32_t n_pairs, void* base, int32_t arrays,
                              int32_t num_blocks, int64_t block_bytes, hipStream_t s);

}  // namespace pa
