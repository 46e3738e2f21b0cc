// Launcher for the chunked-prefill kernel (prefill.hip).  Host-side only; every pointer
// is device memory owned by the caller, the launch is asynchronous on `stream`.
// Argument checking happens in the C ABI layer (capi.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pa {

struct PrefillArgs {
  const void* q;              // [num_rows][Hq][128]
  const void* k_cache;        // one layer: [N][Hkv][bs][128]
  const void* v_cache;
  const int32_t* query_start; // [S + 1]
  const int32_t* tables;      // [S][max_blocks]
  const int32_t* ctx;         // [S]
  float* out;                 // [num_rows][Hq][128]
  int32_t num_rows, num_seqs, num_q_heads, num_kv_heads, max_blocks, num_blocks, block_size;
  int32_t block_shift;        // log2(block_size): block sizes are powers of two here
  int32_t max_context;
  float scale_log2;           // scale * log2(e)
};

// dtype: 1 fp16, 2 bf16; group = num_q_heads / num_kv_heads in {1, 2, 4, 8}.  The grid
// covers max_query_len rows of every sequence.
hipError_t launch_prefill(const PrefillArgs& a, int dtype, int group, int max_query_len,
                          hipStream_t s);

}  // namespace pa
