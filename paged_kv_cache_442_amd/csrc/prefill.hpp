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
  float scale_log2;           // |scale| * log2(e), or log2(e) for a zero scale: always > 0
  // Applied to every dword of the query rows as (q & q_and) ^ q_xor: a negative scale
  // flips the queries' sign bits (scale q.k = |scale| (-q).k, exactly), a zero scale
  // clears them (every score 0, as scale q.k = 0).  The kernel's masking and running
  // maximum need a positive score scale.
  uint32_t q_and, q_xor;
  // Split of long key ranges: a row block's keys go in parts of part_keys (a multiple of
  // the 32-key tile); with more than one part each part writes its normalized output and
  // base-2 log-sum-exp here, and the merge kernel combines them into `out`.
  int32_t part_keys, pmax;
  float* part_o;              // [num_rows][Hq][pmax][128]
  float* part_lse;            // [num_rows][Hq][pmax]
  // Work list of the persistent kernel, written by the plan kernel: one queue per XCD,
  // each a run of units (sequence, KV head, row block, key part) longest first.
  int32_t* work_header;       // kPrefillHeaderBytes: per queue its start, length, claim counter
  int32_t* work_units;        // [work_cap][4]
  int32_t work_cap;           // units the list can hold
  int32_t row_blocks;         // row blocks per sequence covered: ceil(max_query_len / rows per block)
};

// (row, query head) columns per workgroup: 128 / group consecutive rows of one sequence
// times the group's query heads.
constexpr int kPrefillColumns = 128;

// Keys per part of the split (64 tiles): long enough to amortize a part's start and keep
// few rows to merge, short enough that no single unit outlasts the batch.  Measured on the
// mixed chunked-prefill batch (prefixes up to 4096 keys, chunks of 256-512 rows), plan,
// prefill and merge kernels together: 175 us at 2048-key parts, 181 at 1536, 178 at 3072,
// 210 at 4096.
constexpr int kPrefillPartKeys = 2048;

// Work queues of the persistent prefill kernel: one per XCD, so that the units of one
// (sequence, KV head), which read the same keys, share that XCD's L2.
constexpr int kPrefillQueues = 8;
// The work list's header: int32 [0, 8) the queues' starts in the unit list, [8, 16) their
// lengths, and queue x's claim counter at int32 kPrefillClaimStride * (x + 1), each counter
// in a 256-byte line of its own.
constexpr int kPrefillClaimStride = 64;
constexpr int64_t kPrefillHeaderBytes = 4 * kPrefillClaimStride * (kPrefillQueues + 1);

// Lists the units of the batch into work_header / work_units (one workgroup); the prefill
// kernel launched after it on the same stream claims them.  group as below.
hipError_t launch_prefill_plan(const PrefillArgs& a, int group, hipStream_t s);
// dtype: 1 fp16, 2 bf16; group = num_q_heads / num_kv_heads in {1, 2, 4, 8}.  Persistent:
// as many workgroups as the device holds at once, each claiming units until the queues
// are empty.
hipError_t launch_prefill(const PrefillArgs& a, int dtype, int group, hipStream_t s);
// Combines the parts of every row block that has more than one (nothing to do when
// pmax == 1); launched after launch_prefill on the same stream.
hipError_t launch_prefill_merge(const PrefillArgs& a, int group, int max_query_len, hipStream_t s);

}  // namespace pa
