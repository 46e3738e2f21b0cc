// C ABI of libpa (declared in include/pa.h): argument checking, the pool object and
// dispatch to the host block manager and the gfx950 kernels.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <limits>
#include <memory>
#include <string>
#include <vector>

#include "block_manager.hpp"
#include "kernels.hpp"
#include "prefill.hpp"
#include "preconditions.hpp"

// The debug build (-DPA_DEBUG, libpa_debug.so) checks the caller's slot and copy-pair
// preconditions on host copies of the device arrays before launching; the release build
// trusts them (a violation races on the device).
#ifdef PA_DEBUG
constexpr bool kDebugChecks = true;
#else
constexpr bool kDebugChecks = false;
#endif

struct pa_pool {
  pa_pool_desc desc;
  char* dev_base;  // NULL for a host-only pool
  int64_t dev_bytes;
  int64_t elem_bytes;
  int64_t array_bytes;  // one layer's K (or V): num_blocks * heads * block_size * head_dim * elem
  std::vector<float> k_scale, v_scale;  // per layer (FP8 caches; 1 by default)
  std::unique_ptr<pa::BlockManager> mgr;
};

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() { return PA_OK; }

int64_t elem_bytes_of(int32_t dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    case PA_FP8_E4M3: return 1;
    default: return 0;
  }
}

int check_desc(const pa_pool_desc* d) {
  if (!d) return fail(PA_E_INVAL, "desc is NULL");
  if (d->num_layers < 1 || d->num_blocks < 1 || d->block_size < 1 || d->num_kv_heads < 1 ||
      d->head_dim < 1)
    return fail(PA_E_INVAL, "desc fields must be >= 1 (layers %d blocks %d block_size %d heads %d dim %d)",
                d->num_layers, d->num_blocks, d->block_size, d->num_kv_heads, d->head_dim);
  if (elem_bytes_of(d->kv_dtype) == 0) return fail(PA_E_INVAL, "unknown kv_dtype %d", d->kv_dtype);
  return PA_OK;
}

// Bytes of one block in one layer's K (or V) array, with overflow checking.
bool array_block_bytes(const pa_pool_desc* d, int64_t* out) {
  __int128 b = static_cast<__int128>(d->num_kv_heads) * d->block_size * d->head_dim *
               elem_bytes_of(d->kv_dtype);
  if (b > std::numeric_limits<int64_t>::max() / 4) return false;
  *out = static_cast<int64_t>(b);
  return true;
}

int mgr_status(pa::MgrStatus st, const char* what) {
  switch (st) {
    case pa::MgrStatus::ok: return ok();
    case pa::MgrStatus::invalid: return fail(PA_E_INVAL, "%s: unknown or freed sequence, or bad count", what);
    case pa::MgrStatus::no_blocks: return fail(PA_E_NOMEM, "%s: not enough free blocks", what);
    case pa::MgrStatus::range: return fail(PA_E_RANGE, "%s: capacity exceeded", what);
  }
  return fail(PA_E_INVAL, "%s: unknown status", what);
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

int check_device_pool(const pa_pool* p, int32_t layer) {
  if (!p) return fail(PA_E_INVAL, "pool is NULL");
  if (!p->dev_base) return fail(PA_E_INVAL, "pool is host-only (no device memory bound)");
  if (layer < 0 || layer >= p->desc.num_layers)
    return fail(PA_E_INVAL, "layer %d outside [0, %d)", layer, p->desc.num_layers);
  return PA_OK;
}

// Workspace: [work header | work items | partition outputs | partition log-sum-exps].
constexpr int64_t kWorkHeaderBytes = 256;

// Default partition, measured best on the Llama-shaped layers.  Workgroups claim their
// next unit only near the end of the current one, so long units cost little at the end
// of the grid and the fixed cost of a unit (descriptor, query rows, the merge of its
// waves, the partial's write) decides.  The MFMA path (16-bit queries, groups of 4 or 8)
// has the larger fixed cost and takes long partitions: 4096 tokens with 16-bit K/V at
// groups of 8 (the Llama-3-70B layer's step 1.3% faster than at 2048), 2048 at groups of
// 4 and for e4m3 caches (4096 measured 17% and 14% slower there); the vector path takes
// 256 KiB of K and V per KV head (512 tokens of fp16/bf16, 1024 of e4m3, 256 of fp32).
int default_partition(int group, int elem_bytes) {
  if (elem_bytes == 2 && group == 8) return pa::kMaxPartition;
  if (elem_bytes <= 2 && group >= 4) return pa::kMaxPartition / 2;
  return 1024 / elem_bytes;
}

// A sliding window holds each sequence to at most `window` tokens, so long partitions
// leave too few units to balance the grid: windowed calls take at most 2048-token
// partitions by default (at a 4096-token window 0.706 of peak against 0.680 with 4096;
// at a 1024-token window 2048 and 4096 both make one unit of each sequence's window).
int default_window_partition(int group, int elem_bytes) {
  return std::min(default_partition(group, elem_bytes), pa::kMaxPartition / 2);
}

int64_t items_bytes(int64_t num_seqs, int64_t pmax) {
  return (num_seqs * pmax * 16 + 255) / 256 * 256;
}


struct DecodeCall {
  pa::DecodeArgs args;
  int group;
};

int prepare_decode(pa_pool* pool, int32_t layer, const void* q, int32_t num_seqs,
                   int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                   const int32_t* context_lens, int32_t max_context, float scale,
                   int32_t partition_tokens, float* out, void* workspace, int64_t workspace_bytes,
                   DecodeCall* call, int32_t window = 0) {
  if (window < 0) return fail(PA_E_INVAL, "window %d < 0", window);
  int st = check_device_pool(pool, layer);
  if (st) return st;
  const pa_pool_desc& d = pool->desc;
  if (num_seqs < 0 || num_q_heads < 1 || max_blocks < 0 || max_context < 0)
    return fail(PA_E_INVAL, "negative size (num_seqs %d num_q_heads %d max_blocks %d max_context %d)",
                num_seqs, num_q_heads, max_blocks, max_context);
  if (num_q_heads % d.num_kv_heads != 0)
    return fail(PA_E_INVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                d.num_kv_heads);
  const int group = num_q_heads / d.num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PA_E_UNSUPPORTED, "query group size %d (supported: 1, 2, 4, 8)", group);
  if (d.head_dim != pa::kHeadDim)
    return fail(PA_E_UNSUPPORTED, "head_dim %d (supported: %d)", d.head_dim, pa::kHeadDim);
  if (d.block_size % pa::kTileTokens != 0)
    return fail(PA_E_UNSUPPORTED, "block_size %d (must be a multiple of %d)", d.block_size,
                pa::kTileTokens);
  if (partition_tokens == 0)
    partition_tokens = window > 0 ? default_window_partition(group, static_cast<int>(pool->elem_bytes))
                                  : default_partition(group, static_cast<int>(pool->elem_bytes));
  if (partition_tokens < 0 || partition_tokens % (pa::kTileTokens * pa::kDecodeWaves) != 0 ||
      partition_tokens > pa::kMaxPartition)
    return fail(PA_E_INVAL, "partition_tokens %d must be a positive multiple of %d, at most %d",
                partition_tokens, pa::kTileTokens * pa::kDecodeWaves, pa::kMaxPartition);
  if (!std::isfinite(scale)) return fail(PA_E_INVAL, "scale is not finite");
  if (num_seqs == 0) {
    call->args = pa::DecodeArgs{};
    call->args.num_seqs = 0;
    call->group = group;
    return PA_OK;
  }
  if (!q || !block_tables || !context_lens || !out)
    return fail(PA_E_INVAL, "q, block_tables, context_lens and out must be non-NULL");
  if (num_seqs > 0x7fffffff / num_q_heads) return fail(PA_E_RANGE, "num_seqs * num_q_heads overflows");
  const int64_t pmax = std::max<int64_t>(1, (static_cast<int64_t>(max_context) + partition_tokens - 1) /
                                                partition_tokens);
  if (static_cast<int64_t>(num_seqs) * pmax * d.num_kv_heads > 0x7fffffff)
    return fail(PA_E_RANGE, "num_seqs * partitions * num_kv_heads exceeds 2^31 - 1");
  const int64_t need = pa_decode_workspace_bytes(pool, num_seqs, num_q_heads, max_context,
                                                 partition_tokens);
  if (need < 0) return static_cast<int>(need);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_E_RANGE, "workspace of %lld bytes is smaller than the %lld needed",
                static_cast<long long>(workspace_bytes), static_cast<long long>(need));
  for (const void* ptr : {q, static_cast<const void*>(out), static_cast<const void*>(workspace)})
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
      return fail(PA_E_INVAL, "q, out and workspace must be 16-byte aligned");

  pa::DecodeArgs& a = call->args;
  a.q = q;
  a.k_cache = pool->dev_base + static_cast<int64_t>(2 * layer) * pool->array_bytes;
  a.v_cache = pool->dev_base + static_cast<int64_t>(2 * layer + 1) * pool->array_bytes;
  a.tables = block_tables;
  a.ctx = context_lens;
  a.out = out;
  const int64_t rows = static_cast<int64_t>(num_seqs) * num_q_heads;
  char* ws = static_cast<char*>(workspace);
  a.work_header = reinterpret_cast<int32_t*>(ws);
  a.work_items = reinterpret_cast<int32_t*>(ws + kWorkHeaderBytes);
  a.part_o = reinterpret_cast<float*>(ws + kWorkHeaderBytes + items_bytes(num_seqs, pmax));
  a.part_lse = a.part_o + rows * pmax * pa::kHeadDim;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = d.num_kv_heads;
  a.max_blocks = max_blocks;
  a.num_blocks = d.num_blocks;
  a.block_size = d.block_size;
  a.max_context = max_context;
  a.partition_tokens = partition_tokens;
  a.pmax = static_cast<int32_t>(pmax);
  a.window = window;
  a.scale_log2 = scale * pool->k_scale[layer] * 1.4426950408889634f;
  a.v_scale = pool->v_scale[layer];
  call->group = group;
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return g_last_error.c_str(); }

int32_t pa_debug_build(void) { return kDebugChecks ? 1 : 0; }

int pa_check_slots(const int64_t* slots, int32_t n_tokens, int64_t num_slots) {
  if (n_tokens < 0 || (n_tokens > 0 && !slots)) return fail(PA_E_INVAL, "bad arguments");
  std::string why;
  if (!pa::slots_are_unique(slots, n_tokens, num_slots, &why)) return fail(PA_E_INVAL, "%s", why.c_str());
  return ok();
}

int pa_check_copy_pairs(const int32_t* pairs, int32_t n_pairs, int32_t num_blocks) {
  if (n_pairs < 0 || (n_pairs > 0 && !pairs)) return fail(PA_E_INVAL, "bad arguments");
  std::string why;
  if (!pa::copy_pairs_are_disjoint(pairs, n_pairs, num_blocks, &why))
    return fail(PA_E_INVAL, "%s", why.c_str());
  return ok();
}

int64_t pa_block_bytes(const pa_pool_desc* desc) {
  int st = check_desc(desc);
  if (st) return st;
  int64_t per_array;
  if (!array_block_bytes(desc, &per_array)) return fail(PA_E_RANGE, "block bytes overflow");
  __int128 b = static_cast<__int128>(per_array) * 2 * desc->num_layers;
  if (b > std::numeric_limits<int64_t>::max()) return fail(PA_E_RANGE, "block bytes overflow");
  return static_cast<int64_t>(b);
}

int64_t pa_pool_bytes(const pa_pool_desc* desc) {
  int64_t b = pa_block_bytes(desc);
  if (b < 0) return b;
  __int128 p = static_cast<__int128>(b) * desc->num_blocks;
  if (p > std::numeric_limits<int64_t>::max()) return fail(PA_E_RANGE, "pool bytes overflow");
  return static_cast<int64_t>(p);
}

int pa_alloc_pool(const pa_pool_desc* desc, void* dev_base, int64_t dev_bytes,
                  const int32_t* initial_free_order, pa_pool** out) {
  if (!out) return fail(PA_E_INVAL, "out is NULL");
  *out = nullptr;
  int st = check_desc(desc);
  if (st) return st;
  const int64_t need = pa_pool_bytes(desc);
  if (need < 0) return static_cast<int>(need);
  if (dev_base) {
    if (reinterpret_cast<uintptr_t>(dev_base) % 256 != 0)
      return fail(PA_E_INVAL, "dev_base must be 256-byte aligned");
    if (dev_bytes < need)
      return fail(PA_E_RANGE, "dev_bytes %lld < pool bytes %lld", static_cast<long long>(dev_bytes),
                  static_cast<long long>(need));
  } else if (dev_bytes != 0) {
    return fail(PA_E_INVAL, "dev_bytes must be 0 for a host-only pool");
  }
  std::vector<int32_t> order;
  if (initial_free_order) {
    order.assign(initial_free_order, initial_free_order + desc->num_blocks);
    std::vector<char> seen(desc->num_blocks, 0);
    for (int32_t b : order) {
      if (b < 0 || b >= desc->num_blocks || seen[b])
        return fail(PA_E_INVAL, "initial_free_order is not a permutation of 0..%d", desc->num_blocks - 1);
      seen[b] = 1;
    }
  }
  std::unique_ptr<pa_pool> p(new (std::nothrow) pa_pool);
  if (!p) return fail(PA_E_NOMEM, "host allocation failed");
  p->desc = *desc;
  p->dev_base = static_cast<char*>(dev_base);
  p->dev_bytes = dev_bytes;
  p->elem_bytes = elem_bytes_of(desc->kv_dtype);
  int64_t per_array_block;
  array_block_bytes(desc, &per_array_block);
  p->array_bytes = per_array_block * desc->num_blocks;
  p->k_scale.assign(desc->num_layers, 1.0f);
  p->v_scale.assign(desc->num_layers, 1.0f);
  p->mgr.reset(new (std::nothrow) pa::BlockManager(desc->num_blocks, desc->block_size, order));
  if (!p->mgr) return fail(PA_E_NOMEM, "host allocation failed");
  *out = p.release();
  return ok();
}

int pa_free_pool(pa_pool* pool) {
  delete pool;
  return ok();
}

int pa_pool_layer_ptrs(const pa_pool* pool, int32_t layer, void** k_base, void** v_base) {
  int st = check_device_pool(pool, layer);
  if (st) return st;
  if (!k_base || !v_base) return fail(PA_E_INVAL, "k_base and v_base must be non-NULL");
  *k_base = pool->dev_base + static_cast<int64_t>(2 * layer) * pool->array_bytes;
  *v_base = pool->dev_base + static_cast<int64_t>(2 * layer + 1) * pool->array_bytes;
  return ok();
}

int pa_seq_new(pa_pool* pool, int32_t* seq_out) {
  if (!pool || !seq_out) return fail(PA_E_INVAL, "pool and seq_out must be non-NULL");
  return mgr_status(pool->mgr->seq_new(seq_out), "pa_seq_new");
}

static int append_one(pa_pool* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens,
               int64_t* slots_out, int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow_out,
               const char* what) {
  if (!pool || !n_cow_out) return fail(PA_E_INVAL, "%s: pool and n_cow_out must be non-NULL", what);
  if (n_tokens > 0 && !slots_out) return fail(PA_E_INVAL, "%s: slots_out is NULL", what);
  if (cow_cap < 0 || (cow_cap > 0 && !cow_pairs_out))
    return fail(PA_E_INVAL, "%s: bad cow_pairs_out / cow_cap", what);
  int32_t dummy_pair[2];
  int32_t* pairs = cow_cap > 0 ? cow_pairs_out : dummy_pair;
  int32_t n_cow = 0;
  int st = mgr_status(pool->mgr->seq_append(seq, n_tokens, tokens, slots_out, pairs, cow_cap, &n_cow),
                      what);
  if (st == PA_OK) *n_cow_out = n_cow;
  return st;
}

static int append_batch(pa_pool* pool, const int32_t* seqs, int32_t count, const int32_t* n_tokens,
                 const int32_t* tokens, int64_t* slots_out, int32_t* cow_pairs_out, int32_t cow_cap,
                 int32_t* n_cow_out, const char* what) {
  if (!pool || !n_cow_out) return fail(PA_E_INVAL, "%s: pool and n_cow_out must be non-NULL", what);
  if (count < 0 || (count > 0 && (!seqs || !slots_out)))
    return fail(PA_E_INVAL, "%s: bad seqs / count / slots_out", what);
  if (cow_cap < 0 || (cow_cap > 0 && !cow_pairs_out))
    return fail(PA_E_INVAL, "%s: bad cow_pairs_out / cow_cap", what);
  int32_t dummy_pair[2];
  int32_t* pairs = cow_cap > 0 ? cow_pairs_out : dummy_pair;
  int32_t n_cow = 0;
  int st = mgr_status(pool->mgr->seq_append_batch(seqs, count, n_tokens, tokens, slots_out, pairs,
                                                  cow_cap, &n_cow),
                      what);
  if (st == PA_OK) *n_cow_out = n_cow;
  return st;
}

int pa_seq_append(pa_pool* pool, int32_t seq, int32_t n_tokens, int64_t* slots_out,
                  int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow_out) {
  return append_one(pool, seq, nullptr, n_tokens, slots_out, cow_pairs_out, cow_cap, n_cow_out,
                    "pa_seq_append");
}

int pa_seq_append_tokens(pa_pool* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens,
                         int64_t* slots_out, int32_t* cow_pairs_out, int32_t cow_cap,
                         int32_t* n_cow_out) {
  if (n_tokens > 0 && !tokens) return fail(PA_E_INVAL, "pa_seq_append_tokens: tokens is NULL");
  return append_one(pool, seq, tokens, n_tokens, slots_out, cow_pairs_out, cow_cap, n_cow_out,
                    "pa_seq_append_tokens");
}

int pa_seq_append_batch(pa_pool* pool, const int32_t* seqs, int32_t count, const int32_t* n_tokens,
                        int64_t* slots_out, int32_t* cow_pairs_out, int32_t cow_cap,
                        int32_t* n_cow_out) {
  return append_batch(pool, seqs, count, n_tokens, nullptr, slots_out, cow_pairs_out, cow_cap,
                      n_cow_out, "pa_seq_append_batch");
}

int pa_seq_append_batch_tokens(pa_pool* pool, const int32_t* seqs, int32_t count,
                               const int32_t* n_tokens, const int32_t* tokens, int64_t* slots_out,
                               int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow_out) {
  if (count > 0 && !tokens) return fail(PA_E_INVAL, "pa_seq_append_batch_tokens: tokens is NULL");
  return append_batch(pool, seqs, count, n_tokens, tokens, slots_out, cow_pairs_out, cow_cap,
                      n_cow_out, "pa_seq_append_batch_tokens");
}

int pa_pool_enable_prefix_caching(pa_pool* pool) {
  if (!pool) return fail(PA_E_INVAL, "pool is NULL");
  if (pool->mgr->enable_prefix_caching() != pa::MgrStatus::ok)
    return fail(PA_E_INVAL, "pa_pool_enable_prefix_caching: sequences are live");
  return ok();
}

int pa_seq_new_prefix(pa_pool* pool, const int32_t* prompt, int32_t n_prompt, int32_t* seq_out,
                      int32_t* n_cached_out) {
  if (!pool || !seq_out || !n_cached_out)
    return fail(PA_E_INVAL, "pool, seq_out and n_cached_out must be non-NULL");
  if (!pool->mgr->prefix_caching()) return fail(PA_E_INVAL, "pa_seq_new_prefix: prefix caching is off");
  if (n_prompt < 0 || (n_prompt > 0 && !prompt)) return fail(PA_E_INVAL, "pa_seq_new_prefix: bad prompt");
  return mgr_status(pool->mgr->seq_new_prefix(prompt, n_prompt, seq_out, n_cached_out),
                    "pa_seq_new_prefix");
}

int pa_seq_fork(pa_pool* pool, int32_t parent, int32_t* child_out) {
  if (!pool || !child_out) return fail(PA_E_INVAL, "pool and child_out must be non-NULL");
  return mgr_status(pool->mgr->seq_fork(parent, child_out), "pa_seq_fork");
}

int pa_seq_free(pa_pool* pool, int32_t seq) {
  if (!pool) return fail(PA_E_INVAL, "pool is NULL");
  return mgr_status(pool->mgr->seq_free(seq), "pa_seq_free");
}

int pa_seq_length(const pa_pool* pool, int32_t seq, int32_t* len_out) {
  if (!pool || !len_out) return fail(PA_E_INVAL, "pool and len_out must be non-NULL");
  if (!pool->mgr->live(seq)) return fail(PA_E_INVAL, "unknown or freed sequence %d", seq);
  *len_out = pool->mgr->length(seq);
  return ok();
}

int pa_export_block_tables(const pa_pool* pool, const int32_t* seqs, int32_t n, int32_t max_blocks,
                           int32_t* tables_out, int32_t* ctx_out) {
  if (!pool || n < 0 || max_blocks < 0) return fail(PA_E_INVAL, "bad pool, n or max_blocks");
  if (n > 0 && (!seqs || !ctx_out || (max_blocks > 0 && !tables_out)))
    return fail(PA_E_INVAL, "seqs, tables_out and ctx_out must be non-NULL");
  for (int32_t i = 0; i < n; ++i) {
    if (!pool->mgr->live(seqs[i])) return fail(PA_E_INVAL, "unknown or freed sequence %d", seqs[i]);
    if (pool->mgr->swapped(seqs[i])) return fail(PA_E_INVAL, "sequence %d is swapped out", seqs[i]);
    if (static_cast<int64_t>(pool->mgr->table(seqs[i]).size()) > max_blocks)
      return fail(PA_E_RANGE, "sequence %d holds %zu blocks > max_blocks %d", seqs[i],
                  pool->mgr->table(seqs[i]).size(), max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const std::vector<int32_t>& t = pool->mgr->table(seqs[i]);
    int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < static_cast<int32_t>(t.size()) ? t[j] : -1;
    ctx_out[i] = pool->mgr->length(seqs[i]);
  }
  return ok();
}

int pa_block_refcount(const pa_pool* pool, int32_t block, int32_t* rc_out) {
  if (!pool || !rc_out) return fail(PA_E_INVAL, "pool and rc_out must be non-NULL");
  if (block < 0 || block >= pool->desc.num_blocks) return fail(PA_E_INVAL, "block %d out of range", block);
  *rc_out = pool->mgr->refcount(block);
  return ok();
}

int pa_num_free_blocks(const pa_pool* pool, int32_t* n_out) {
  if (!pool || !n_out) return fail(PA_E_INVAL, "pool and n_out must be non-NULL");
  *n_out = pool->mgr->num_free();
  return ok();
}

int pa_block_state(const pa_pool* pool, int32_t block, int32_t* state_out) {
  if (!pool || !state_out) return fail(PA_E_INVAL, "pool and state_out must be non-NULL");
  if (block < 0 || block >= pool->desc.num_blocks) return fail(PA_E_INVAL, "block %d out of range", block);
  *state_out = static_cast<int32_t>(pool->mgr->state(block));
  return ok();
}

int pa_export_evictable(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!pool || !n_out || cap < 0 || (cap > 0 && !out)) return fail(PA_E_INVAL, "bad arguments");
  std::vector<int32_t> v;
  pool->mgr->evictable_lru_first(&v);
  *n_out = static_cast<int32_t>(v.size());
  if (static_cast<int64_t>(v.size()) > cap) return fail(PA_E_RANGE, "cap %d < %zu evictable blocks", cap, v.size());
  for (size_t i = 0; i < v.size(); ++i) out[i] = v[i];
  return ok();
}

int pa_export_free_stack(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!pool || !n_out || cap < 0 || (cap > 0 && !out)) return fail(PA_E_INVAL, "bad arguments");
  std::vector<int32_t> v;
  pool->mgr->free_stack_top_first(&v);
  *n_out = static_cast<int32_t>(v.size());
  if (static_cast<int64_t>(v.size()) > cap) return fail(PA_E_RANGE, "cap %d < %zu free blocks", cap, v.size());
  for (size_t i = 0; i < v.size(); ++i) out[i] = v[i];
  return ok();
}

// Debug build only: a host copy of a device array, ordered after the stream's earlier
// work (the call then waits for the stream).
extern "C++" {
template <class T>
static int fetch_to_host(const T* dev, int64_t n, hipStream_t s, std::vector<T>* host,
                         const char* what) {
  host->resize(static_cast<size_t>(n));
  if (n == 0) return PA_OK;
  hipError_t e = hipMemcpyAsync(host->data(), dev, static_cast<size_t>(n) * sizeof(T),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return hip_status(e, what);
}
}

// Debug build: the slots of a cache write are distinct (pa_check_slots).
static int debug_check_slots(const pa::CacheWrite& w, int32_t n_tokens, hipStream_t s,
                             const char* what) {
  if (!kDebugChecks || w.total_chunks == 0) return PA_OK;
  std::vector<int64_t> h;
  int st = fetch_to_host(w.slots, n_tokens, s, &h, what);
  if (st) return st;
  std::string why;
  if (!pa::slots_are_unique(h.data(), n_tokens, w.num_slots, &why))
    return fail(PA_E_INVAL, "%s: %s", what, why.c_str());
  return PA_OK;
}

// Checks a cache write's arguments and fills `w`; n_tokens == 0 gives total_chunks 0.
static int prepare_cache_write(pa_pool* pool, int32_t layer, const void* k, const void* v,
                               const int64_t* slots, int32_t n_tokens, pa::CacheWrite* w) {
  int st = check_device_pool(pool, layer);
  if (st) return st;
  if (n_tokens < 0) return fail(PA_E_INVAL, "n_tokens < 0");
  const int64_t row_bytes = static_cast<int64_t>(pool->desc.head_dim) * pool->elem_bytes;
  if (row_bytes % 16 != 0)
    return fail(PA_E_UNSUPPORTED, "head_dim * element bytes = %lld is not a multiple of 16",
                static_cast<long long>(row_bytes));
  const bool fp8 = pool->desc.kv_dtype == PA_FP8_E4M3;
  if (fp8 && pool->desc.head_dim != pa::kHeadDim)
    return fail(PA_E_UNSUPPORTED, "FP8 cache writes need head_dim %d", pa::kHeadDim);
  *w = pa::CacheWrite{};
  if (n_tokens == 0) return PA_OK;
  if (!k || !v || !slots) return fail(PA_E_INVAL, "k, v and slots must be non-NULL");
  if (reinterpret_cast<uintptr_t>(k) % 16 || reinterpret_cast<uintptr_t>(v) % 16)
    return fail(PA_E_INVAL, "k and v must be 16-byte aligned");
  void *kc, *vc;
  pa_pool_layer_ptrs(pool, layer, &kc, &vc);
  w->k = k;
  w->v = v;
  w->slots = slots;
  w->k_cache = kc;
  w->v_cache = vc;
  w->row_chunks = static_cast<int32_t>(row_bytes / 16);
  w->total_chunks = static_cast<int64_t>(n_tokens) * pool->desc.num_kv_heads * w->row_chunks;
  w->num_slots = static_cast<int64_t>(pool->desc.num_blocks) * pool->desc.block_size;
  w->num_kv_heads = pool->desc.num_kv_heads;
  w->block_size = pool->desc.block_size;
  w->fp8 = fp8 ? 1 : 0;
  w->inv_k = 1.0f / pool->k_scale[layer];
  w->inv_v = 1.0f / pool->v_scale[layer];
  return PA_OK;
}

int pa_reshape_and_cache(pa_pool* pool, int32_t layer, const void* k, const void* v,
                         const int64_t* slots, int32_t n_tokens, void* stream) {
  pa::CacheWrite w;
  int st = prepare_cache_write(pool, layer, k, v, slots, n_tokens, &w);
  if (st) return st;
  if (w.total_chunks == 0) return ok();
  st = debug_check_slots(w, n_tokens, static_cast<hipStream_t>(stream), "pa_reshape_and_cache");
  if (st) return st;
  return hip_status(pa::launch_reshape_and_cache(w, static_cast<hipStream_t>(stream)),
                    "pa_reshape_and_cache");
}

int pa_copy_blocks(pa_pool* pool, const int32_t* pairs, int32_t n_pairs, void* stream) {
  int st = check_device_pool(pool, 0);
  if (st) return st;
  if (n_pairs < 0) return fail(PA_E_INVAL, "n_pairs < 0");
  if (n_pairs == 0) return ok();
  if (!pairs) return fail(PA_E_INVAL, "pairs is NULL");
  if (2 * pool->desc.num_layers > 65535) return fail(PA_E_UNSUPPORTED, "too many layers");
  const int64_t block_bytes = pool->array_bytes / pool->desc.num_blocks;
  if (block_bytes % 16 != 0) return fail(PA_E_UNSUPPORTED, "per-layer block bytes not a multiple of 16");
  if (kDebugChecks) {
    std::vector<int32_t> h;
    st = fetch_to_host(pairs, 2 * static_cast<int64_t>(n_pairs), static_cast<hipStream_t>(stream), &h,
                       "pa_copy_blocks");
    if (st) return st;
    std::string why;
    if (!pa::copy_pairs_are_disjoint(h.data(), n_pairs, pool->desc.num_blocks, &why))
      return fail(PA_E_INVAL, "pa_copy_blocks: %s", why.c_str());
  }
  return hip_status(pa::launch_copy_blocks(pairs, n_pairs, pool->dev_base, 2 * pool->desc.num_layers,
                                           pool->desc.num_blocks, block_bytes,
                                           static_cast<hipStream_t>(stream)),
                    "pa_copy_blocks");
}

int32_t pa_decode_default_partition(const pa_pool* pool, int32_t num_q_heads) {
  if (!pool) return fail(PA_E_INVAL, "pool is NULL");
  const int32_t hkv = pool->desc.num_kv_heads;
  if (num_q_heads < 1 || num_q_heads % hkv != 0)
    return fail(PA_E_INVAL, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, hkv);
  return default_partition(num_q_heads / hkv, static_cast<int>(pool->elem_bytes));
}

int64_t pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_context, int32_t partition_tokens) {
  if (!pool) return fail(PA_E_INVAL, "pool is NULL");
  if (num_seqs < 0 || num_q_heads < 0 || max_context < 0 || partition_tokens < 0)
    return fail(PA_E_INVAL, "negative size");
  if (partition_tokens == 0) {
    // Sized for the smaller of the two defaults, so that it serves pa_decode and
    // pa_decode_window alike.
    const int32_t hkv = pool->desc.num_kv_heads;
    partition_tokens = default_window_partition(hkv > 0 ? num_q_heads / hkv : 1,
                                                static_cast<int>(pool->elem_bytes));
  }
  const int64_t pmax =
      std::max<int64_t>(1, (static_cast<int64_t>(max_context) + partition_tokens - 1) / partition_tokens);
  // Partials are needed only when a sequence can span more than one partition.
  const __int128 partials =
      pmax > 1 ? static_cast<__int128>(num_seqs) * num_q_heads * pmax * (pa::kHeadDim + 1) * 4 : 0;
  const __int128 b = kWorkHeaderBytes + items_bytes(num_seqs, pmax) + partials;
  if (b > std::numeric_limits<int64_t>::max()) return fail(PA_E_RANGE, "workspace size overflows");
  return static_cast<int64_t>(b);
}

int pa_decode_plan(pa_pool* pool, int32_t layer, const void* q, int32_t num_seqs,
                   int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                   const int32_t* context_lens, int32_t max_context, float scale,
                   int32_t partition_tokens, float* out, void* workspace, int64_t workspace_bytes,
                   void* stream) {
  DecodeCall c;
  int st = prepare_decode(pool, layer, q, num_seqs, num_q_heads, block_tables, max_blocks,
                          context_lens, max_context, scale, partition_tokens, out, workspace,
                          workspace_bytes, &c);
  if (st) return st;
  if (c.args.num_seqs == 0) return ok();
  return hip_status(pa::launch_decode_plan(c.args, static_cast<hipStream_t>(stream)), "pa_decode_plan");
}

int pa_decode_partitions(pa_pool* pool, int32_t layer, const void* q, int32_t num_seqs,
                         int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                         const int32_t* context_lens, int32_t max_context, float scale,
                         int32_t partition_tokens, float* out, void* workspace,
                         int64_t workspace_bytes, void* stream) {
  DecodeCall c;
  int st = prepare_decode(pool, layer, q, num_seqs, num_q_heads, block_tables, max_blocks,
                          context_lens, max_context, scale, partition_tokens, out, workspace,
                          workspace_bytes, &c);
  if (st) return st;
  if (c.args.num_seqs == 0) return ok();
  return hip_status(pa::launch_decode_partitions(c.args, static_cast<int>(pool->desc.kv_dtype), c.group,
                                                 static_cast<hipStream_t>(stream)),
                    "pa_decode_partitions");
}

int pa_decode_reduce(pa_pool* pool, int32_t layer, const void* q, int32_t num_seqs,
                     int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                     const int32_t* context_lens, int32_t max_context, float scale,
                     int32_t partition_tokens, float* out, void* workspace,
                     int64_t workspace_bytes, void* stream) {
  DecodeCall c;
  int st = prepare_decode(pool, layer, q, num_seqs, num_q_heads, block_tables, max_blocks,
                          context_lens, max_context, scale, partition_tokens, out, workspace,
                          workspace_bytes, &c);
  if (st) return st;
  if (c.args.num_seqs == 0 || c.args.pmax <= 1) return ok();
  return hip_status(pa::launch_decode_reduce(c.args, static_cast<hipStream_t>(stream)),
                    "pa_decode_reduce");
}

int pa_decode(pa_pool* pool, int32_t layer, const void* q, int32_t num_seqs, int32_t num_q_heads,
              const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
              int32_t max_context, float scale, int32_t partition_tokens, float* out,
              void* workspace, int64_t workspace_bytes, void* stream) {
  int st = pa_decode_plan(pool, layer, q, num_seqs, num_q_heads, block_tables, max_blocks,
                          context_lens, max_context, scale, partition_tokens, out, workspace,
                          workspace_bytes, stream);
  if (st) return st;
  st = pa_decode_partitions(pool, layer, q, num_seqs, num_q_heads, block_tables, max_blocks,
                            context_lens, max_context, scale, partition_tokens, out, workspace,
                            workspace_bytes, stream);
  if (st) return st;
  return pa_decode_reduce(pool, layer, q, num_seqs, num_q_heads, block_tables, max_blocks,
                          context_lens, max_context, scale, partition_tokens, out, workspace,
                          workspace_bytes, stream);
}

// The new rows' cache write and a decode step (window 0: all tokens): the write and the plan
// in one launch, then the partitions and the merge unless plan_only.  Every argument is
// checked before the first launch.
static int cache_and_decode(pa_pool* pool, int32_t layer, const void* k, const void* v,
                            const int64_t* slots, int32_t n_tokens, const void* q, int32_t num_seqs,
                            int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                            const int32_t* context_lens, int32_t max_context, int32_t window,
                            float scale, int32_t partition_tokens, float* out, void* workspace,
                            int64_t workspace_bytes, bool plan_only, const char* what, void* stream) {
  pa::CacheWrite w;
  int st = prepare_cache_write(pool, layer, k, v, slots, n_tokens, &w);
  if (st) return st;
  DecodeCall c;
  st = prepare_decode(pool, layer, q, num_seqs, num_q_heads, block_tables, max_blocks,
                      context_lens, max_context, scale, partition_tokens, out, workspace,
                      workspace_bytes, &c, window);
  if (st) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = debug_check_slots(w, n_tokens, s, what);
  if (st) return st;
  if (c.args.num_seqs == 0) {
    if (w.total_chunks == 0) return ok();
    return hip_status(pa::launch_reshape_and_cache(w, s), what);
  }
  st = hip_status(pa::launch_cache_write_plan(w, c.args, s), what);
  if (st || plan_only) return st;
  st = hip_status(pa::launch_decode_partitions(c.args, static_cast<int>(pool->desc.kv_dtype), c.group, s),
                  what);
  if (st) return st;
  if (c.args.pmax <= 1) return ok();
  return hip_status(pa::launch_decode_reduce(c.args, s), what);
}

int pa_cache_and_decode_plan(pa_pool* pool, int32_t layer, const void* k, const void* v,
                             const int64_t* slots, int32_t n_tokens, const void* q,
                             int32_t num_seqs, int32_t num_q_heads, const int32_t* block_tables,
                             int32_t max_blocks, const int32_t* context_lens, int32_t max_context,
                             float scale, int32_t partition_tokens, float* out, void* workspace,
                             int64_t workspace_bytes, void* stream) {
  return cache_and_decode(pool, layer, k, v, slots, n_tokens, q, num_seqs, num_q_heads, block_tables,
                          max_blocks, context_lens, max_context, 0, scale, partition_tokens, out,
                          workspace, workspace_bytes, true, "pa_cache_and_decode_plan", stream);
}

int pa_cache_and_decode(pa_pool* pool, int32_t layer, const void* k, const void* v,
                        const int64_t* slots, int32_t n_tokens, const void* q, int32_t num_seqs,
                        int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                        const int32_t* context_lens, int32_t max_context, float scale,
                        int32_t partition_tokens, float* out, void* workspace,
                        int64_t workspace_bytes, void* stream) {
  return cache_and_decode(pool, layer, k, v, slots, n_tokens, q, num_seqs, num_q_heads, block_tables,
                          max_blocks, context_lens, max_context, 0, scale, partition_tokens, out,
                          workspace, workspace_bytes, false, "pa_cache_and_decode", stream);
}

int pa_cache_and_decode_window(pa_pool* pool, int32_t layer, const void* k, const void* v,
                               const int64_t* slots, int32_t n_tokens, const void* q,
                               int32_t num_seqs, int32_t num_q_heads, const int32_t* block_tables,
                               int32_t max_blocks, const int32_t* context_lens,
                               int32_t max_context, int32_t window, float scale,
                               int32_t partition_tokens, float* out, void* workspace,
                               int64_t workspace_bytes, void* stream) {
  return cache_and_decode(pool, layer, k, v, slots, n_tokens, q, num_seqs, num_q_heads, block_tables,
                          max_blocks, context_lens, max_context, window, scale, partition_tokens,
                          out, workspace, workspace_bytes, false, "pa_cache_and_decode_window",
                          stream);
}

int64_t pa_static_scratch_bytes(void) { return pa::kStaticScratchBytes; }

int pa_cache_and_decode_static(pa_pool* pool, int32_t layer, const void* k, const void* v,
                               const int64_t* slots, int32_t n_tokens, const void* q,
                               int32_t num_seqs, int32_t num_q_heads, const int32_t* block_tables,
                               int32_t max_blocks, const int32_t* context_lens, int32_t max_context,
                               float scale, int32_t partition_tokens, float* out, void* stream) {
  int st = check_device_pool(pool, layer);
  if (st) return st;
  const int64_t need = pa_decode_workspace_bytes(pool, num_seqs, num_q_heads, max_context,
                                                 partition_tokens);
  if (need < 0) return static_cast<int>(need);
  if (need > pa::kStaticScratchBytes)
    return fail(PA_E_RANGE, "pa_cache_and_decode_static: this decode needs %lld bytes of "
                "workspace, more than the %lld the library holds (use pa_cache_and_decode)",
                static_cast<long long>(need), static_cast<long long>(pa::kStaticScratchBytes));
  void* ws = nullptr;
  st = hip_status(pa::static_scratch(&ws), "pa_cache_and_decode_static (scratch address)");
  if (st) return st;
  return cache_and_decode(pool, layer, k, v, slots, n_tokens, q, num_seqs, num_q_heads, block_tables,
                          max_blocks, context_lens, max_context, 0, scale, partition_tokens, out,
                          ws, pa::kStaticScratchBytes, false, "pa_cache_and_decode_static", stream);
}

int32_t pa_prefill_part_keys(void) { return pa::kPrefillPartKeys; }

static int64_t prefill_pmax(int32_t max_context) {
  return std::max<int64_t>(1, (static_cast<int64_t>(max_context) + pa::kPrefillPartKeys - 1) /
                                  pa::kPrefillPartKeys);
}

// Units the prefill work list can hold: a sequence's row blocks number at most its rows,
// so num_rows x key parts x KV heads bounds every nondecreasing query_start.
static __int128 prefill_work_cap(const pa_pool* pool, int32_t num_rows, int32_t max_context) {
  return static_cast<__int128>(num_rows) * prefill_pmax(max_context) * pool->desc.num_kv_heads;
}

static int64_t round256(__int128 bytes) { return static_cast<int64_t>((bytes + 255) / 256 * 256); }

int64_t pa_prefill_workspace_bytes(const pa_pool* pool, int32_t num_rows, int32_t num_q_heads,
                                   int32_t max_context) {
  if (!pool) return fail(PA_E_INVAL, "pool is NULL");
  if (num_rows < 0 || num_q_heads < 0 || max_context < 0) return fail(PA_E_INVAL, "negative size");
  const int64_t pmax = prefill_pmax(max_context);
  const __int128 cap = prefill_work_cap(pool, num_rows, max_context);
  if (cap > 0x7fffffff) return fail(PA_E_RANGE, "more than 2^31 - 1 prefill work units");
  __int128 bytes = pa::kPrefillHeaderBytes + round256(cap * 16);
  if (pmax > 1) {
    const __int128 items = static_cast<__int128>(num_rows) * num_q_heads * pmax;
    bytes += items * pa::kHeadDim * 4 + round256(items * 4);
  }
  if (bytes > std::numeric_limits<int64_t>::max() / 2) return fail(PA_E_RANGE, "workspace too large");
  return static_cast<int64_t>(bytes);
}

int pa_prefill_chunked(pa_pool* pool, int32_t layer, const void* q, int32_t num_rows,
                       int32_t num_q_heads, const int32_t* query_start, int32_t num_seqs,
                       const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                       int32_t max_context, int32_t max_query_len, float scale, float* out,
                       void* workspace, int64_t workspace_bytes, void* stream) {
  int st = check_device_pool(pool, layer);
  if (st) return st;
  const pa_pool_desc& d = pool->desc;
  if (num_rows < 0 || num_seqs < 0 || num_q_heads < 1 || max_blocks < 0 || max_context < 0 ||
      max_query_len < 0)
    return fail(PA_E_INVAL, "negative size (num_rows %d num_seqs %d num_q_heads %d max_blocks %d "
                "max_context %d max_query_len %d)", num_rows, num_seqs, num_q_heads, max_blocks,
                max_context, max_query_len);
  if (num_q_heads % d.num_kv_heads != 0)
    return fail(PA_E_INVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                d.num_kv_heads);
  const int group = num_q_heads / d.num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PA_E_UNSUPPORTED, "query group size %d (supported: 1, 2, 4, 8)", group);
  if (d.head_dim != pa::kHeadDim)
    return fail(PA_E_UNSUPPORTED, "head_dim %d (supported: %d)", d.head_dim, pa::kHeadDim);
  if (d.kv_dtype != PA_F16 && d.kv_dtype != PA_BF16)
    return fail(PA_E_UNSUPPORTED, "chunked prefill runs on the matrix cores: fp16 or bf16 caches only");
  if (d.block_size < 16 || (d.block_size & (d.block_size - 1)) != 0)
    return fail(PA_E_UNSUPPORTED, "block_size %d (chunked prefill: a power of two >= 16)", d.block_size);
  if (!std::isfinite(scale)) return fail(PA_E_INVAL, "scale is not finite");
  if (num_seqs == 0 || max_query_len == 0) return ok();
  if (!q || !query_start || !block_tables || !context_lens || !out)
    return fail(PA_E_INVAL, "q, query_start, block_tables, context_lens and out must be non-NULL");
  if (static_cast<int64_t>(num_rows) * num_q_heads > 0x7fffffff)
    return fail(PA_E_RANGE, "num_rows * num_q_heads exceeds 2^31 - 1");
  for (const void* ptr : {q, static_cast<const void*>(out)})
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
      return fail(PA_E_INVAL, "q and out must be 16-byte aligned");
  if (num_seqs > 65535 || d.num_kv_heads > 65535)
    return fail(PA_E_UNSUPPORTED, "more than 65535 sequences or KV heads in one call");
  const int64_t rows_per_block = pa::kPrefillColumns / group;
  const int64_t row_blocks = (max_query_len + rows_per_block - 1) / rows_per_block;
  if (row_blocks * num_seqs > 0x7fffffff)
    return fail(PA_E_UNSUPPORTED, "%lld row blocks (sequences x row blocks of max_query_len) "
                "exceed 2^31 - 1", static_cast<long long>(row_blocks * num_seqs));
  pa::PrefillArgs a{};
  a.q = q;
  a.k_cache = pool->dev_base + static_cast<int64_t>(2 * layer) * pool->array_bytes;
  a.v_cache = pool->dev_base + static_cast<int64_t>(2 * layer + 1) * pool->array_bytes;
  a.query_start = query_start;
  a.tables = block_tables;
  a.ctx = context_lens;
  a.out = out;
  a.num_rows = num_rows;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = d.num_kv_heads;
  a.max_blocks = max_blocks;
  a.num_blocks = d.num_blocks;
  a.block_size = d.block_size;
  a.block_shift = __builtin_ctz(static_cast<unsigned>(d.block_size));
  a.max_context = max_context;
  // The kernel takes a positive score scale; the caller's sign goes into the queries
  // (a sign flip of each 16-bit element, exact) and a zero scale zeroes them.
  a.scale_log2 = (scale == 0.0f ? 1.0f : std::fabs(scale)) * 1.4426950408889634f;
  a.q_and = scale == 0.0f ? 0u : 0xffffffffu;
  a.q_xor = scale < 0.0f ? 0x80008000u : 0u;
  a.part_keys = pa::kPrefillPartKeys;
  a.pmax = static_cast<int32_t>(prefill_pmax(max_context));
  a.row_blocks = static_cast<int32_t>(row_blocks);
  a.part_o = nullptr;
  a.part_lse = nullptr;
  {
    const int64_t need = pa_prefill_workspace_bytes(pool, num_rows, num_q_heads, max_context);
    if (need < 0) return static_cast<int>(need);
    if (!workspace || workspace_bytes < need)
      return fail(PA_E_INVAL, "workspace of %lld bytes < %lld needed (pa_prefill_workspace_bytes)",
                  static_cast<long long>(workspace_bytes), static_cast<long long>(need));
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(PA_E_INVAL, "workspace must be 256-byte aligned");
    // Layout: the work list's header, its units, then (with more than one key part) the
    // parts' log-sum-exps and outputs.
    char* base = static_cast<char*>(workspace);
    const __int128 cap = prefill_work_cap(pool, num_rows, max_context);
    a.work_header = reinterpret_cast<int32_t*>(base);
    a.work_units = reinterpret_cast<int32_t*>(base + pa::kPrefillHeaderBytes);
    a.work_cap = static_cast<int32_t>(cap);
    base += pa::kPrefillHeaderBytes + round256(cap * 16);
    if (a.pmax > 1) {
      const int64_t items = static_cast<int64_t>(num_rows) * num_q_heads * a.pmax;
      a.part_lse = reinterpret_cast<float*>(base);
      a.part_o = reinterpret_cast<float*>(base + round256(items * 4));
    }
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(pa::launch_prefill_plan(a, group, s), "pa_prefill_chunked (plan)");
  if (st) return st;
  st = hip_status(pa::launch_prefill(a, static_cast<int>(d.kv_dtype), group, s),
                  "pa_prefill_chunked");
  if (st) return st;
  return hip_status(pa::launch_prefill_merge(a, group, max_query_len, s), "pa_prefill_chunked (merge)");
}

int pa_decode_window(pa_pool* pool, int32_t layer, const void* q, int32_t num_seqs,
                     int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                     const int32_t* context_lens, int32_t max_context, int32_t window, float scale,
                     int32_t partition_tokens, float* out, void* workspace, int64_t workspace_bytes,
                     void* stream) {
  DecodeCall c;
  int st = prepare_decode(pool, layer, q, num_seqs, num_q_heads, block_tables, max_blocks,
                          context_lens, max_context, scale, partition_tokens, out, workspace,
                          workspace_bytes, &c, window);
  if (st) return st;
  if (c.args.num_seqs == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(pa::launch_decode_plan(c.args, s), "pa_decode_window (plan)");
  if (st) return st;
  st = hip_status(pa::launch_decode_partitions(c.args, static_cast<int>(pool->desc.kv_dtype), c.group, s),
                  "pa_decode_window (partitions)");
  if (st) return st;
  if (c.args.pmax <= 1) return ok();
  return hip_status(pa::launch_decode_reduce(c.args, s), "pa_decode_window (reduce)");
}

int pa_seq_release_before(pa_pool* pool, int32_t seq, int32_t token, int32_t* n_released_out) {
  if (!pool || !n_released_out) return fail(PA_E_INVAL, "pool and n_released_out must be non-NULL");
  int32_t n = 0;
  int st = mgr_status(pool->mgr->seq_release_before(seq, token, &n), "pa_seq_release_before");
  if (st == PA_OK) *n_released_out = n;
  return st;
}

int64_t pa_swap_space_bytes(const pa_pool_desc* desc, int32_t host_blocks) {
  if (host_blocks < 0) return fail(PA_E_INVAL, "host_blocks < 0");
  const int64_t b = pa_block_bytes(desc);
  if (b < 0) return b;
  return b * host_blocks;
}

int pa_pool_set_swap_space(pa_pool* pool, int32_t host_blocks) {
  if (!pool) return fail(PA_E_INVAL, "pool is NULL");
  if (pool->mgr->set_swap_space(host_blocks) != pa::MgrStatus::ok)
    return fail(PA_E_INVAL, "pa_pool_set_swap_space: bad size, or sequences are swapped out");
  return ok();
}

static int swap_call(pa_pool* pool, const int32_t* seqs, int32_t count, int32_t* pairs_out,
                     int32_t cap, int32_t* n_pairs_out, bool out, const char* what) {
  if (!pool || !n_pairs_out) return fail(PA_E_INVAL, "%s: pool and n_pairs_out must be non-NULL", what);
  if (count < 0 || (count > 0 && !seqs)) return fail(PA_E_INVAL, "%s: bad seqs / count", what);
  if (cap < 0 || (cap > 0 && !pairs_out)) return fail(PA_E_INVAL, "%s: bad pairs_out / cap", what);
  int32_t n = 0;
  const pa::MgrStatus st = out ? pool->mgr->seq_swap_out(seqs, count, pairs_out, cap, &n)
                               : pool->mgr->seq_swap_in(seqs, count, pairs_out, cap, &n);
  const int rc = mgr_status(st, what);
  if (rc == PA_OK) *n_pairs_out = n;
  return rc;
}

int pa_seq_swap_out(pa_pool* pool, const int32_t* seqs, int32_t count, int32_t* pairs_out,
                    int32_t cap, int32_t* n_pairs_out) {
  return swap_call(pool, seqs, count, pairs_out, cap, n_pairs_out, true, "pa_seq_swap_out");
}

int pa_seq_swap_in(pa_pool* pool, const int32_t* seqs, int32_t count, int32_t* pairs_out,
                   int32_t cap, int32_t* n_pairs_out) {
  return swap_call(pool, seqs, count, pairs_out, cap, n_pairs_out, false, "pa_seq_swap_in");
}

int pa_seq_swapped(const pa_pool* pool, int32_t seq, int32_t* swapped_out) {
  if (!pool || !swapped_out) return fail(PA_E_INVAL, "pool and swapped_out must be non-NULL");
  if (!pool->mgr->live(seq)) return fail(PA_E_INVAL, "unknown or freed sequence %d", seq);
  *swapped_out = pool->mgr->swapped(seq) ? 1 : 0;
  return ok();
}

int pa_host_block_refcount(const pa_pool* pool, int32_t host_block, int32_t* rc_out) {
  if (!pool || !rc_out) return fail(PA_E_INVAL, "pool and rc_out must be non-NULL");
  if (host_block < 0 || host_block >= pool->mgr->num_host_blocks())
    return fail(PA_E_INVAL, "host block %d out of range", host_block);
  *rc_out = pool->mgr->host_refcount(host_block);
  return ok();
}

int pa_export_host_free_stack(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!pool || !n_out || cap < 0 || (cap > 0 && !out)) return fail(PA_E_INVAL, "bad arguments");
  std::vector<int32_t> v;
  pool->mgr->host_free_stack_top_first(&v);
  *n_out = static_cast<int32_t>(v.size());
  if (static_cast<int64_t>(v.size()) > cap) return fail(PA_E_RANGE, "cap %d < %zu free host blocks", cap, v.size());
  for (size_t i = 0; i < v.size(); ++i) out[i] = v[i];
  return ok();
}

int pa_swap_blocks(pa_pool* pool, void* host_base, int64_t host_bytes, const int32_t* pairs,
                   int32_t n_pairs, int32_t to_host, void* stream) {
  int st = check_device_pool(pool, 0);
  if (st) return st;
  if (n_pairs < 0) return fail(PA_E_INVAL, "n_pairs < 0");
  if (n_pairs == 0) return ok();
  if (!pairs || !host_base) return fail(PA_E_INVAL, "pairs and host_base must be non-NULL");
  const int32_t host_blocks = pool->mgr->num_host_blocks();
  if (host_blocks == 0) return fail(PA_E_INVAL, "pa_swap_blocks: the pool has no swap space");
  const int64_t need = pa_block_bytes(&pool->desc) * host_blocks;
  if (host_bytes < need)
    return fail(PA_E_INVAL, "host buffer holds %lld bytes < %lld of the swap space",
                static_cast<long long>(host_bytes), static_cast<long long>(need));
  if (reinterpret_cast<uintptr_t>(host_base) % 16 != 0) return fail(PA_E_INVAL, "host_base not 16-byte aligned");
  if (2 * pool->desc.num_layers > 65535) return fail(PA_E_UNSUPPORTED, "too many layers");
  const int64_t block_bytes = pool->array_bytes / pool->desc.num_blocks;
  if (block_bytes % 16 != 0) return fail(PA_E_UNSUPPORTED, "per-layer block bytes not a multiple of 16");
  // The kernel reaches the host buffer through its device mapping; memory that is not
  // pinned host memory has none and is rejected here, before any launch.
  void* mapped = nullptr;
  if (hipHostGetDevicePointer(&mapped, host_base, 0) != hipSuccess || !mapped) {
    (void)hipGetLastError();
    return fail(PA_E_INVAL, "pa_swap_blocks: host_base is not pinned host memory");
  }
  const int32_t N = pool->desc.num_blocks;
  const hipError_t e = to_host
      ? pa::launch_swap_blocks(pairs, n_pairs, pool->dev_base, N, mapped, host_blocks,
                               2 * pool->desc.num_layers, block_bytes, static_cast<hipStream_t>(stream))
      : pa::launch_swap_blocks(pairs, n_pairs, mapped, host_blocks, pool->dev_base, N,
                               2 * pool->desc.num_layers, block_bytes, static_cast<hipStream_t>(stream));
  return hip_status(e, "pa_swap_blocks");
}

int pa_pool_set_kv_scales(pa_pool* pool, int32_t layer, float k_scale, float v_scale) {
  if (!pool) return fail(PA_E_INVAL, "pool is NULL");
  if (layer < 0 || layer >= pool->desc.num_layers)
    return fail(PA_E_INVAL, "layer %d outside [0, %d)", layer, pool->desc.num_layers);
  if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_E_INVAL, "scales must be finite and > 0");
  pool->k_scale[layer] = k_scale;
  pool->v_scale[layer] = v_scale;
  return ok();
}

}  // extern "C"

