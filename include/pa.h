/*
 * pa.h -- C ABI of libpa: paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * Two layers, as the pages split the method ("vLLM explained", jackchen890311.github.io,
 * section on the two implementation layers):
 *   1. a memory manager: fixed-size blocks, per-sequence block tables, allocation on
 *      demand, release, reference counts and copy-on-write (host, C++);
 *   2. kernels that read K/V by jumping through the block table (HIP, gfx950).
 *
 * Conventions shared by every call
 *   - Return value: PA_OK (0) or a negative PA_E_* code; the message for the last error
 *     on the calling thread is returned by pa_last_error().  Calls returning int64_t
 *     return a negative PA_E_* code on error.
 *   - Ownership: every device buffer is allocated and freed by the caller.  The library
 *     owns only the host-side pa_pool object (descriptor plus manager state).
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device calls only enqueue work; they never synchronize or read device memory
 *     back.  Launch failures are reported as PA_E_HIP.
 *   - Validation: host-side arguments are checked (null pointers, sizes, supported
 *     shapes).  Device-resident indices (block tables, context lengths, slots, copy
 *     pairs) are trusted to be in range, but the kernels never access memory outside
 *     the pool for out-of-range values: see each call.
 *   - Threading: a pa_pool is not thread-safe; calls on one pool must be serialized.
 *
 * Cache layout (one pool, caller memory at dev_base):
 *     [num_layers][2 (K, V)][num_blocks][num_kv_heads][block_size][head_dim]
 *   elements of kv_dtype.  One block id addresses the same block in every layer, which
 *   is why a block's byte size carries the layer count ("vLLM explained", block-size
 *   section, block-byte formula).  Inside a block the layout is head-major, so the
 *   block_size x head_dim tile of one KV head is one contiguous run.
 */
#ifndef PA_H
#define PA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PA_OK = 0,
  PA_E_INVAL = -1,       /* bad argument (null pointer, negative size, unknown id, ...) */
  PA_E_NOMEM = -2,       /* the free list cannot cover the request; nothing changed     */
  PA_E_HIP = -3,         /* a HIP runtime call or kernel launch failed                  */
  PA_E_UNSUPPORTED = -4, /* valid but not implemented shape (see each call)              */
  PA_E_RANGE = -5        /* an output buffer or capacity is too small                    */
};

/* Cache element types.  PA_FP8_E4M3 is the OCP 8-bit float (1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, largest magnitude 448, no infinities): a KV cache of one
 * byte per value ("vLLM explained", block-size section: FP8 takes 1 byte; appendix:
 * quantization shrinks the KV cache).  Its rows come in, and its queries are given, as
 * bf16; each layer holds a K and a V scale (pa_pool_set_kv_scales). */
enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 };

typedef struct {
  int32_t num_layers;   /* >= 1                                   */
  int32_t num_blocks;   /* N physical blocks, >= 1                */
  int32_t block_size;   /* tokens per block, >= 1                 */
  int32_t num_kv_heads; /* >= 1                                   */
  int32_t head_dim;     /* >= 1 (the attention kernels need 128)  */
  int32_t kv_dtype;     /* PA_F32, PA_F16, PA_BF16 or PA_FP8_E4M3 */
} pa_pool_desc;

typedef struct pa_pool pa_pool; /* opaque, host-side, owned by the library */

/* ---------------------------------------------------------------- sizes
 * pa_block_bytes: bytes of one physical block across all layers, K and V:
 *   2 * block_size * num_layers * num_kv_heads * head_dim * element bytes
 *   ("vLLM explained", block-size section, block-byte formula; e.g. 8,388,608 B for a
 *   Llama-2-7B-shaped fp16 cache with 16-token blocks).
 * pa_pool_bytes: num_blocks * pa_block_bytes.  Both return PA_E_INVAL for a bad desc. */
int64_t pa_block_bytes(const pa_pool_desc* desc);
int64_t pa_pool_bytes(const pa_pool_desc* desc);

/* ---------------------------------------------------------------- pool
 * pa_alloc_pool: binds `dev_bytes` bytes of caller device memory at `dev_base`
 *   (256-byte aligned, dev_bytes >= pa_pool_bytes) and builds the block manager over
 *   the desc's num_blocks blocks.  `initial_free_order` (host, num_blocks entries, a
 *   permutation of 0..N-1, or NULL for 0,1,2,...) is the order in which free blocks
 *   are handed out.  With dev_base == NULL and dev_bytes == 0 the pool is host-only:
 *   the manager works and every device call returns PA_E_INVAL.  Nothing is written
 *   to device memory.  The caller keeps the memory alive until pa_free_pool.
 * pa_free_pool: releases the host object only (NULL is accepted).
 * pa_pool_layer_ptrs: device addresses of layer `layer`'s K and V
 *   [num_blocks][num_kv_heads][block_size][head_dim] arrays. */
int pa_alloc_pool(const pa_pool_desc* desc, void* dev_base, int64_t dev_bytes,
                  const int32_t* initial_free_order, pa_pool** out);
int pa_free_pool(pa_pool* pool);
int pa_pool_layer_ptrs(const pa_pool* pool, int32_t layer, void** k_base, void** v_base);

/* pa_pool_set_kv_scales: per-tensor scales of layer `layer` (both finite and > 0; 1 by
 *   default).  For an FP8 cache a stored code c stands for decode(c) * scale:
 *   pa_reshape_and_cache stores round_to_nearest_even(clamp(x * (1/scale), -448, 448))
 *   with x * (1/scale) computed in float32 (NaN stays NaN), and pa_decode /
 *   pa_decode_window multiply scores by k_scale and outputs by v_scale.  The scales are
 *   read at each call (host state); other dtypes ignore them. */
int pa_pool_set_kv_scales(pa_pool* pool, int32_t layer, float k_scale, float v_scale);

/* ---------------------------------------------------------------- block manager (host)
 * The KV cache is cut into fixed-size blocks that need not be contiguous; a block
 * table maps each sequence's logical blocks to physical ones; blocks are taken on
 * demand and returned when the sequence ends ("vLLM explained", PagedAttention
 * section, items 1-4; "LLM inference optimization: KV cache & PagedAttention",
 * carlstack.gravito.dev, section 三.1 and Fig. 1).  Sequences forked from one parent
 * share physical blocks by reference count, and a shared block is copied only when
 * a branch writes a different token into it (carlstack page, section 三.2).
 *
 * Rules where the pages are silent (all operations are deterministic):
 *   - Free list: a LIFO stack; freed blocks are pushed in logical order (last to
 *     first when prefix caching is on, see below).
 *   - Append of n tokens at length L: if L % block_size != 0 and the last block's
 *     reference count is > 1, that block is first copied (copy-on-write): a fresh
 *     block p' is taken, the pair (p, p') is reported, p loses one reference and p'
 *     replaces p in the table.  Full blocks are never copied.  Then each position
 *     with pos % block_size == 0 takes a fresh block.  Token pos gets the slot
 *     table[pos / block_size] * block_size + pos % block_size.
 *   - All-or-nothing: PA_E_NOMEM (free list too short) or PA_E_RANGE (cow_cap too
 *     small) leave the manager unchanged.
 *   - Sequence ids are 0, 1, 2, ... in creation order and are never reused.
 *
 * pa_seq_new:    creates an empty sequence.
 * pa_seq_append: appends n_tokens (>= 0) tokens; writes their slots to slots_out
 *                (host, n_tokens entries) and the copy-on-write pairs (src, dst) to
 *                cow_pairs_out (host, 2 * cow_cap entries; an append makes at most
 *                one pair) with their count in *n_cow_out.
 * pa_seq_fork:   new sequence with a copy of parent's table and length; every block
 *                gains one reference.
 * pa_seq_free:   drops one reference from each block in logical order; blocks that
 *                reach zero go back on the free stack.  The id becomes invalid.
 * pa_seq_length: the sequence's token count.
 * pa_export_block_tables: for the n sequences in seqs (host), writes
 *                tables_out[n][max_blocks] (physical ids, padded with -1) and
 *                ctx_out[n] (lengths).  PA_E_RANGE if a table is longer than max_blocks.
 * pa_block_refcount, pa_num_free_blocks: queries.
 * pa_export_free_stack: free blocks in the order they will be handed out (next first);
 *                PA_E_RANGE if cap is too small (*n_out is still set). */
int pa_seq_new(pa_pool* pool, int32_t* seq_out);
int pa_seq_append(pa_pool* pool, int32_t seq, int32_t n_tokens, int64_t* slots_out,
                  int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow_out);
/* pa_seq_append_batch: one scheduling step's appends in one call: n_tokens[i] tokens
 *                (n_tokens == NULL: one each) to seqs[i] (host, `count` distinct live
 *                ids), in that order, with exactly the effect of consecutive
 *                pa_seq_append calls, but all-or-nothing for the whole batch
 *                (PA_E_NOMEM / PA_E_RANGE / PA_E_INVAL leave the manager unchanged).
 *                slots_out (host) receives the slots back to back, in batch order;
 *                cow_pairs_out (host, 2 * cow_cap) the copy-on-write pairs in batch
 *                order, their count in *n_cow_out. */
int pa_seq_append_batch(pa_pool* pool, const int32_t* seqs, int32_t count, const int32_t* n_tokens,
                        int64_t* slots_out, int32_t* cow_pairs_out, int32_t cow_cap,
                        int32_t* n_cow_out);
int pa_seq_fork(pa_pool* pool, int32_t parent, int32_t* child_out);
int pa_seq_free(pa_pool* pool, int32_t seq);
int pa_seq_length(const pa_pool* pool, int32_t seq, int32_t* len_out);
int pa_export_block_tables(const pa_pool* pool, const int32_t* seqs, int32_t n,
                           int32_t max_blocks, int32_t* tables_out, int32_t* ctx_out);
int pa_block_refcount(const pa_pool* pool, int32_t block, int32_t* rc_out);
/* pa_num_free_blocks: blocks an append may take (free and empty, plus free and cached
 *                when prefix caching is on). */
int pa_num_free_blocks(const pa_pool* pool, int32_t* n_out);
int pa_export_free_stack(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n_out);

/* ---------------------------------------------------------------- prefix caching (host)
 * A prompt prefix that many requests share has its KV computed once and reused.  The
 * cache is not a separate region: it lives in the same block pool.  A block is in use
 * (reference count > 0), free and empty, or free but still holding cached content; a
 * request that needs a block takes an empty one first and only then evicts a free
 * cached block, least recently used first; blocks in use are never evicted ("vLLM
 * explained", jackchen890311.github.io, section on prefix caching and its figure of
 * the three block states).
 *
 * Rules where the pages are silent (deterministic, like the rest of the manager):
 *   - Identity: a full block is identified by the token ids of its sequence from the
 *     first token through the block's last token (exactly; no hash collisions).  Only
 *     full blocks are cached.
 *   - A block is registered when an append fills it, if every token of the sequence
 *     was appended with its id (pa_seq_append_tokens / _batch_tokens; one append
 *     without ids stops this for the rest of the sequence's life, forks included) and
 *     no other block has that identity yet.
 *   - pa_seq_new_prefix takes the longest run of cached blocks (in use or free) whose
 *     identities match the prompt's leading full blocks, at most (n_prompt - 1) /
 *     block_size of them, so at least one prompt token is left to compute.
 *   - A block whose reference count reaches 0 goes to the most-recent end of the LRU
 *     list if it is cached, else onto the free stack.  When prefix caching is on,
 *     blocks released together (pa_seq_free, pa_seq_release_before) are released
 *     from the last logical block to the first, so a sequence's tail is evicted before
 *     its prefix.  Eviction drops the block's identity.
 *
 * pa_pool_enable_prefix_caching: turns prefix caching on for the pool's manager;
 *   PA_E_INVAL while any sequence is live.  It stays on.
 * pa_seq_new_prefix: new sequence (id in *seq_out) that shares the matching cached
 *   blocks; *n_cached_out = tokens they cover (a multiple of block_size), which is the
 *   new sequence's length.  prompt: host int32 [n_prompt] token ids.  The caller then
 *   appends prompt[*n_cached_out:] with pa_seq_append_tokens, writes those tokens' K/V
 *   and runs prefill over them only.  PA_E_INVAL if prefix caching is off.
 * pa_seq_append_tokens / pa_seq_append_batch_tokens: pa_seq_append /
 *   pa_seq_append_batch with the appended tokens' ids (host int32, one per appended
 *   token, back to back in batch order).  On a pool without prefix caching the ids
 *   are ignored.
 * pa_block_state: 0 free and empty, 1 in use, 2 free and cached.
 * pa_export_evictable: free cached blocks, next to be evicted first; PA_E_RANGE if
 *   cap is too small (*n_out is still set). */
enum { PA_BLOCK_FREE_EMPTY = 0, PA_BLOCK_IN_USE = 1, PA_BLOCK_FREE_CACHED = 2 };
int pa_pool_enable_prefix_caching(pa_pool* pool);
int pa_seq_new_prefix(pa_pool* pool, const int32_t* prompt, int32_t n_prompt, int32_t* seq_out,
                      int32_t* n_cached_out);
int pa_seq_append_tokens(pa_pool* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens,
                         int64_t* slots_out, int32_t* cow_pairs_out, int32_t cow_cap,
                         int32_t* n_cow_out);
int pa_seq_append_batch_tokens(pa_pool* pool, const int32_t* seqs, int32_t count,
                               const int32_t* n_tokens, const int32_t* tokens, int64_t* slots_out,
                               int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow_out);
int pa_block_state(const pa_pool* pool, int32_t block, int32_t* state_out);
int pa_export_evictable(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n_out);

/* ---------------------------------------------------------------- swap preemption
 * When blocks run short, a request can be preempted and its KV moved to CPU memory
 * (swap) instead of being recomputed later ("vLLM explained", jackchen890311.github.io,
 * table on when KV may be overwritten).
 *
 * The swap space is caller-owned pinned host memory laid out like the pool, with its
 * own block count M: [num_layers][K|V][M][num_kv_heads][block_size][head_dim]
 * (pa_swap_space_bytes).  The manager keeps a LIFO free stack of host blocks (0 first)
 * and their reference counts.
 *
 * Rules where the pages are silent (deterministic, all-or-nothing):
 *   - pa_seq_swap_out(seqs): every distinct device block in the tables of the given
 *     sequences (distinct, live, resident) gets one host block, in order of first use
 *     (sequence order, then logical order); a block shared by several of them is
 *     copied once.  The pairs (device, host) are reported; the tables now name host
 *     blocks; each sequence then drops its device references as pa_seq_free would
 *     (blocks reaching zero go back to the free stack, or the LRU list if cached).
 *     PA_E_NOMEM if the swap space is short, PA_E_RANGE if cap is short.
 *   - pa_seq_swap_in(seqs): the mirror image: each distinct host block gets a device
 *     block (taken as an append takes them: empty first, then eviction), pairs (host,
 *     device) reported; host references dropped in logical order.
 *   - A swapped-out sequence may only be swapped in or freed: appends, forks, window
 *     releases and table exports are PA_E_INVAL.  Swapped-in blocks are not entered
 *     into the prefix cache.
 *   - The caller copies the reported pairs with pa_swap_blocks, on the stream that
 *     later reuses the freed blocks, before that reuse (swap-out) or before the next
 *     decode of the sequences (swap-in).
 *
 * pa_swap_space_bytes: bytes of a swap space of host_blocks blocks for this layout.
 * pa_pool_set_swap_space: sizes the manager's swap space (PA_E_INVAL while a sequence
 *   is swapped out).
 * pa_swap_blocks: copies whole blocks (every layer, K and V) for n_pairs pairs (device
 *   int32 [n_pairs][2]): to_host != 0 copies device block -> host block (swap-out
 *   pairs), to_host == 0 host block -> device block (swap-in pairs).  host_base: pinned
 *   host memory (hipHostMalloc, or a pinned torch tensor) of at least
 *   pa_swap_space_bytes bytes, 16-byte aligned; the kernel reads or writes it through
 *   its device mapping, so memory without one is PA_E_INVAL.  Pairs naming a block
 *   outside either side are skipped.  Asynchronous on `stream`. */
int64_t pa_swap_space_bytes(const pa_pool_desc* desc, int32_t host_blocks);
int pa_pool_set_swap_space(pa_pool* pool, int32_t host_blocks);
int pa_seq_swap_out(pa_pool* pool, const int32_t* seqs, int32_t count, int32_t* pairs_out,
                    int32_t cap, int32_t* n_pairs_out);
int pa_seq_swap_in(pa_pool* pool, const int32_t* seqs, int32_t count, int32_t* pairs_out,
                   int32_t cap, int32_t* n_pairs_out);
int pa_seq_swapped(const pa_pool* pool, int32_t seq, int32_t* swapped_out);
int pa_host_block_refcount(const pa_pool* pool, int32_t host_block, int32_t* rc_out);
int pa_export_host_free_stack(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n_out);
int pa_swap_blocks(pa_pool* pool, void* host_base, int64_t host_bytes, const int32_t* pairs,
                   int32_t n_pairs, int32_t to_host, void* stream);

/* ---------------------------------------------------------------- device ops
 * pa_reshape_and_cache: writes new tokens' K and V rows into their slots of layer
 *   `layer` (a bit copy).  k, v: device [n_tokens][num_kv_heads][head_dim] in the
 *   pool's dtype, contiguous.  slots: device int64 [n_tokens]; slot s goes to block
 *   s / block_size, offset s % block_size; -1 means "skip this token".  Slots must be
 *   distinct (two tokens writing one slot race; pa_check_slots checks, and the debug
 *   build returns PA_E_INVAL before launching).  Slots outside [0, num_blocks *
 *   block_size) are skipped like -1, never written.  Blocks are filled on demand,
 *   token by token ("vLLM explained", PagedAttention section, item 4; carlstack page,
 *   section 三.1 figure: logical block 2 is placed in a block allocated on demand).
 *   head_dim * element bytes must be a multiple of 16 (else PA_E_UNSUPPORTED). */
int pa_reshape_and_cache(pa_pool* pool, int32_t layer, const void* k, const void* v,
                         const int64_t* slots, int32_t n_tokens, void* stream);

/* pa_copy_blocks: copy-on-write data movement: for each pair (src, dst) in pairs
 *   (device int32 [n_pairs][2]), block dst <- block src in every layer, K and V, all
 *   slots (carlstack page, section 三.2 and Fig. 1: copy only when a branch writes a
 *   different token).  The pairs run concurrently, so no dst may appear twice or also
 *   appear as a src (pairs from one step of the manager satisfy this; pa_check_copy_pairs
 *   checks, and the debug build returns PA_E_INVAL before launching).  Pairs with an id
 *   outside [0, num_blocks) are skipped. */
int pa_copy_blocks(pa_pool* pool, const int32_t* pairs, int32_t n_pairs, void* stream);

/* Paged-attention decode of one layer: for each sequence s and query head h,
 *     out[s][h] = softmax(scale * q[s][h] . K_s^T) V_s
 *   over the sequence's context_lens[s] cached tokens (the newest one included),
 *   with K_s, V_s read from KV head h / (num_q_heads / num_kv_heads) by jumping
 *   through the sequence's block table (carlstack page, section 二, attention formula;
 *   "vLLM explained", two implementation layers: same result as ordinary attention).
 *
 * The work is split over partitions of `partition_tokens` consecutive tokens (0 =
 * default: pa_decode_default_partition; else a positive multiple of 64, at most 4096),
 * run as three kernels
 * on `stream`:
 *   pa_decode_plan        lists the (sequence, partition) work items in the workspace
 *                         and zeroes its work counter;
 *   pa_decode_partitions  persistent workgroups draw items from that counter and
 *                         compute each partition's softmax statistics and normalized
 *                         output; sequences that fit one partition are finished here;
 *   pa_decode_reduce      merges each longer sequence's partitions with log-sum-exp
 *                         weights.
 * pa_decode runs all three.  pa_decode_partitions needs a pa_decode_plan with the same
 * arguments earlier on the stream, and pa_decode_reduce needs both.  The result does
 * not depend on which physical blocks hold the data: the summation order follows
 * logical token order only.  Calls that share one workspace must not overlap.
 *
 *   q            device [num_seqs][num_q_heads][head_dim], pool dtype (bf16 for an FP8
 *                cache), contiguous
 *   block_tables device int32 [num_seqs][max_blocks]; entries past a sequence's last
 *                block are never read
 *   context_lens device int32 [num_seqs], 0 <= context_lens[s] <= max_context
 *   max_context  host bound on context_lens (sizes the grid and the workspace)
 *   scale        softmax scale, any finite value (usually 1/sqrt(head_dim))
 *   out          device fp32 [num_seqs][num_q_heads][head_dim]; an empty sequence
 *                gets zeros
 *   workspace    device scratch of at least pa_decode_workspace_bytes(...) bytes,
 *                16-byte aligned (work list, counter and partition partials); its
 *                contents need no initialization
 * A sequence whose length exceeds max_context or max_blocks * block_size, or whose
 * table holds an id outside [0, num_blocks), gets NaN outputs; nothing outside the
 * pool is read.  Supported: head_dim 128; num_q_heads / num_kv_heads in {1, 2, 4, 8};
 * any block_size that is a multiple of 16; all dtypes (fp32 accumulation). */
int64_t pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_context, int32_t partition_tokens);
/* The partition size a decode call with partition_tokens = 0 uses for this pool and
 * num_q_heads (host only, no GPU call): 4096 tokens for fp16 and bf16 caches at groups
 * (num_q_heads / num_kv_heads) of 8, 2048 for fp16 and bf16 at groups of 4 and for e4m3
 * caches at groups of 4 or 8; otherwise 1024 / element bytes tokens (512 for fp16/bf16,
 * 1024 for e4m3, 256 for fp32).  Windowed calls (pa_decode_window,
 * pa_cache_and_decode_window) take at most 2048 by default, and
 * pa_decode_workspace_bytes with partition_tokens = 0 sizes for the smaller of the two, so
 * that one workspace serves both.  Returns PA_E_INVAL (negative) for a NULL pool or
 * num_q_heads that is not a positive multiple of num_kv_heads. */
int32_t pa_decode_default_partition(const pa_pool* pool, int32_t num_q_heads);
int pa_decode_plan(pa_pool* pool, int32_t layer, const void* q, int32_t num_seqs,
                   int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                   const int32_t* context_lens, int32_t max_context, float scale,
                   int32_t partition_tokens, float* out, void* workspace, int64_t workspace_bytes,
                   void* stream);
int pa_decode(pa_pool* pool, int32_t layer, const void* q, int32_t num_seqs,
              int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
              const int32_t* context_lens, int32_t max_context, float scale,
              int32_t partition_tokens, float* out, void* workspace, int64_t workspace_bytes,
              void* stream);
int pa_decode_partitions(pa_pool* pool, int32_t layer, const void* q, int32_t num_seqs,
                         int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                         const int32_t* context_lens, int32_t max_context, float scale,
                         int32_t partition_tokens, float* out, void* workspace,
                         int64_t workspace_bytes, void* stream);
int pa_decode_reduce(pa_pool* pool, int32_t layer, const void* q, int32_t num_seqs,
                     int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                     const int32_t* context_lens, int32_t max_context, float scale,
                     int32_t partition_tokens, float* out, void* workspace,
                     int64_t workspace_bytes, void* stream);

/* One decode step of one layer in three launches instead of four: pa_reshape_and_cache
 *   of the new rows (k, v, slots, n_tokens exactly as there) followed by pa_decode
 *   (every other argument exactly as there), with the cache write and the decode plan
 *   sharing one launch.  Outputs, cache contents and errors are those of the two calls
 *   made one after the other: the plan reads only context_lens, so it may run beside
 *   the writes, and the attention kernels start after both.  The order is the pages':
 *   the new token's K/V lands in a block allocated on demand, then the attention kernel
 *   reads the whole context through the block table ("vLLM explained", PagedAttention
 *   section, item 4, and its two implementation layers).
 *   Arguments are checked before anything is launched: an error launches nothing.
 * pa_cache_and_decode_plan is the first of the three launches alone (the write and
 *   the plan); pa_decode_partitions and pa_decode_reduce with the same decode
 *   arguments finish the step. */
int pa_cache_and_decode_plan(pa_pool* pool, int32_t layer, const void* k, const void* v,
                             const int64_t* slots, int32_t n_tokens, const void* q,
                             int32_t num_seqs, int32_t num_q_heads, const int32_t* block_tables,
                             int32_t max_blocks, const int32_t* context_lens, int32_t max_context,
                             float scale, int32_t partition_tokens, float* out, void* workspace,
                             int64_t workspace_bytes, void* stream);
int pa_cache_and_decode(pa_pool* pool, int32_t layer, const void* k, const void* v,
                        const int64_t* slots, int32_t n_tokens, const void* q, int32_t num_seqs,
                        int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                        const int32_t* context_lens, int32_t max_context, float scale,
                        int32_t partition_tokens, float* out, void* workspace,
                        int64_t workspace_bytes, void* stream);

/* pa_cache_and_decode_static: pa_cache_and_decode for callers that cannot allocate
 *   device memory (code under HIP graph capture, tight serving loops, harnesses that
 *   forbid hipMalloc): the decode workspace is the library's own, a static device array
 *   of pa_static_scratch_bytes() bytes (32 MiB) on each GPU the library runs on, held
 *   until the process ends.  The call allocates nothing: no hipMalloc or hipFree, no
 *   allocating library routine.  Every argument is pa_cache_and_decode's without the
 *   workspace; the caller still owns q, the tables, the new rows and out.  A decode whose
 *   workspace (pa_decode_workspace_bytes) exceeds the array is refused with PA_E_RANGE
 *   before anything is launched.  Every call on a GPU shares that GPU's array, which
 *   keeps the last call's contents (nothing needs clearing: each call's plan rewrites
 *   the work list and the counter), so calls that overlap on one GPU (two streams, two
 *   threads) race: serialize them.  Outputs and cache contents equal pa_cache_and_decode's
 *   with the same arguments, bit for bit. */
int64_t pa_static_scratch_bytes(void);
int pa_cache_and_decode_static(pa_pool* pool, int32_t layer, const void* k, const void* v,
                               const int64_t* slots, int32_t n_tokens, const void* q,
                               int32_t num_seqs, int32_t num_q_heads, const int32_t* block_tables,
                               int32_t max_blocks, const int32_t* context_lens,
                               int32_t max_context, float scale, int32_t partition_tokens,
                               float* out, void* stream);

/* Sliding-window decode: pa_decode in which sequence s attends only to its last
 *   `window` tokens, [max(0, L_s - window), L_s) ("vLLM explained", table of when KV may be
 *   overwritten: with a sliding-window model the KV outside the window can be dropped).
 *   window == 0 is plain pa_decode.  Table entries of blocks wholly before a sequence's
 *   window are never read, so they may be -1 (see pa_seq_release_before).  Arguments,
 *   workspace and errors as for pa_decode (PA_E_INVAL for window < 0). */
int pa_decode_window(pa_pool* pool, int32_t layer, const void* q, int32_t num_seqs,
                     int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                     const int32_t* context_lens, int32_t max_context, int32_t window, float scale,
                     int32_t partition_tokens, float* out, void* workspace, int64_t workspace_bytes,
                     void* stream);

/* pa_cache_and_decode_window: pa_cache_and_decode with the sliding window of
 *   pa_decode_window: the new rows' cache write and the windowed decode in three launches
 *   (the write and the plan share the first).  Outputs, cache contents and errors are
 *   those of pa_reshape_and_cache followed by pa_decode_window with the same arguments;
 *   an argument error launches nothing. */
int pa_cache_and_decode_window(pa_pool* pool, int32_t layer, const void* k, const void* v,
                               const int64_t* slots, int32_t n_tokens, const void* q,
                               int32_t num_seqs, int32_t num_q_heads, const int32_t* block_tables,
                               int32_t max_blocks, const int32_t* context_lens,
                               int32_t max_context, int32_t window, float scale,
                               int32_t partition_tokens, float* out, void* workspace,
                               int64_t workspace_bytes, void* stream);

/* pa_seq_release_before: the sliding window of `seq` has moved past `token`: every block
 *   whose tokens all lie before `token` (block j with (j + 1) * block_size <= token),
 *   except the sequence's last block, loses this sequence's reference (going back on
 *   the free stack, in logical order, when no holder is left) and its table entry
 *   becomes -1.  The length does not change; appends and forks work as before (a fork
 *   shares the holes).  *n_released_out = entries cleared now.  PA_E_INVAL for an
 *   unknown sequence or token < 0. */
int pa_seq_release_before(pa_pool* pool, int32_t seq, int32_t token, int32_t* n_released_out);

/* Chunked prefill of one layer: causal attention of the query rows of several
 *   sequences, each over that sequence's paged cache ("LLM inference optimization: KV
 *   cache & PagedAttention", carlstack.gravito.dev, section 六 item 2: long prompts in
 *   chunks, batched with decode work; "vLLM explained", appendix).  Sequence s owns query
 *   rows query_start[s] .. query_start[s+1] - 1; with n_s rows and context length L_s,
 *   its row i is the token at position L_s - n_s + i (so its K/V, like the whole chunk's,
 *   must already be in the cache: write them with pa_reshape_and_cache first) and
 *       out[row][h] = softmax(scale * q[row][h] . K^T) V  over tokens 0 .. L_s - n_s + i
 *   of the sequence, KV head h / (num_q_heads / num_kv_heads).  A decode row is the case
 *   n_s = 1.  QK^T and PV run on the matrix cores (fp16 / bf16 inputs, fp32 accumulation;
 *   the probabilities enter as a 16-bit value plus the 16-bit rounding of the rest).
 *
 *   q            device [num_rows][num_q_heads][head_dim], pool dtype, contiguous
 *   query_start  device int32 [num_seqs + 1], nondecreasing, query_start[num_seqs] <= num_rows
 *   block_tables device int32 [num_seqs][max_blocks]; entries past a sequence's last
 *                block are never read
 *   context_lens device int32 [num_seqs]
 *   max_context  host bound on context_lens
 *   max_query_len host bound on every n_s (sizes the grid: rows past it are not computed)
 *   scale        softmax scale, any finite value (usually 1/sqrt(head_dim)); a negative
 *                scale is applied exactly (the kernel flips the queries' sign bits and
 *                scales by |scale|), a zero scale gives every visible key equal weight
 *   out          device fp32 [num_rows][num_q_heads][head_dim]
 *   workspace    device, caller-owned, 256-byte aligned, at least
 *                pa_prefill_workspace_bytes(pool, num_rows, num_q_heads, max_context)
 *                bytes: it holds the work list (a 2304-byte header and 16 bytes per
 *                unit, at most num_rows x key parts x num_kv_heads units) and, past one
 *                key part, the parts' outputs and log-sum-exps
 * The work is cut into units of (sequence, KV head, 128 / group query rows, key part): the
 * keys of a long row range are split in parts of pa_prefill_part_keys() keys (2048), so that
 * no unit outlasts the batch.  A plan kernel lists the units longest first, in one queue per
 * XCD (KV heads spread over the queues); the prefill kernel then runs as many workgroups as
 * the device holds at once, each claiming units, first from its own XCD's queue; rows whose
 * keys span several parts are combined by a log-sum-exp merge kernel.  All three launches
 * go on the same stream.
 * A sequence with n_s > L_s, L_s > max_context or L_s > max_blocks * block_size, or whose
 * keys touch a table id outside [0, num_blocks), gets NaN rows; nothing outside the pool
 * or the row range is read or written.  Rows not owned by any sequence are untouched.
 * Supported: head_dim 128; fp16 and bf16 caches (PA_E_UNSUPPORTED for fp32);
 * num_q_heads / num_kv_heads in {1, 2, 4, 8}; block_size a power of two >= 16; at most
 * 65535 sequences per call, and at most 2^31 - 1 row blocks: ceil(max_query_len /
 * (128 / group)) x num_seqs (PA_E_UNSUPPORTED beyond either). */
int64_t pa_prefill_workspace_bytes(const pa_pool* pool, int32_t num_rows, int32_t num_q_heads,
                                   int32_t max_context);
/* Keys per part of pa_prefill_chunked's split (host only, no GPU call). */
int32_t pa_prefill_part_keys(void);
int pa_prefill_chunked(pa_pool* pool, int32_t layer, const void* q, int32_t num_rows,
                       int32_t num_q_heads, const int32_t* query_start, int32_t num_seqs,
                       const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                       int32_t max_context, int32_t max_query_len, float scale, float* out,
                       void* workspace, int64_t workspace_bytes, void* stream);

/* Precondition checks of the device calls, on host arrays (host only, no GPU call).
 *   pa_check_slots: the slots of one pa_reshape_and_cache (or pa_cache_and_decode*) call
 *   are distinct; slots outside [0, num_slots) are skipped by the kernels and not checked.
 *   pa_check_copy_pairs: the (src, dst) pairs [n_pairs][2] of one pa_copy_blocks call
 *   have distinct destinations, none of which is also a source; pairs with an id outside
 *   [0, num_blocks) are skipped by the kernel and not checked.
 *   PA_OK, or PA_E_INVAL with a message naming the offending slot or block.  Callers for
 *   whom such a mistake would otherwise go unseen (the writes would race) use them, and
 *   the library's debug build (libpa_debug.so, compiled with PA_DEBUG) runs them inside
 *   those device calls on host copies of the arrays (the call then waits for `stream`),
 *   returning PA_E_INVAL before anything is launched.
 * pa_debug_build: 1 in the debug build, 0 otherwise. */
int pa_check_slots(const int64_t* slots, int32_t n_tokens, int64_t num_slots);
int pa_check_copy_pairs(const int32_t* pairs, int32_t n_pairs, int32_t num_blocks);
int32_t pa_debug_build(void);

/* Thread-local message of the last failed call on this thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
