// Host block manager: free list, reference counts, per-sequence block tables and
// copy-on-write for a pool of fixed-size KV blocks.
//
// The pages describe the manager's job: blocks of a fixed token count, a per-sequence
// table from logical to physical blocks, allocation only when a sequence crosses into
// a new block, release of every block when a sequence ends ("vLLM explained",
// jackchen890311.github.io, PagedAttention section, items 1-4, and the table on when
// KV may be overwritten), and reference-counted sharing between forked sequences with
// a copy made only when a branch first writes a different token into a shared block
// ("LLM inference optimization: KV cache & PagedAttention", carlstack.gravito.dev,
// section 三.2 and Fig. 1).
//
// Policy where the pages are silent: LIFO free stack; copy-on-write only for a partial
// last block with more than one holder; operations are all-or-nothing.
//
// Automatic prefix caching ("vLLM explained", section on prefix caching: the prefix
// cache shares the one block pool; a block is in use (reference count > 0), free and
// empty, or free but still holding cached content; a new request takes empty blocks
// first and only then evicts free cached blocks, least recently used first; blocks in
// use are never touched).  Readings where the pages are silent:
//   * a full block's identity is the token ids of its sequence from the first token
//     through the block's last one; only full blocks are cached;
//   * a block is registered when an append fills it, if the sequence's token ids are
//     known (every token appended with its id) and no block has that identity yet;
//   * a new sequence with a prompt takes the longest run of cached blocks matching the
//     prompt's leading full blocks, leaving at least one prompt token to compute;
//   * a block whose count drops to 0 goes to the back of the LRU list if it is cached,
//     else onto the free stack; blocks released together go from the last logical block
//     to the first, so a sequence's tail is evicted before its prefix.
// Identities are interned exactly (a trie of block-sized token runs), so equal prefixes
// always meet and different ones never do.
//
// Swap preemption ("vLLM explained", table on when KV may be overwritten: when memory
// runs short a request is preempted, its KV recomputed later or moved to CPU memory).
// A swap space of host blocks has its own LIFO free stack and reference counts.
// Swapping a set of sequences out gives every distinct device block in their tables one
// host block (a block shared by several of them is copied once), reports the (device,
// host) pairs to copy, points the tables at the host blocks and drops the sequences'
// device references as a free would.  Swapping in is the mirror image, taking device
// blocks as an append does (empty first, then eviction).  A swapped-out sequence can
// only be swapped in or freed.
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

namespace pa {

enum class MgrStatus { ok, invalid, no_blocks, range };

enum class BlockState { free_empty = 0, in_use = 1, free_cached = 2 };

class BlockManager {
 public:
  // `pop_order` (num_blocks entries, a permutation) is the order in which free blocks
  // are handed out; empty means 0, 1, 2, ...
  BlockManager(int32_t num_blocks, int32_t block_size, const std::vector<int32_t>& pop_order);

  // Turns prefix caching on; only while no sequence is live.
  MgrStatus enable_prefix_caching();
  bool prefix_caching() const { return caching_; }

  MgrStatus seq_new(int32_t* seq);
  // New sequence sharing the cached blocks that match the prompt's leading full blocks
  // (prefix caching only).  *cached = tokens covered (a multiple of the block size).
  MgrStatus seq_new_prefix(const int32_t* prompt, int32_t n_prompt, int32_t* seq, int32_t* cached);
  // Appends n tokens (token ids in `tokens`, or nullptr: ids unknown, and the sequence's
  // later blocks are never cached).  On success writes n slots and at most one
  // copy-on-write pair.
  MgrStatus seq_append(int32_t seq, int32_t n, const int32_t* tokens, int64_t* slots,
                       int32_t* cow_pairs, int32_t cow_cap, int32_t* n_cow);
  // Appends n[i] tokens (n == nullptr: one each) to seqs[0..count) in that order, as
  // consecutive seq_append calls would, but all-or-nothing for the whole batch.  Token
  // ids (or nullptr) and slots are back to back; at most one copy-on-write pair per
  // sequence.  A sequence may appear only once.
  MgrStatus seq_append_batch(const int32_t* seqs, int32_t count, const int32_t* n,
                             const int32_t* tokens, int64_t* slots, int32_t* cow_pairs,
                             int32_t cow_cap, int32_t* n_cow);
  MgrStatus seq_fork(int32_t parent, int32_t* child);
  MgrStatus seq_free(int32_t seq);
  // Releases every block of seq whose tokens all lie before `token` (a sliding window
  // that has moved past them); their table entries become -1.  Sets *released.
  MgrStatus seq_release_before(int32_t seq, int32_t token, int32_t* released);

  // Swap space of `host_blocks` blocks (only while no sequence is swapped out).
  MgrStatus set_swap_space(int32_t host_blocks);
  // Moves seqs[0..count) (distinct, live, resident) to host blocks; pairs (device,
  // host) in order of first use; all-or-nothing.
  MgrStatus seq_swap_out(const int32_t* seqs, int32_t count, int32_t* pairs, int32_t cap,
                         int32_t* n_pairs);
  // Moves seqs[0..count) (distinct, live, swapped out) back to device blocks; pairs
  // (host, device); all-or-nothing.
  MgrStatus seq_swap_in(const int32_t* seqs, int32_t count, int32_t* pairs, int32_t cap,
                        int32_t* n_pairs);
  bool swapped(int32_t seq) const { return live(seq) && seqs_[seq].swapped; }
  int32_t num_host_blocks() const { return static_cast<int32_t>(host_refcount_.size()); }
  int32_t host_refcount(int32_t h) const { return host_refcount_[h]; }
  void host_free_stack_top_first(std::vector<int32_t>* out) const;

  bool live(int32_t seq) const;
  int32_t length(int32_t seq) const { return seqs_[seq].length; }
  const std::vector<int32_t>& table(int32_t seq) const { return seqs_[seq].table; }
  int32_t refcount(int32_t block) const { return refcount_[block]; }
  // Blocks an append may take: free and empty, plus free and cached (evictable).
  int32_t num_free() const { return static_cast<int32_t>(free_stack_.size()) + lru_size_; }
  int32_t num_blocks() const { return num_blocks_; }
  BlockState state(int32_t block) const;
  bool cached(int32_t block) const { return caching_ && node_of_block_[block] >= 0; }
  // Free empty blocks, next to be handed out first.
  void free_stack_top_first(std::vector<int32_t>* out) const;
  // Free cached blocks, next to be evicted first.
  void evictable_lru_first(std::vector<int32_t>* out) const;

 private:
  struct Seq {
    bool live = false;
    bool swapped = false;      // table holds host blocks
    bool tracked = true;       // every token's id is known (prefix caching)
    int32_t length = 0;
    int64_t node = -1;         // identity node of the last full block (-1: none yet)
    std::vector<int32_t> table;
    std::vector<int32_t> tail;  // token ids of the partial last block
  };
  // One interned prefix identity: the identity `parent` extended by one block of tokens.
  struct Node {
    int64_t parent;
    std::vector<int32_t> tokens;
    int32_t block;   // the cached block with this identity, or -1
    int64_t refs;    // cached block + child nodes + sequences whose last full block it is
  };
  struct KeyHash {
    size_t operator()(const std::pair<int64_t, std::vector<int32_t>>& k) const;
  };

  int32_t pop();
  void release(int32_t block);             // drop one reference
  void lru_push_back(int32_t block);
  void lru_remove(int32_t block);
  int64_t find_node(int64_t parent, const int32_t* tokens) const;
  int64_t intern(int64_t parent, const int32_t* tokens);
  void unref(int64_t node);
  void block_filled(Seq& s, int32_t block);  // s.tail holds the block's tokens

  int32_t num_blocks_;
  int32_t block_size_;
  std::vector<int32_t> free_stack_;  // back() is handed out next
  std::vector<int32_t> refcount_;
  std::vector<Seq> seqs_;            // index = sequence id

  std::vector<int32_t> host_free_;       // back() is handed out next
  std::vector<int32_t> host_refcount_;

  bool caching_ = false;
  std::vector<int64_t> node_of_block_;       // identity a block is cached under, or -1
  std::vector<int32_t> lru_prev_, lru_next_;  // free cached blocks, intrusive list
  int32_t lru_head_ = -1, lru_tail_ = -1, lru_size_ = 0;
  std::vector<Node> nodes_;                  // slots of erased nodes are reused
  std::vector<int64_t> free_nodes_;
  std::unordered_map<std::pair<int64_t, std::vector<int32_t>>, int64_t, KeyHash> node_index_;
};

}  // namespace pa
