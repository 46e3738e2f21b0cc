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
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

namespace pa {

enum class MgrStatus { ok, invalid, no_blocks, range };

class BlockManager {
 public:
  // `pop_order` (num_blocks entries, a permutation) is the order in which free blocks
  // are handed out; empty means 0, 1, 2, ...
  BlockManager(int32_t num_blocks, int32_t block_size, const std::vector<int32_t>& pop_order);

  MgrStatus seq_new(int32_t* seq);
  // Appends n tokens.  On success writes n slots and at most one copy-on-write pair.
  MgrStatus seq_append(int32_t seq, int32_t n, int64_t* slots, int32_t* cow_pairs,
                       int32_t cow_cap, int32_t* n_cow);
  // Appends n[i] tokens (n == nullptr: one each) to seqs[0..count) in that order, as
  // consecutive seq_append calls would, but all-or-nothing for the whole batch.  Slots
  // are written back to back; at most one copy-on-write pair per sequence.  A sequence
  // may appear only once.
  MgrStatus seq_append_batch(const int32_t* seqs, int32_t count, const int32_t* n, int64_t* slots,
                             int32_t* cow_pairs, int32_t cow_cap, int32_t* n_cow);
  MgrStatus seq_fork(int32_t parent, int32_t* child);
  MgrStatus seq_free(int32_t seq);
  // Releases every block of seq whose tokens all lie before `token` (a sliding window
  // that has moved past them); their table entries become -1.  Sets *released.
  MgrStatus seq_release_before(int32_t seq, int32_t token, int32_t* released);

  bool live(int32_t seq) const;
  int32_t length(int32_t seq) const { return seqs_[seq].length; }
  const std::vector<int32_t>& table(int32_t seq) const { return seqs_[seq].table; }
  int32_t refcount(int32_t block) const { return refcount_[block]; }
  int32_t num_free() const { return static_cast<int32_t>(free_stack_.size()); }
  int32_t num_blocks() const { return num_blocks_; }
  // Free blocks, next to be handed out first.
  void free_stack_top_first(std::vector<int32_t>* out) const;

 private:
  struct Seq {
    bool live = false;
    int32_t length = 0;
    std::vector<int32_t> table;
  };
  int32_t pop();

  int32_t num_blocks_;
  int32_t block_size_;
  std::vector<int32_t> free_stack_;  // back() is handed out next
  std::vector<int32_t> refcount_;
  std::vector<Seq> seqs_;            // index = sequence id
};

}  // namespace pa
