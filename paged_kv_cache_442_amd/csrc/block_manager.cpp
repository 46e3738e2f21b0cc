// Host block manager (see block_manager.hpp for the rules and their sources).
#include "block_manager.hpp"

#include <algorithm>

namespace pa {

BlockManager::BlockManager(int32_t num_blocks, int32_t block_size,
                           const std::vector<int32_t>& pop_order)
    : num_blocks_(num_blocks), block_size_(block_size), refcount_(num_blocks, 0) {
  free_stack_.reserve(num_blocks);
  // The stack hands out its back() first, so push the pop order reversed.
  for (int32_t i = num_blocks - 1; i >= 0; --i)
    free_stack_.push_back(pop_order.empty() ? i : pop_order[i]);
}

bool BlockManager::live(int32_t seq) const {
  return seq >= 0 && seq < static_cast<int32_t>(seqs_.size()) && seqs_[seq].live;
}

int32_t BlockManager::pop() {
  int32_t b = free_stack_.back();
  free_stack_.pop_back();
  return b;
}

MgrStatus BlockManager::seq_new(int32_t* seq) {
  if (seqs_.size() >= static_cast<size_t>(INT32_MAX)) return MgrStatus::range;
  seqs_.emplace_back();
  seqs_.back().live = true;
  *seq = static_cast<int32_t>(seqs_.size() - 1);
  return MgrStatus::ok;
}

MgrStatus BlockManager::seq_append(int32_t seq, int32_t n, int64_t* slots, int32_t* cow_pairs,
                                   int32_t cow_cap, int32_t* n_cow) {
  if (!live(seq) || n < 0) return MgrStatus::invalid;
  Seq& s = seqs_[seq];
  const int64_t L = s.length;
  if (L + n > INT32_MAX) return MgrStatus::range;
  const int64_t bs = block_size_;
  // Work out every block this append takes before changing anything.
  const bool cow = n > 0 && L % bs != 0 && refcount_[s.table.back()] > 1;
  const int64_t fresh = (L + n + bs - 1) / bs - (L + bs - 1) / bs;
  if (cow && cow_cap < 1) return MgrStatus::range;
  if (fresh + (cow ? 1 : 0) > static_cast<int64_t>(free_stack_.size())) return MgrStatus::no_blocks;

  *n_cow = 0;
  if (cow) {
    const int32_t shared = s.table.back();
    const int32_t copy = pop();
    refcount_[shared] -= 1;
    refcount_[copy] = 1;
    s.table.back() = copy;
    cow_pairs[0] = shared;
    cow_pairs[1] = copy;
    *n_cow = 1;
  }
  for (int64_t i = 0; i < n; ++i) {
    const int64_t pos = L + i;
    if (pos % bs == 0) {
      const int32_t b = pop();
      refcount_[b] = 1;
      s.table.push_back(b);
    }
    slots[i] = static_cast<int64_t>(s.table[pos / bs]) * bs + pos % bs;
  }
  s.length = static_cast<int32_t>(L + n);
  return MgrStatus::ok;
}

MgrStatus BlockManager::seq_append_batch(const int32_t* seqs, int32_t count, const int32_t* n,
                                         int64_t* slots, int32_t* cow_pairs, int32_t cow_cap,
                                         int32_t* n_cow) {
  // Work out what the whole batch takes before changing anything: copies depend on
  // reference counts that earlier copies in the batch lower.
  std::unordered_map<int32_t, int32_t> dropped;  // block -> references given up so far
  std::unordered_map<int32_t, char> seen;
  int64_t need = 0, copies = 0;
  const int64_t bs = block_size_;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t s = seqs[i];
    const int32_t k = n ? n[i] : 1;
    if (!live(s) || k < 0 || seen.count(s)) return MgrStatus::invalid;
    seen[s] = 1;
    const Seq& q = seqs_[s];
    const int64_t L = q.length;
    if (L + k > INT32_MAX) return MgrStatus::range;
    if (k > 0 && L % bs != 0) {
      const int32_t last = q.table.back();
      if (refcount_[last] - dropped[last] > 1) {
        ++dropped[last];
        ++copies;
      }
    }
    need += (L + k + bs - 1) / bs - (L + bs - 1) / bs;
  }
  if (copies > cow_cap) return MgrStatus::range;
  if (need + copies > static_cast<int64_t>(free_stack_.size())) return MgrStatus::no_blocks;

  int32_t made = 0;
  int64_t at = 0;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t k = n ? n[i] : 1;
    int32_t c = 0;
    seq_append(seqs[i], k, slots + at, cow_pairs + 2 * made, cow_cap - made, &c);
    made += c;
    at += k;
  }
  *n_cow = made;
  return MgrStatus::ok;
}

MgrStatus BlockManager::seq_release_before(int32_t seq, int32_t token, int32_t* released) {
  if (!live(seq) || token < 0) return MgrStatus::invalid;
  Seq& s = seqs_[seq];
  // Block j holds tokens [j * bs, (j + 1) * bs); it is wholly before `token` when
  // (j + 1) * bs <= token.  The last block of a sequence stays whatever `token` is.
  const int64_t whole = std::min<int64_t>(token / block_size_, static_cast<int64_t>(s.table.size()) - 1);
  int32_t n = 0;
  for (int64_t j = 0; j < whole; ++j) {
    const int32_t b = s.table[j];
    if (b < 0) continue;
    if (--refcount_[b] == 0) free_stack_.push_back(b);
    s.table[j] = -1;
    ++n;
  }
  *released = n;
  return MgrStatus::ok;
}

MgrStatus BlockManager::seq_fork(int32_t parent, int32_t* child) {
  if (!live(parent)) return MgrStatus::invalid;
  int32_t id;
  MgrStatus st = seq_new(&id);
  if (st != MgrStatus::ok) return st;
  Seq& c = seqs_[id];
  const Seq& p = seqs_[parent];  // re-read: seq_new may have moved the vector
  c.table = p.table;
  c.length = p.length;
  for (int32_t b : c.table)
    if (b >= 0) refcount_[b] += 1;
  *child = id;
  return MgrStatus::ok;
}

MgrStatus BlockManager::seq_free(int32_t seq) {
  if (!live(seq)) return MgrStatus::invalid;
  Seq& s = seqs_[seq];
  for (int32_t b : s.table) {
    if (b >= 0 && --refcount_[b] == 0) free_stack_.push_back(b);
  }
  s.live = false;
  s.length = 0;
  std::vector<int32_t>().swap(s.table);
  return MgrStatus::ok;
}

void BlockManager::free_stack_top_first(std::vector<int32_t>* out) const {
  out->assign(free_stack_.rbegin(), free_stack_.rend());
}

}  // namespace pa
