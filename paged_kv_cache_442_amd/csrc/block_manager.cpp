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

MgrStatus BlockManager::enable_prefix_caching() {
  for (const Seq& s : seqs_)
    if (s.live) return MgrStatus::invalid;
  if (caching_) return MgrStatus::ok;
  caching_ = true;
  node_of_block_.assign(num_blocks_, -1);
  lru_prev_.assign(num_blocks_, -1);
  lru_next_.assign(num_blocks_, -1);
  return MgrStatus::ok;
}

// ------------------------------------------------------------------ free lists

int32_t BlockManager::pop() {
  // Empty blocks first; only then the least recently used cached block, whose cached
  // identity is dropped.  Callers have checked that num_free() covers every pop.
  if (!free_stack_.empty()) {
    const int32_t b = free_stack_.back();
    free_stack_.pop_back();
    return b;
  }
  const int32_t b = lru_head_;
  lru_remove(b);
  const int64_t n = node_of_block_[b];
  node_of_block_[b] = -1;
  nodes_[n].block = -1;
  unref(n);
  return b;
}

void BlockManager::release(int32_t block) {
  if (--refcount_[block] != 0) return;
  if (caching_ && node_of_block_[block] >= 0)
    lru_push_back(block);
  else
    free_stack_.push_back(block);
}

void BlockManager::lru_push_back(int32_t b) {
  lru_prev_[b] = lru_tail_;
  lru_next_[b] = -1;
  if (lru_tail_ >= 0)
    lru_next_[lru_tail_] = b;
  else
    lru_head_ = b;
  lru_tail_ = b;
  ++lru_size_;
}

void BlockManager::lru_remove(int32_t b) {
  const int32_t p = lru_prev_[b], n = lru_next_[b];
  if (p >= 0) lru_next_[p] = n; else lru_head_ = n;
  if (n >= 0) lru_prev_[n] = p; else lru_tail_ = p;
  lru_prev_[b] = lru_next_[b] = -1;
  --lru_size_;
}

// ------------------------------------------------------------------ identities

size_t BlockManager::KeyHash::operator()(const std::pair<int64_t, std::vector<int32_t>>& k) const {
  // splitmix64 finalizer folded over the parent id and the tokens.
  auto mix = [](uint64_t z) {
    z += 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
  };
  uint64_t h = mix(static_cast<uint64_t>(k.first));
  for (int32_t t : k.second) h = mix(h ^ static_cast<uint32_t>(t));
  return static_cast<size_t>(h);
}

int64_t BlockManager::find_node(int64_t parent, const int32_t* tokens) const {
  const auto it = node_index_.find({parent, std::vector<int32_t>(tokens, tokens + block_size_)});
  return it == node_index_.end() ? -1 : it->second;
}

int64_t BlockManager::intern(int64_t parent, const int32_t* tokens) {
  std::vector<int32_t> key(tokens, tokens + block_size_);
  const auto it = node_index_.find({parent, key});
  if (it != node_index_.end()) return it->second;
  int64_t id;
  if (!free_nodes_.empty()) {
    id = free_nodes_.back();
    free_nodes_.pop_back();
  } else {
    id = static_cast<int64_t>(nodes_.size());
    nodes_.emplace_back();
  }
  nodes_[id] = Node{parent, key, -1, 0};
  if (parent >= 0) nodes_[parent].refs += 1;  // the child's link
  node_index_.emplace(std::make_pair(parent, std::move(key)), id);
  return id;
}

void BlockManager::unref(int64_t n) {
  // A node with no cached block, no child and no sequence ending on it is erased, which
  // drops its link on the parent in turn.
  while (n >= 0) {
    if (--nodes_[n].refs > 0) return;
    Node& node = nodes_[n];
    const int64_t parent = node.parent;
    node_index_.erase({parent, node.tokens});
    std::vector<int32_t>().swap(node.tokens);
    free_nodes_.push_back(n);
    n = parent;
  }
}

void BlockManager::block_filled(Seq& s, int32_t block) {
  const int64_t id = intern(s.node, s.tail.data());
  nodes_[id].refs += 1;  // the sequence now ends on this identity
  if (s.node >= 0) unref(s.node);
  s.node = id;
  s.tail.clear();
  if (nodes_[id].block < 0) {  // the first block with this identity is the cached one
    nodes_[id].block = block;
    nodes_[id].refs += 1;
    node_of_block_[block] = id;
  }
}

BlockState BlockManager::state(int32_t block) const {
  if (refcount_[block] > 0) return BlockState::in_use;
  return cached(block) ? BlockState::free_cached : BlockState::free_empty;
}

// ------------------------------------------------------------------ sequences

MgrStatus BlockManager::seq_new(int32_t* seq) {
  if (seqs_.size() >= static_cast<size_t>(INT32_MAX)) return MgrStatus::range;
  seqs_.emplace_back();
  seqs_.back().live = true;
  *seq = static_cast<int32_t>(seqs_.size() - 1);
  return MgrStatus::ok;
}

MgrStatus BlockManager::seq_new_prefix(const int32_t* prompt, int32_t n_prompt, int32_t* seq,
                                       int32_t* cached) {
  if (!caching_ || n_prompt < 0 || (n_prompt > 0 && !prompt)) return MgrStatus::invalid;
  int32_t id;
  const MgrStatus st = seq_new(&id);
  if (st != MgrStatus::ok) return st;
  Seq& s = seqs_[id];
  const int32_t max_hits = n_prompt > 0 ? (n_prompt - 1) / block_size_ : 0;
  int64_t node = -1;
  for (int32_t j = 0; j < max_hits; ++j) {
    const int64_t child = find_node(node, prompt + static_cast<int64_t>(j) * block_size_);
    if (child < 0 || nodes_[child].block < 0) break;
    const int32_t b = nodes_[child].block;
    if (refcount_[b] == 0) lru_remove(b);
    refcount_[b] += 1;
    s.table.push_back(b);
    node = child;
  }
  s.node = node;
  if (node >= 0) nodes_[node].refs += 1;
  s.length = static_cast<int32_t>(s.table.size()) * block_size_;
  *seq = id;
  *cached = s.length;
  return MgrStatus::ok;
}

MgrStatus BlockManager::seq_append(int32_t seq, int32_t n, const int32_t* tokens, int64_t* slots,
                                   int32_t* cow_pairs, int32_t cow_cap, int32_t* n_cow) {
  if (!live(seq) || n < 0 || seqs_[seq].swapped) return MgrStatus::invalid;
  Seq& s = seqs_[seq];
  const int64_t L = s.length;
  if (L + n > INT32_MAX) return MgrStatus::range;
  const int64_t bs = block_size_;
  // Work out every block this append takes before changing anything.
  const bool cow = n > 0 && L % bs != 0 && refcount_[s.table.back()] > 1;
  const int64_t fresh = (L + n + bs - 1) / bs - (L + bs - 1) / bs;
  if (cow && cow_cap < 1) return MgrStatus::range;
  if (fresh + (cow ? 1 : 0) > static_cast<int64_t>(num_free())) return MgrStatus::no_blocks;

  if (caching_ && s.tracked && n > 0 && !tokens) {
    // Ids unknown from here on: this sequence's later blocks are never cached.
    s.tracked = false;
    if (s.node >= 0) unref(s.node);
    s.node = -1;
    std::vector<int32_t>().swap(s.tail);
  }
  const bool track = caching_ && s.tracked;

  *n_cow = 0;
  if (cow) {
    const int32_t shared = s.table.back();
    const int32_t copy = pop();
    refcount_[shared] -= 1;  // stays above zero: it had more than one holder
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
    if (track) {
      s.tail.push_back(tokens[i]);
      if ((pos + 1) % bs == 0) block_filled(s, s.table[pos / bs]);
    }
  }
  s.length = static_cast<int32_t>(L + n);
  return MgrStatus::ok;
}

MgrStatus BlockManager::seq_append_batch(const int32_t* seqs, int32_t count, const int32_t* n,
                                         const int32_t* tokens, int64_t* slots, int32_t* cow_pairs,
                                         int32_t cow_cap, int32_t* n_cow) {
  // Work out what the whole batch takes before changing anything: copies depend on
  // reference counts that earlier copies in the batch lower.  An append frees nothing,
  // so once the total fits, every append of the batch succeeds.
  std::unordered_map<int32_t, int32_t> dropped;  // block -> references given up so far
  std::unordered_map<int32_t, char> seen;
  int64_t need = 0, copies = 0;
  const int64_t bs = block_size_;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t s = seqs[i];
    const int32_t k = n ? n[i] : 1;
    if (!live(s) || k < 0 || seen.count(s) || seqs_[s].swapped) return MgrStatus::invalid;
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
  if (need + copies > static_cast<int64_t>(num_free())) return MgrStatus::no_blocks;

  int32_t made = 0;
  int64_t at = 0;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t k = n ? n[i] : 1;
    int32_t c = 0;
    seq_append(seqs[i], k, tokens ? tokens + at : nullptr, slots + at, cow_pairs + 2 * made,
               cow_cap - made, &c);
    made += c;
    at += k;
  }
  *n_cow = made;
  return MgrStatus::ok;
}

MgrStatus BlockManager::seq_release_before(int32_t seq, int32_t token, int32_t* released) {
  if (!live(seq) || token < 0 || seqs_[seq].swapped) return MgrStatus::invalid;
  Seq& s = seqs_[seq];
  // Block j holds tokens [j * bs, (j + 1) * bs); it is wholly before `token` when
  // (j + 1) * bs <= token.  The last block of a sequence stays whatever `token` is.
  const int64_t whole = std::min<int64_t>(token / block_size_, static_cast<int64_t>(s.table.size()) - 1);
  int32_t n = 0;
  for (int64_t i = 0; i < whole; ++i) {
    const int64_t j = caching_ ? whole - 1 - i : i;  // last to first when caching
    const int32_t b = s.table[j];
    if (b < 0) continue;
    release(b);
    s.table[j] = -1;
    ++n;
  }
  *released = n;
  return MgrStatus::ok;
}

MgrStatus BlockManager::seq_fork(int32_t parent, int32_t* child) {
  if (!live(parent) || seqs_[parent].swapped) return MgrStatus::invalid;
  int32_t id;
  MgrStatus st = seq_new(&id);
  if (st != MgrStatus::ok) return st;
  Seq& c = seqs_[id];
  const Seq& p = seqs_[parent];  // re-read: seq_new may have moved the vector
  c.table = p.table;
  c.length = p.length;
  c.tracked = p.tracked;
  c.node = p.node;
  c.tail = p.tail;
  if (c.node >= 0) nodes_[c.node].refs += 1;
  for (int32_t b : c.table)
    if (b >= 0) refcount_[b] += 1;
  *child = id;
  return MgrStatus::ok;
}

MgrStatus BlockManager::seq_free(int32_t seq) {
  if (!live(seq)) return MgrStatus::invalid;
  Seq& s = seqs_[seq];
  const size_t nb = s.table.size();
  if (s.swapped) {
    for (int32_t h : s.table)
      if (h >= 0 && --host_refcount_[h] == 0) host_free_.push_back(h);
  } else {
    for (size_t i = 0; i < nb; ++i) {
      const int32_t b = s.table[caching_ ? nb - 1 - i : i];  // last to first when caching
      if (b >= 0) release(b);
    }
  }
  if (s.node >= 0) unref(s.node);
  s = Seq();
  return MgrStatus::ok;
}

// ------------------------------------------------------------------ swap

MgrStatus BlockManager::set_swap_space(int32_t host_blocks) {
  if (host_blocks < 0) return MgrStatus::invalid;
  for (const Seq& s : seqs_)
    if (s.live && s.swapped) return MgrStatus::invalid;
  host_refcount_.assign(host_blocks, 0);
  host_free_.clear();
  for (int32_t i = host_blocks - 1; i >= 0; --i) host_free_.push_back(i);  // 0 first
  return MgrStatus::ok;
}

MgrStatus BlockManager::seq_swap_out(const int32_t* seqs, int32_t count, int32_t* pairs,
                                     int32_t cap, int32_t* n_pairs) {
  std::unordered_map<int32_t, int32_t> to_host;  // device block -> host block
  for (int32_t i = 0; i < count; ++i) {
    const int32_t q = seqs[i];
    if (!live(q) || seqs_[q].swapped) return MgrStatus::invalid;
    for (int32_t k = 0; k < i; ++k)
      if (seqs[k] == q) return MgrStatus::invalid;
    for (int32_t b : seqs_[q].table)
      if (b >= 0) to_host.emplace(b, -1);
  }
  const int64_t need = static_cast<int64_t>(to_host.size());
  if (need > cap) return MgrStatus::range;
  if (need > static_cast<int64_t>(host_free_.size())) return MgrStatus::no_blocks;

  int32_t made = 0;
  for (int32_t i = 0; i < count; ++i) {
    Seq& s = seqs_[seqs[i]];
    const std::vector<int32_t> device = s.table;
    for (int32_t& e : s.table) {
      if (e < 0) continue;
      int32_t& h = to_host[e];
      if (h < 0) {
        h = host_free_.back();
        host_free_.pop_back();
        pairs[2 * made] = e;
        pairs[2 * made + 1] = h;
        ++made;
      }
      host_refcount_[h] += 1;
      e = h;
    }
    const size_t nb = device.size();
    for (size_t k = 0; k < nb; ++k) {
      const int32_t b = device[caching_ ? nb - 1 - k : k];  // as a free would
      if (b >= 0) release(b);
    }
    s.swapped = true;
  }
  *n_pairs = made;
  return MgrStatus::ok;
}

MgrStatus BlockManager::seq_swap_in(const int32_t* seqs, int32_t count, int32_t* pairs,
                                    int32_t cap, int32_t* n_pairs) {
  std::unordered_map<int32_t, int32_t> to_device;  // host block -> device block
  for (int32_t i = 0; i < count; ++i) {
    const int32_t q = seqs[i];
    if (!live(q) || !seqs_[q].swapped) return MgrStatus::invalid;
    for (int32_t k = 0; k < i; ++k)
      if (seqs[k] == q) return MgrStatus::invalid;
    for (int32_t h : seqs_[q].table)
      if (h >= 0) to_device.emplace(h, -1);
  }
  const int64_t need = static_cast<int64_t>(to_device.size());
  if (need > cap) return MgrStatus::range;
  if (need > static_cast<int64_t>(num_free())) return MgrStatus::no_blocks;

  int32_t made = 0;
  for (int32_t i = 0; i < count; ++i) {
    Seq& s = seqs_[seqs[i]];
    const std::vector<int32_t> host = s.table;
    for (int32_t& e : s.table) {
      if (e < 0) continue;
      int32_t& b = to_device[e];
      if (b < 0) {
        b = pop();
        pairs[2 * made] = e;
        pairs[2 * made + 1] = b;
        ++made;
      }
      refcount_[b] += 1;
      e = b;
    }
    for (int32_t h : host)
      if (h >= 0 && --host_refcount_[h] == 0) host_free_.push_back(h);
    s.swapped = false;
  }
  *n_pairs = made;
  return MgrStatus::ok;
}

void BlockManager::host_free_stack_top_first(std::vector<int32_t>* out) const {
  out->assign(host_free_.rbegin(), host_free_.rend());
}

void BlockManager::free_stack_top_first(std::vector<int32_t>* out) const {
  out->assign(free_stack_.rbegin(), free_stack_.rend());
}

void BlockManager::evictable_lru_first(std::vector<int32_t>* out) const {
  out->clear();
  for (int32_t b = lru_head_; b >= 0; b = lru_next_[b]) out->push_back(b);
}

}  // namespace pa
