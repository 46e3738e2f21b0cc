// Random-operation run of the host block manager, built by tests/test_manager_sanitizers.py
// with AddressSanitizer and UndefinedBehaviorSanitizer (host code only, g++).  Every
// operation of the manager is exercised (appends with and without token ids, batch
// appends, prefix lookups, forks, window releases, frees, swap-out / swap-in) on a small
// pool, and the manager's own accounting is checked after each step:
//   * every block is in exactly one state, and the free stack plus the evictable list
//     plus the blocks in use cover the pool;
//   * a block's reference count equals the number of resident live sequences that hold
//     it; a host block's equals the number of swapped-out sequences that hold it.
// Usage: manager_fuzz SEED STEPS
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "block_manager.hpp"

using pa::BlockManager;
using pa::BlockState;
using pa::MgrStatus;

namespace {

int fail(const char* what, long step) {
  std::fprintf(stderr, "invariant broken at step %ld: %s\n", step, what);
  return 1;
}

}  // namespace

int main(int argc, char** argv) {
  const unsigned seed = argc > 1 ? static_cast<unsigned>(std::atoi(argv[1])) : 1u;
  const long steps = argc > 2 ? std::atol(argv[2]) : 20000;
  std::mt19937 rng(seed);
  auto uni = [&](int n) { return static_cast<int>(rng() % static_cast<unsigned>(n)); };

  const int N = 48, bs = 2 + uni(3) * 2, M = 24;
  std::vector<int32_t> order(N);
  for (int i = 0; i < N; ++i) order[i] = i;
  for (int i = N - 1; i > 0; --i) std::swap(order[i], order[uni(i + 1)]);
  BlockManager m(N, bs, order);
  const bool caching = seed % 2 == 0;
  if (caching && m.enable_prefix_caching() != MgrStatus::ok) return fail("enable", -1);
  if (m.set_swap_space(M) != MgrStatus::ok) return fail("swap space", -1);

  std::vector<int32_t> live;  // live sequence ids
  std::vector<std::vector<int32_t>> prompts(4);
  for (auto& p : prompts) {
    const int n = 1 + uni(4 * bs);
    for (int i = 0; i < n; ++i) p.push_back(uni(6));
  }
  constexpr int kCap = 1024;
  std::vector<int64_t> slots(kCap);
  std::vector<int32_t> pairs(2 * kCap), toks(kCap);

  for (long step = 0; step < steps; ++step) {
    const int r = uni(100);
    int32_t seq = -1;
    if (!live.empty()) seq = live[uni(static_cast<int>(live.size()))];
    int32_t n_cow = 0, out = 0, cached = 0;
    if (r < 15 || live.empty()) {
      if (caching && uni(2)) {
        std::vector<int32_t> p = prompts[uni(4)];
        const int extra = uni(2 * bs);
        for (int i = 0; i < extra; ++i) p.push_back(uni(6));
        if (m.seq_new_prefix(p.data(), static_cast<int32_t>(p.size()), &seq, &cached) != MgrStatus::ok)
          return fail("new prefix", step);
        const int rest = static_cast<int>(p.size()) - cached;
        (void)m.seq_append(seq, rest, p.data() + cached, slots.data(), pairs.data(), 1, &n_cow);
      } else if (m.seq_new(&seq) != MgrStatus::ok) {
        return fail("new", step);
      }
      live.push_back(seq);
    } else if (r < 45) {
      const int k = uni(3 * bs);
      for (int i = 0; i < k; ++i) toks[i] = uni(6);
      (void)m.seq_append(seq, k, uni(8) ? toks.data() : nullptr, slots.data(), pairs.data(), 1, &n_cow);
    } else if (r < 55) {
      std::vector<int32_t> batch, counts;
      int total = 0;
      for (int32_t s : live)
        if (uni(2) && !m.swapped(s) && total + 2 < kCap) {
          batch.push_back(s);
          counts.push_back(uni(3));
          total += counts.back();
        }
      for (int i = 0; i < total; ++i) toks[i] = uni(6);
      (void)m.seq_append_batch(batch.data(), static_cast<int32_t>(batch.size()), counts.data(),
                               toks.data(), slots.data(), pairs.data(), kCap, &n_cow);
    } else if (r < 63) {
      if (m.seq_fork(seq, &out) == MgrStatus::ok) live.push_back(out);
    } else if (r < 70) {
      (void)m.seq_release_before(seq, uni(m.length(seq) + 1), &out);
    } else if (r < 80) {
      (void)m.seq_swap_out(&seq, 1, pairs.data(), kCap, &out);
    } else if (r < 88) {
      (void)m.seq_swap_in(&seq, 1, pairs.data(), kCap, &out);
    } else {
      if (m.seq_free(seq) != MgrStatus::ok) return fail("free", step);
      for (size_t i = 0; i < live.size(); ++i)
        if (live[i] == seq) {
          live.erase(live.begin() + static_cast<long>(i));
          break;
        }
    }

    // Accounting.
    std::vector<int32_t> held(N, 0), host_held(M, 0);
    for (int32_t s : live) {
      for (int32_t b : m.table(s)) {
        if (b < 0) continue;
        if (m.swapped(s)) {
          if (b >= M) return fail("host block out of range", step);
          ++host_held[b];
        } else {
          if (b >= N) return fail("block out of range", step);
          ++held[b];
        }
      }
    }
    std::vector<int32_t> stack, lru;
    m.free_stack_top_first(&stack);
    m.evictable_lru_first(&lru);
    std::vector<int> seen(N, 0);
    for (int32_t b : stack) {
      if (b < 0 || b >= N || seen[b]++) return fail("free stack entry", step);
      if (m.state(b) != BlockState::free_empty) return fail("free stack state", step);
    }
    for (int32_t b : lru) {
      if (b < 0 || b >= N || seen[b]++) return fail("evictable entry", step);
      if (m.state(b) != BlockState::free_cached) return fail("evictable state", step);
    }
    for (int b = 0; b < N; ++b) {
      if (m.refcount(b) != held[b]) return fail("refcount", step);
      if ((held[b] > 0) == (seen[b] > 0)) return fail("block in use and free, or neither", step);
    }
    if (m.num_free() != static_cast<int32_t>(stack.size() + lru.size())) return fail("num_free", step);
    std::vector<int32_t> hstack;
    m.host_free_stack_top_first(&hstack);
    std::vector<int> hseen(M, 0);
    for (int32_t h : hstack)
      if (h < 0 || h >= M || hseen[h]++ || host_held[h]) return fail("host free stack", step);
    for (int h = 0; h < M; ++h) {
      if (m.host_refcount(h) != host_held[h]) return fail("host refcount", step);
      if ((host_held[h] > 0) == (hseen[h] > 0)) return fail("host block in use and free", step);
    }
  }
  std::printf("ok seed %u steps %ld caching %d block_size %d\n", seed, steps, caching ? 1 : 0, bs);
  return 0;
}
