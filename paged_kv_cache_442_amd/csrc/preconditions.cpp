#include "preconditions.hpp"

#include <cstdio>
#include <unordered_map>
#include <unordered_set>

namespace pa {

bool slots_are_unique(const int64_t* slots, int64_t n, int64_t num_slots, std::string* why) {
  std::unordered_map<int64_t, int64_t> first;  // slot -> first token index writing it
  first.reserve(static_cast<size_t>(n));
  for (int64_t t = 0; t < n; ++t) {
    const int64_t s = slots[t];
    if (s < 0 || s >= num_slots) continue;
    const auto ins = first.emplace(s, t);
    if (!ins.second) {
      char buf[160];
      std::snprintf(buf, sizeof buf, "slot %lld is written by tokens %lld and %lld",
                    static_cast<long long>(s), static_cast<long long>(ins.first->second),
                    static_cast<long long>(t));
      *why = buf;
      return false;
    }
  }
  return true;
}

bool copy_pairs_are_disjoint(const int32_t* pairs, int64_t n_pairs, int32_t num_blocks,
                             std::string* why) {
  auto in_range = [&](int32_t b) { return b >= 0 && b < num_blocks; };
  std::unordered_map<int32_t, int64_t> dst_at;
  std::unordered_set<int32_t> srcs;
  for (int64_t i = 0; i < n_pairs; ++i) {
    const int32_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (!in_range(s) || !in_range(d)) continue;
    srcs.insert(s);
    const auto ins = dst_at.emplace(d, i);
    if (!ins.second) {
      char buf[160];
      std::snprintf(buf, sizeof buf, "block %d is the destination of pairs %lld and %lld", d,
                    static_cast<long long>(ins.first->second), static_cast<long long>(i));
      *why = buf;
      return false;
    }
  }
  for (int64_t i = 0; i < n_pairs; ++i) {
    const int32_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (in_range(s) && in_range(d) && srcs.count(d)) {
      char buf[160];
      std::snprintf(buf, sizeof buf, "block %d is the destination of pair %lld and also a source",
                    d, static_cast<long long>(i));
      *why = buf;
      return false;
    }
  }
  return true;
}

}  // namespace pa
