// Checks of the caller's preconditions that the kernels cannot afford: host-side, on host
// copies of the device arrays.  The library's debug build (PA_DEBUG) runs them inside the
// device calls before launching; every build exports them for callers (pa.h).
#pragma once

#include <cstdint>
#include <string>

namespace pa {

// Slots of one cache write: every slot in [0, num_slots) appears at most once (the
// writes of one call run concurrently, so two tokens aimed at one slot race).  Slots
// outside the range are skipped by the kernels and not checked.  Returns false and a
// message naming the slot and both token indices on the first repeat.
bool slots_are_unique(const int64_t* slots, int64_t n, int64_t num_slots, std::string* why);

// Copy pairs (src, dst) of one copy call: the pairs run concurrently, so each in-range
// destination appears once and is no in-range pair's source.  Pairs with an id outside
// [0, num_blocks) are skipped by the kernel and not checked.
bool copy_pairs_are_disjoint(const int32_t* pairs, int64_t n_pairs, int32_t num_blocks,
                             std::string* why);

}  // namespace pa
