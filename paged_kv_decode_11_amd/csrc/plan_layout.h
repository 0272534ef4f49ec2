// Fixed offsets of the plan image (pkd.h): slot_indptr right after the
// header, then the table of each slot's first item, then the merge list.
// They depend only on the slot count, so a decode workgroup can read its
// slot's bounds and its first item, and a merge workgroup its first merge
// entry, at once with the header, before they have read it.  The items
// follow the merge list (the header's PKD_H_OFF_ITEMS).
// Internal to the library; shared by the host planner and the kernels.
#pragma once

#include <cstdint>

#include "pkd.h"

namespace pkd {

// Query rows one workgroup of the shared-prefix kernel covers (8 waves of
// 16 rows): a row block holds 128 / gqa requests.
constexpr int kSharedRowsPerWorkgroup = 128;

constexpr int64_t plan_off_slots() { return PKD_HEADER_BASE + 32; }
constexpr int64_t plan_off_first(int64_t num_slots) {
  return (plan_off_slots() + num_slots + 1 + 7) / 8 * 8;
}
constexpr int64_t plan_off_merge(int64_t num_slots) {
  return plan_off_first(num_slots) + 8 * num_slots;
}
// items start at the first multiple of 8 past a merge list of n_merge entries
constexpr int64_t plan_off_items(int64_t num_slots, int64_t n_merge) {
  return (plan_off_merge(num_slots) + 4 * n_merge + 7) / 8 * 8;
}

}  // namespace pkd
