// Fixed offsets of the plan image (pkd.h): slot_indptr right after the
// header, then the table of each slot's first item, then the items.  They
// depend only on the slot count, so a decode workgroup can read its slot's
// bounds and its first item at once, before it has read the header.
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
constexpr int64_t plan_off_items(int64_t num_slots) {
  return plan_off_first(num_slots) + 8 * num_slots;
}

}  // namespace pkd
