// Host scheduler for paged GQA decode: validation, split-KV chunking,
// longest-first assignment of chunks to a fixed set of slots, and the
// reduction map.  Plain C++17, no HIP: it runs (and is tested) without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "pkd.h"

namespace pkd {

// A decode plan has one KV row per request.  A shared-prefix plan (qo_indptr
// non-null) has one KV row per group of requests: group g's requests are rows
// qo_indptr[g] .. qo_indptr[g+1]-1 of q, and all of them attend to the
// group's pages.
struct PlanInput {
  const int32_t* indptr = nullptr;     // [batch+1], host
  const int32_t* last = nullptr;       // [batch], host
  const int32_t* qo_indptr = nullptr;  // [batch+1], host; shared-prefix plans only
  int32_t batch = 0;                   // KV rows: requests, or groups
  int32_t num_qo_heads = 0;
  int32_t num_kv_heads = 0;
  int32_t head_dim = 0;
  int32_t page_size = 0;
  int32_t num_slots = 0;
  int32_t fixed_chunk_pages = 0;
  int32_t min_chunk_tokens = 128;
  int32_t alpha = 1;
  int32_t beta = 1;
  int32_t flags = 0;  // PKD_PLAN_* (PKD_PLAN_ALL_PARTIALS: every row writes partial states)
  int64_t plan_id = 0;
};

struct PlanLayout {
  int32_t kind = PKD_PLAN_DECODE;
  int32_t num_requests = 0;  // rows of q the plan's runs read
  int32_t num_groups = 0;    // shared-prefix plans: KV rows (groups)
  int32_t rows_per_block = 1;
  int64_t off_slots = 0;
  int64_t off_first = 0;
  int64_t off_items = 0;
  int64_t off_merge = 0;
  int64_t off_groups = 0;
  int64_t off_indices = 0;  // == ints in the plan image
  int64_t nnz = 0;
  int64_t total_tokens = 0;
  int32_t chunk_pages = 0;
  int32_t num_items = 0;
  int32_t n_partials = 0;
  int32_t n_split = 0;
};

struct PlanItem {
  int64_t cost;
  int32_t request, chunk, page_begin, num_pages, last_len, length, out;  // request: KV row
  int32_t block = 0, head = 0;  // shared-prefix plans: row block and KV head
};

// One entry of the reduction map: `k` partial states of `request` from id
// `first` on.
struct PlanMerge {
  int32_t request, first, k;
};

// Shared-prefix plans: per group, its first request row, its request count,
// its chunk count and its first partial id (-1 when not split).
struct PlanGroup {
  int32_t row0, rows, k, base;
};

// Reused host memory, so steady-state planning does not allocate.
struct PlanScratch {
  std::vector<PlanItem> items;
  std::vector<PlanMerge> merges;
  std::vector<PlanGroup> groups;
  std::vector<int32_t> order;
  std::vector<int32_t> slot_of;  // slot of each item, by position in `order`
  std::vector<int64_t> heap_load;
  std::vector<int32_t> heap_slot;
  std::vector<int32_t> cursor;
};

// Check the page table and shapes; on failure return a pkd_status code and
// set *err.
int plan_validate(const PlanInput& in, std::string* err);

// Chunks and counts only (no assignment): fills *layout.
int plan_measure(const PlanInput& in, PlanScratch& s, PlanLayout* layout, std::string* err);

// Full schedule into `image` (capacity `image_ints` int32), laid out as the
// plan image of pkd.h: ints [0, layout.off_indices).  Calls plan_measure.
int plan_build(const PlanInput& in, PlanScratch& s, int32_t* image, int64_t image_ints,
               PlanLayout* layout, std::string* err);

// Worst-case counts used by the workspace-size functions.
int64_t max_items(int64_t max_batch, int64_t num_slots);
// Shared-prefix plans with derived chunks: at most
// S + 2 Hkv (max_groups + ceil(max_requests gqa / 128)) items, and
// max_requests (S / Hkv + 2) partial states.
int64_t max_items_shared(int64_t max_groups, int64_t max_requests, int64_t num_slots,
                         int64_t num_qo_heads, int64_t num_kv_heads);
int64_t max_partials_shared(int64_t max_requests, int64_t num_slots, int64_t num_kv_heads);
int64_t plan_image_ints(int64_t num_slots, int64_t num_items, int64_t n_merge,
                        int64_t num_groups = 0);

}  // namespace pkd
