// Host scheduler for paged GQA decode: validation, split-KV chunking,
// longest-first assignment of chunks to a fixed set of slots, and the
// reduction map.  Plain C++17, no HIP: it runs (and is tested) without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace pkd {

struct PlanInput {
  const int32_t* indptr = nullptr;  // [batch+1], host
  const int32_t* last = nullptr;    // [batch], host
  int32_t batch = 0;
  int32_t num_qo_heads = 0;
  int32_t num_kv_heads = 0;
  int32_t head_dim = 0;
  int32_t page_size = 0;
  int32_t num_slots = 0;
  int32_t fixed_chunk_pages = 0;
  int32_t min_chunk_tokens = 128;
  int32_t alpha = 1;
  int32_t beta = 1;
  int64_t plan_id = 0;
};

struct PlanLayout {
  int64_t off_slots = 0;
  int64_t off_first = 0;
  int64_t off_items = 0;
  int64_t off_merge = 0;
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
  int32_t request, chunk, page_begin, num_pages, last_len, length, out;
};

// Reused host memory, so steady-state planning does not allocate.
struct PlanScratch {
  std::vector<PlanItem> items;
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
int64_t plan_image_ints(int64_t num_slots, int64_t num_items, int64_t n_split);

}  // namespace pkd
