// Host scheduler (see plan.h).
//
// The algorithm follows the pinghaoyang FlashInfer page, section
// "先切长 KV，再做最长任务优先分配" (split long KV, then longest-first
// assignment): a chunk bound equal to the total KV work over the fixed slot
// count, chunks cut along the sequence, cost C = alpha * l_q + beta * l_kv per
// chunk, items taken longest first and each given to the slot with the least
// accumulated cost, and a fixed reduction map instead of atomics.  Requests
// that fit in one chunk are not split and write their output directly
// ("writethrough", same page, section on split-KV; aicassindra "Load
// balancing with split-KV").
//
// Chunks are whole pages.  Derived chunk size:
//   cp = max(ceil(min_chunk_tokens / P), ceil(ceil(T / S) / P)).
// Ties: items ordered by (-cost, request, chunk); a slot is chosen by
// (load, slot id).  Split request i owns partial ids base_i .. base_i+k_i-1,
// base_i counting the chunks of the split requests before it.

#include "plan.h"

#include <algorithm>

#include "pkd.h"
#include "plan_layout.h"

namespace pkd {

namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t align_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Binary min-heap over (load, slot), written out so the tie rule is explicit.
struct SlotHeap {
  std::vector<int64_t>& load;
  std::vector<int32_t>& slot;
  int32_t n = 0;

  bool less(int32_t a, int32_t b) const {
    return load[a] < load[b] || (load[a] == load[b] && slot[a] < slot[b]);
  }
  void swap_nodes(int32_t a, int32_t b) {
    std::swap(load[a], load[b]);
    std::swap(slot[a], slot[b]);
  }
  void sift_down(int32_t i) {
    for (;;) {
      int32_t l = 2 * i + 1, r = l + 1, m = i;
      if (l < n && less(l, m)) m = l;
      if (r < n && less(r, m)) m = r;
      if (m == i) return;
      swap_nodes(i, m);
      i = m;
    }
  }
  // Slots 0..S-1 all at load 0 already form a heap in slot order.
  void init(int32_t S) {
    n = S;
    load.assign(S, 0);
    slot.resize(S);
    for (int32_t s = 0; s < S; ++s) slot[s] = s;
  }
  // Take the least-loaded slot, add `cost` to it, restore the heap.
  int32_t take(int64_t cost) {
    int32_t s = slot[0];
    load[0] += cost;
    sift_down(0);
    return s;
  }
};

}  // namespace

int64_t max_items(int64_t max_batch, int64_t num_slots) { return num_slots + 2 * max_batch; }

int64_t plan_image_ints(int64_t num_slots, int64_t num_items, int64_t n_split) {
  int64_t off_items = plan_off_items(num_slots);
  int64_t off_merge = off_items + 8 * num_items;
  return align_up(off_merge + 4 * n_split, 32);
}

int plan_validate(const PlanInput& in, std::string* err) {
  auto fail = [&](int code, const char* msg) {
    if (err) *err = msg;
    return code;
  };
  if (!in.indptr || !in.last) return fail(PKD_ERR_INVALID_ARG, "kv_indptr and kv_last_page_len must be non-null");
  if (in.batch < 1) return fail(PKD_ERR_INVALID_ARG, "batch must be >= 1");
  if (in.num_slots < 1) return fail(PKD_ERR_INVALID_ARG, "num_slots must be >= 1");
  if (in.page_size < 1) return fail(PKD_ERR_INVALID_ARG, "page_size must be >= 1");
  if (in.num_qo_heads < 1 || in.num_kv_heads < 1)
    return fail(PKD_ERR_INVALID_ARG, "head counts must be >= 1");
  if (in.num_qo_heads % in.num_kv_heads != 0)
    return fail(PKD_ERR_INVALID_ARG, "num_qo_heads must be a multiple of num_kv_heads");
  if (in.head_dim < 1) return fail(PKD_ERR_INVALID_ARG, "head_dim must be >= 1");
  if (in.indptr[0] != 0) return fail(PKD_ERR_INVALID_ARG, "kv_indptr[0] must be 0");
  for (int32_t i = 0; i < in.batch; ++i) {
    if (in.indptr[i + 1] - in.indptr[i] < 1)
      return fail(PKD_ERR_INVALID_ARG, "every request needs at least one page (kv_indptr must increase)");
    if (in.last[i] < 1 || in.last[i] > in.page_size)
      return fail(PKD_ERR_INVALID_ARG, "kv_last_page_len must lie in [1, page_size]");
  }
  return PKD_OK;
}

int plan_measure(const PlanInput& in, PlanScratch& s, PlanLayout* layout, std::string* err) {
  int rc = plan_validate(in, err);
  if (rc != PKD_OK) return rc;
  const int64_t P = in.page_size;
  const int64_t S = in.num_slots;
  const int64_t alpha = in.alpha < 0 ? 1 : in.alpha;
  const int64_t beta = in.beta <= 0 ? 1 : in.beta;
  const int64_t min_chunk = in.min_chunk_tokens <= 0 ? 128 : in.min_chunk_tokens;

  int64_t total = 0;
  for (int32_t i = 0; i < in.batch; ++i)
    total += P * (int64_t(in.indptr[i + 1] - in.indptr[i]) - 1) + in.last[i];

  int64_t cp = in.fixed_chunk_pages > 0
                   ? int64_t(in.fixed_chunk_pages)
                   : std::max<int64_t>({1, ceil_div(min_chunk, P), ceil_div(ceil_div(total, S), P)});
  if (cp > INT32_MAX) cp = INT32_MAX;

  s.items.clear();
  int32_t next_partial = 0, n_split = 0;
  for (int32_t i = 0; i < in.batch; ++i) {
    const int64_t n = in.indptr[i + 1] - in.indptr[i];
    const int64_t k = ceil_div(n, cp);
    const bool split = k > 1;
    const int32_t base = next_partial;
    if (split) {
      if (int64_t(next_partial) + k > INT32_MAX) {
        if (err) *err = "too many partial states";
        return PKD_ERR_INVALID_ARG;
      }
      next_partial += int32_t(k);
      ++n_split;
    }
    for (int64_t j = 0; j < k; ++j) {
      PlanItem it;
      it.request = i;
      it.chunk = int32_t(j);
      it.page_begin = int32_t(in.indptr[i] + j * cp);
      it.num_pages = int32_t(std::min<int64_t>(cp, n - j * cp));
      it.last_len = j == k - 1 ? in.last[i] : int32_t(P);
      it.length = int32_t((it.num_pages - 1) * P + it.last_len);
      it.out = split ? base + int32_t(j) : -1;
      it.cost = alpha + beta * it.length;
      s.items.push_back(it);
    }
  }
  const int64_t I = int64_t(s.items.size());
  layout->off_slots = plan_off_slots();
  layout->off_first = plan_off_first(S);
  layout->off_items = plan_off_items(S);
  layout->off_merge = layout->off_items + 8 * I;
  layout->off_indices = align_up(layout->off_merge + 4 * int64_t(n_split), 32);
  layout->nnz = in.indptr[in.batch];
  layout->total_tokens = total;
  layout->chunk_pages = int32_t(cp);
  layout->num_items = int32_t(I);
  layout->n_partials = next_partial;
  layout->n_split = n_split;
  return PKD_OK;
}

int plan_build(const PlanInput& in, PlanScratch& s, int32_t* image, int64_t image_ints,
               PlanLayout* layout, std::string* err) {
  int rc = plan_measure(in, s, layout, err);
  if (rc != PKD_OK) return rc;
  if (!image || image_ints < layout->off_indices) {
    if (err) *err = "plan image buffer too small for this plan";
    return PKD_ERR_WORKSPACE_TOO_SMALL;
  }
  const int32_t S = in.num_slots;
  const int32_t I = layout->num_items;

  // Longest first; ties by request, then chunk.
  s.order.resize(I);
  for (int32_t x = 0; x < I; ++x) s.order[x] = x;
  const std::vector<PlanItem>& items = s.items;
  std::sort(s.order.begin(), s.order.end(), [&](int32_t a, int32_t b) {
    const PlanItem& A = items[a];
    const PlanItem& B = items[b];
    if (A.cost != B.cost) return A.cost > B.cost;
    if (A.request != B.request) return A.request < B.request;
    return A.chunk < B.chunk;
  });

  // Each item to the least-loaded slot.
  SlotHeap heap{s.heap_load, s.heap_slot};
  heap.init(S);
  s.slot_of.resize(I);
  for (int32_t x = 0; x < I; ++x) s.slot_of[x] = heap.take(items[s.order[x]].cost);

  // Image: zero the device-only words and the header, then fill.
  std::fill(image, image + layout->off_indices, 0);
  int32_t* hdr = image + PKD_HEADER_BASE;
  hdr[PKD_H_MAGIC] = PKD_PLAN_MAGIC;
  hdr[PKD_H_VERSION] = PKD_PLAN_VERSION;
  hdr[PKD_H_BATCH] = in.batch;
  hdr[PKD_H_QO_HEADS] = in.num_qo_heads;
  hdr[PKD_H_KV_HEADS] = in.num_kv_heads;
  hdr[PKD_H_HEAD_DIM] = in.head_dim;
  hdr[PKD_H_PAGE_SIZE] = in.page_size;
  hdr[PKD_H_SLOTS] = S;
  hdr[PKD_H_CHUNK_PAGES] = layout->chunk_pages;
  hdr[PKD_H_ITEMS] = I;
  hdr[PKD_H_PARTIALS] = layout->n_partials;
  hdr[PKD_H_SPLIT] = layout->n_split;
  hdr[PKD_H_ALPHA] = in.alpha < 0 ? 1 : in.alpha;
  hdr[PKD_H_BETA] = in.beta <= 0 ? 1 : in.beta;
  hdr[PKD_H_NNZ] = int32_t(layout->nnz);
  hdr[PKD_H_PLAN_ID] = int32_t(in.plan_id & 0x7fffffff);
  hdr[PKD_H_OFF_SLOTS] = int32_t(layout->off_slots);
  hdr[PKD_H_OFF_ITEMS] = int32_t(layout->off_items);
  hdr[PKD_H_OFF_MERGE] = int32_t(layout->off_merge);
  hdr[PKD_H_OFF_INDICES] = int32_t(layout->off_indices);
  hdr[PKD_H_TOTAL_TOKENS_LO] = int32_t(layout->total_tokens & 0xffffffff);
  hdr[PKD_H_TOTAL_TOKENS_HI] = int32_t(layout->total_tokens >> 32);
  hdr[PKD_H_OFF_FIRST] = int32_t(layout->off_first);

  int32_t* slot_indptr = image + layout->off_slots;
  for (int32_t q = 0; q <= S; ++q) slot_indptr[q] = 0;
  for (int32_t x = 0; x < I; ++x) ++slot_indptr[s.slot_of[x] + 1];
  for (int32_t q = 0; q < S; ++q) slot_indptr[q + 1] += slot_indptr[q];

  // Per-slot lists in assignment order.
  s.cursor.assign(slot_indptr, slot_indptr + S);
  int32_t* out_items = image + layout->off_items;
  for (int32_t x = 0; x < I; ++x) {
    const PlanItem& it = items[s.order[x]];
    int32_t* row = out_items + 8 * int64_t(s.cursor[s.slot_of[x]]++);
    row[0] = it.request;
    row[1] = it.page_begin;
    row[2] = it.num_pages;
    row[3] = it.last_len;
    row[4] = it.out;
    row[5] = it.length;
  }
  int32_t* first = image + layout->off_first;
  for (int32_t q = 0; q < S; ++q)
    if (slot_indptr[q] < slot_indptr[q + 1])
      std::copy(out_items + 8 * int64_t(slot_indptr[q]), out_items + 8 * int64_t(slot_indptr[q]) + 8,
                first + 8 * int64_t(q));

  // Reduction map: split requests in ascending order.
  int32_t* merge = image + layout->off_merge;
  int32_t e = 0;
  for (int32_t x = 0; x < I; ++x) {
    const PlanItem& it = items[x];  // request/chunk order
    if (it.out >= 0 && it.chunk == 0) {
      int32_t k = 1;
      while (x + k < I && items[x + k].request == it.request) ++k;
      merge[4 * e + 0] = it.request;
      merge[4 * e + 1] = it.out;
      merge[4 * e + 2] = k;
      ++e;
    }
  }
  return PKD_OK;
}

}  // namespace pkd
