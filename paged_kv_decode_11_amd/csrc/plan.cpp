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
#include <cstdint>

#include "pkd.h"
#include "plan_layout.h"

namespace pkd {

namespace {

static_assert(PKD_H_COUNT <= 32, "the header fills the 32 words before slot_indptr");

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
    // saturate: cost weights near 2^31 on long chunks could otherwise
    // overflow a slot's sum
    load[0] = load[0] > INT64_MAX - cost ? INT64_MAX : load[0] + cost;
    sift_down(0);
    return s;
  }
};

}  // namespace

int64_t max_items(int64_t max_batch, int64_t num_slots) { return num_slots + 2 * max_batch; }

int64_t max_items_shared(int64_t max_groups, int64_t max_requests, int64_t num_slots,
                         int64_t num_qo_heads, int64_t num_kv_heads) {
  const int64_t gqa = num_qo_heads / num_kv_heads;
  return num_slots + 2 * num_kv_heads * (max_groups + ceil_div(max_requests * gqa, 128));
}

int64_t max_partials_shared(int64_t max_requests, int64_t num_slots, int64_t num_kv_heads) {
  return max_requests * (ceil_div(num_slots, num_kv_heads) + 2);
}

int64_t plan_image_ints(int64_t num_slots, int64_t num_items, int64_t n_merge,
                        int64_t num_groups) {
  const int64_t off_items = plan_off_items(num_slots, n_merge);
  return align_up(off_items + 8 * num_items + 4 * num_groups, 32);
}

int plan_validate(const PlanInput& in, std::string* err) {
  auto fail = [&](int code, const char* msg) {
    if (err) *err = msg;
    return code;
  };
  if (!in.indptr || !in.last) return fail(PKD_ERR_INVALID_ARG, "kv_indptr and kv_last_page_len must be non-null");
  if (in.batch < 1) return fail(PKD_ERR_INVALID_ARG, "batch must be >= 1");
  if (in.num_slots < 1) return fail(PKD_ERR_INVALID_ARG, "num_slots must be >= 1");
  if (in.flags & ~int32_t(PKD_PLAN_ALL_PARTIALS)) return fail(PKD_ERR_INVALID_ARG, "unknown plan flags");
  if (in.page_size < 1) return fail(PKD_ERR_INVALID_ARG, "page_size must be >= 1");
  if (in.num_qo_heads < 1 || in.num_kv_heads < 1)
    return fail(PKD_ERR_INVALID_ARG, "head counts must be >= 1");
  if (in.num_qo_heads % in.num_kv_heads != 0)
    return fail(PKD_ERR_INVALID_ARG, "num_qo_heads must be a multiple of num_kv_heads");
  if (in.head_dim < 1) return fail(PKD_ERR_INVALID_ARG, "head_dim must be >= 1");
  if (in.indptr[0] != 0) return fail(PKD_ERR_INVALID_ARG, "kv_indptr[0] must be 0");
  if (in.qo_indptr) {
    const int32_t gqa = in.num_qo_heads / in.num_kv_heads;
    if (kSharedRowsPerWorkgroup % gqa != 0)
      return fail(PKD_ERR_UNSUPPORTED, "shared-prefix plans need num_qo_heads / num_kv_heads to divide 128");
    if (in.qo_indptr[0] != 0) return fail(PKD_ERR_INVALID_ARG, "qo_indptr[0] must be 0");
    for (int32_t g = 0; g < in.batch; ++g)
      if (int64_t(in.qo_indptr[g + 1]) - in.qo_indptr[g] < 1)
        return fail(PKD_ERR_INVALID_ARG, "every group needs at least one request (qo_indptr must increase)");
  }
  for (int32_t i = 0; i < in.batch; ++i) {
    // differences in 64 bits: a malformed table may hold any int32 values
    const int64_t n = int64_t(in.indptr[i + 1]) - in.indptr[i];
    if (n < 1)
      return fail(PKD_ERR_INVALID_ARG, "every request needs at least one page (kv_indptr must increase)");
    if (in.last[i] < 1 || in.last[i] > in.page_size)
      return fail(PKD_ERR_INVALID_ARG, "kv_last_page_len must lie in [1, page_size]");
    // chunk and request lengths are 32-bit throughout (plan image, kernels)
    if (int64_t(in.page_size) * (n - 1) + in.last[i] > INT32_MAX)
      return fail(PKD_ERR_INVALID_ARG, "a request is longer than 2^31 - 1 tokens");
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

  const bool shared = in.qo_indptr != nullptr;
  const int32_t gqa = in.num_qo_heads / in.num_kv_heads;
  const int64_t tq = shared ? kSharedRowsPerWorkgroup / gqa : 1;  // requests per row block
  const int64_t heads = shared ? in.num_kv_heads : 1;  // items per chunk and block
  auto rows_of = [&](int32_t i) -> int64_t { return shared ? in.qo_indptr[i + 1] - in.qo_indptr[i] : 1; };

  // Total work: KV tokens times query tiles (row blocks), times the KV heads
  // when each head is an item of its own.
  int64_t total = 0, work = 0;
  for (int32_t i = 0; i < in.batch; ++i) {
    const int64_t l = P * (int64_t(in.indptr[i + 1] - in.indptr[i]) - 1) + in.last[i];
    total += l;
    work += ceil_div(rows_of(i), tq) * l;
  }
  work *= heads;

  int64_t cp = in.fixed_chunk_pages > 0
                   ? int64_t(in.fixed_chunk_pages)
                   : std::max<int64_t>({1, ceil_div(min_chunk, P), ceil_div(ceil_div(work, S), P)});
  if (cp > INT32_MAX) cp = INT32_MAX;

  s.items.clear();
  s.merges.clear();
  s.groups.clear();
  int64_t next_partial = 0;
  for (int32_t i = 0; i < in.batch; ++i) {
    const int64_t n = in.indptr[i + 1] - in.indptr[i];
    const int64_t k = ceil_div(n, cp);
    const int64_t rows = rows_of(i);
    const bool split = k > 1 || (in.flags & PKD_PLAN_ALL_PARTIALS);
    const int64_t base = split ? next_partial : -1;
    if (split) {
      if (next_partial + rows * k > INT32_MAX) {
        if (err) *err = "too many partial states";
        return PKD_ERR_INVALID_ARG;
      }
      const int32_t row0 = shared ? in.qo_indptr[i] : i;
      for (int64_t r = 0; r < rows; ++r)
        s.merges.push_back({int32_t(row0 + r), int32_t(next_partial + r * k), int32_t(k)});
      next_partial += rows * k;
    }
    if (shared) s.groups.push_back({in.qo_indptr[i], int32_t(rows), int32_t(k), int32_t(base)});
    const int64_t blocks = ceil_div(rows, tq);
    for (int64_t b = 0; b < blocks; ++b) {
      const int64_t lq = std::min<int64_t>(tq, rows - b * tq);
      for (int64_t j = 0; j < k; ++j) {
        PlanItem it;
        it.request = i;
        it.chunk = int32_t(j);
        it.page_begin = int32_t(in.indptr[i] + j * cp);
        it.num_pages = int32_t(std::min<int64_t>(cp, n - j * cp));
        it.last_len = j == k - 1 ? in.last[i] : int32_t(P);
        it.length = int32_t((it.num_pages - 1) * P + it.last_len);
        it.out = split ? int32_t(base + j) : -1;
        it.cost = alpha * lq + beta * it.length;
        it.block = int32_t(b);
        for (int64_t h = 0; h < heads; ++h) {
          it.head = int32_t(h);
          s.items.push_back(it);
        }
      }
    }
  }
  const int64_t I = int64_t(s.items.size());
  const int64_t n_merge = int64_t(s.merges.size());
  const int64_t n_groups = int64_t(s.groups.size());
  layout->kind = shared ? PKD_PLAN_SHARED : PKD_PLAN_DECODE;
  layout->num_requests = shared ? in.qo_indptr[in.batch] : in.batch;
  layout->num_groups = int32_t(n_groups);
  layout->rows_per_block = int32_t(tq);
  layout->off_slots = plan_off_slots();
  layout->off_first = plan_off_first(S);
  layout->off_merge = plan_off_merge(S);
  layout->off_items = plan_off_items(S, n_merge);
  layout->off_groups = layout->off_items + 8 * I;
  layout->off_indices = align_up(layout->off_groups + 4 * n_groups, 32);
  layout->nnz = in.indptr[in.batch];
  layout->total_tokens = total;
  layout->chunk_pages = int32_t(cp);
  layout->num_items = int32_t(I);
  layout->n_partials = int32_t(next_partial);
  layout->n_split = int32_t(n_merge);
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
    if (A.block != B.block) return A.block < B.block;
    if (A.chunk != B.chunk) return A.chunk < B.chunk;
    return A.head < B.head;
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
  hdr[PKD_H_BATCH] = layout->num_requests;
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
  hdr[PKD_H_KIND] = layout->kind;
  hdr[PKD_H_NUM_GROUPS] = layout->num_groups;
  hdr[PKD_H_OFF_GROUPS] = int32_t(layout->off_groups);
  hdr[PKD_H_ROWS_PER_BLOCK] = layout->rows_per_block;
  int32_t kmin = 0, kmax = 0;
  for (const PlanMerge& m : s.merges) {
    kmin = kmin == 0 ? m.k : std::min(kmin, m.k);
    kmax = std::max(kmax, m.k);
  }
  hdr[PKD_H_MIN_CHUNKS] = kmin;
  hdr[PKD_H_MAX_CHUNKS] = kmax;
  hdr[PKD_H_FLAGS] = in.flags;

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
    row[6] = it.block;
    row[7] = it.head;
  }
  int32_t* first = image + layout->off_first;
  for (int32_t q = 0; q < S; ++q)
    if (slot_indptr[q] < slot_indptr[q + 1])
      std::copy(out_items + 8 * int64_t(slot_indptr[q]), out_items + 8 * int64_t(slot_indptr[q]) + 8,
                first + 8 * int64_t(q));

  // Reduction map (request order) and, for shared-prefix plans, the group
  // table.
  int32_t* merge = image + layout->off_merge;
  for (size_t e = 0; e < s.merges.size(); ++e) {
    merge[4 * e + 0] = s.merges[e].request;
    merge[4 * e + 1] = s.merges[e].first;
    merge[4 * e + 2] = s.merges[e].k;
  }
  int32_t* groups = image + layout->off_groups;
  for (size_t g = 0; g < s.groups.size(); ++g) {
    groups[4 * g + 0] = s.groups[g].row0;
    groups[4 * g + 1] = s.groups[g].rows;
    groups[4 * g + 2] = s.groups[g].k;
    groups[4 * g + 3] = s.groups[g].base;
  }
  return PKD_OK;
}

}  // namespace pkd
