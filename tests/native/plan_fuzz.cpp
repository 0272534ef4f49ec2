// Randomised check of the host scheduler (plan.cpp) for a sanitizer build.
//
//   plan_fuzz <seed> <cases>
//
// Builds random page tables -- valid ones and ones broken in the ways a
// caller gets them wrong (kv_indptr not starting at 0 or not increasing,
// last-page lengths outside [1, P], extreme values, bad head counts) -- with
// random slot counts, forced chunk sizes, cost weights, and shared-prefix
// group tables, and plans each into an image buffer of exactly the
// requested capacity (so an out-of-bounds write is a heap overflow the
// address sanitizer reports).  For every plan it checks the status code it
// should get and, on success, the invariants of the plan image:
//   * slot_indptr runs from 0 to I without decreasing; the first-item table
//     repeats each slot's first item;
//   * every item lies within its row's pages, and the chunks of each row (per
//     row block and KV head in shared-prefix plans) cover its pages exactly
//     once, in order, with the last page's length only on the last chunk;
//   * unsplit rows write their output directly (out = -1), unless the plan
//     asks for all partials; the chunks of a split row, in page order, write
//     consecutive partial ids, and the merge list names each request of a
//     split row once, in ascending order, with its ids;
//   * with derived chunks, I <= S + 2 B (decode plans);
//   * the longest-first bound: the largest slot load is at most the mean load
//     plus the largest item cost.
// Prints "ok <cases> ..." and exits 0 when every case passes; prints the
// first failure and exits 1 otherwise.

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <random>
#include <string>
#include <vector>

#include "pkd.h"
#include "plan.h"
#include "plan_layout.h"

namespace {

struct Failure {
  std::string what;
};

#define EXPECT(cond, ...)                                                   \
  do {                                                                      \
    if (!(cond)) {                                                          \
      char buf_[512];                                                       \
      std::snprintf(buf_, sizeof(buf_), __VA_ARGS__);                       \
      throw Failure{std::string(#cond) + ": " + buf_};                      \
    }                                                                       \
  } while (0)

struct Case {
  std::vector<int32_t> indptr, last, qo_indptr;
  int32_t batch = 0, Hq = 32, Hkv = 8, D = 128, P = 16, S = 8;
  int32_t fixed = 0, min_tokens = 0, alpha = -1, beta = 0, flags = 0;
  bool shared = false;
  int expect = PKD_OK;  // status the plan must return (OK unless the case is broken)
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

Case make_case(std::mt19937_64& rng, int n) {
  auto uni = [&](int64_t lo, int64_t hi) {
    return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
  };
  Case c;
  static const int32_t page_sizes[] = {1, 2, 4, 8, 16, 32, 64};
  static const int32_t groups[] = {1, 2, 4, 8};
  c.P = page_sizes[uni(0, 6)];
  c.Hkv = int32_t(uni(1, 12));
  c.Hq = c.Hkv * groups[uni(0, 3)];
  c.S = int32_t(uni(1, n % 5 == 0 ? 600 : 40));
  c.batch = int32_t(uni(1, n % 7 == 0 ? 300 : 12));
  c.shared = uni(0, 3) == 0;
  const int64_t kind = uni(0, 9);
  if (kind < 4) c.fixed = int32_t(uni(1, 6));
  if (kind == 4) c.fixed = int32_t(uni(1000, std::numeric_limits<int32_t>::max()));
  if (uni(0, 2) == 0) c.min_tokens = int32_t(uni(-5, 3000));
  if (uni(0, 2) == 0) c.alpha = int32_t(uni(-3, 100));
  if (uni(0, 2) == 0) c.beta = int32_t(uni(-3, 100));
  if (uni(0, 30) == 0) c.alpha = c.beta = std::numeric_limits<int32_t>::max();
  if (uni(0, 3) == 0) c.flags = PKD_PLAN_ALL_PARTIALS;
  c.indptr.assign(c.batch + 1, 0);
  c.last.assign(c.batch, 1);
  const int64_t max_pages = n % 11 == 0 ? 3000 : 40;
  for (int32_t i = 0; i < c.batch; ++i) {
    c.indptr[i + 1] = c.indptr[i] + int32_t(uni(1, max_pages));
    c.last[i] = int32_t(uni(1, c.P));
  }
  if (c.shared) {
    c.qo_indptr.assign(c.batch + 1, 0);
    for (int32_t g = 0; g < c.batch; ++g) c.qo_indptr[g + 1] = c.qo_indptr[g] + int32_t(uni(1, 70));
  }
  // break one thing in about a third of the cases
  switch (uni(0, 29)) {
    case 0: c.indptr[0] = int32_t(uni(1, 5)); c.expect = PKD_ERR_INVALID_ARG; break;
    case 1: {
      const int32_t i = int32_t(uni(0, c.batch - 1));
      c.indptr[i + 1] = c.indptr[i] - int32_t(uni(0, 3));  // a request with no page (or fewer)
      c.expect = PKD_ERR_INVALID_ARG;
      break;
    }
    case 2: c.last[uni(0, c.batch - 1)] = 0; c.expect = PKD_ERR_INVALID_ARG; break;
    case 3: c.last[uni(0, c.batch - 1)] = c.P + int32_t(uni(1, 9)); c.expect = PKD_ERR_INVALID_ARG; break;
    case 4: c.last[uni(0, c.batch - 1)] = std::numeric_limits<int32_t>::min(); c.expect = PKD_ERR_INVALID_ARG; break;
    case 5: {
      // extreme entries: differences that overflow 32 bits
      const int32_t i = int32_t(uni(0, c.batch - 1));
      c.indptr[i + 1] = std::numeric_limits<int32_t>::min();
      c.expect = PKD_ERR_INVALID_ARG;
      break;
    }
    case 6:
      if (c.Hkv == 1) c.Hkv = 2;
      c.Hq = c.Hkv * 3 + 1;  // not a multiple of Hkv
      c.expect = PKD_ERR_INVALID_ARG;
      break;
    case 7: c.S = 0; c.expect = PKD_ERR_INVALID_ARG; break;
    case 8:
      if (c.shared) {
        const int32_t g = int32_t(uni(0, c.batch - 1));
        c.qo_indptr[g + 1] = c.qo_indptr[g];  // a group with no request
        c.expect = PKD_ERR_INVALID_ARG;
      }
      break;
    case 9: {
      // one request longer than 2^31 tokens
      c.P = 64;
      c.last.assign(c.batch, 1);
      c.indptr[c.batch] = c.indptr[c.batch - 1] + (1 << 26) + 5;
      c.expect = PKD_ERR_INVALID_ARG;
      break;
    }
    default: break;
  }
  if (c.expect == PKD_OK && c.shared) {
    if (128 % (c.Hq / c.Hkv) != 0) c.expect = PKD_ERR_UNSUPPORTED;
  }
  return c;
}

pkd::PlanInput input_of(const Case& c) {
  pkd::PlanInput in;
  in.indptr = c.indptr.data();
  in.last = c.last.data();
  in.qo_indptr = c.shared ? c.qo_indptr.data() : nullptr;
  in.batch = c.batch;
  in.num_qo_heads = c.Hq;
  in.num_kv_heads = c.Hkv;
  in.head_dim = c.D;
  in.page_size = c.P;
  in.num_slots = c.S;
  in.fixed_chunk_pages = c.fixed;
  in.min_chunk_tokens = c.min_tokens;
  in.alpha = c.alpha;
  in.beta = c.beta;
  in.flags = c.flags;
  in.plan_id = 7;
  return in;
}

void check_image(const Case& c, const pkd::PlanLayout& L, const int32_t* img) {
  const int32_t* h = img + PKD_HEADER_BASE;
  const int32_t S = c.S, I = L.num_items, P = c.P;
  EXPECT(h[PKD_H_MAGIC] == PKD_PLAN_MAGIC, "magic %x", h[PKD_H_MAGIC]);
  EXPECT(h[PKD_H_SLOTS] == S && h[PKD_H_ITEMS] == I, "header counts");
  EXPECT(h[PKD_H_KIND] == (c.shared ? PKD_PLAN_SHARED : PKD_PLAN_DECODE), "kind");
  EXPECT(h[PKD_H_FLAGS] == c.flags, "flags %d", h[PKD_H_FLAGS]);
  const bool all_partials = (c.flags & PKD_PLAN_ALL_PARTIALS) != 0;
  for (int w = 0; w < PKD_HEADER_BASE; ++w) EXPECT(img[w] == 0, "device word %d not zero", w);
  const int32_t* slots = img + pkd::plan_off_slots();
  EXPECT(slots[0] == 0 && slots[S] == I, "slot_indptr ends %d %d (I=%d)", slots[0], slots[S], I);
  for (int32_t s = 0; s < S; ++s) EXPECT(slots[s] <= slots[s + 1], "slot_indptr decreases at %d", s);
  EXPECT(h[PKD_H_OFF_MERGE] == pkd::plan_off_merge(S), "merge list offset %d", h[PKD_H_OFF_MERGE]);
  EXPECT(h[PKD_H_OFF_ITEMS] == pkd::plan_off_items(S, h[PKD_H_SPLIT]), "items offset %d",
         h[PKD_H_OFF_ITEMS]);
  const int32_t* items = img + h[PKD_H_OFF_ITEMS];
  const int32_t* first = img + pkd::plan_off_first(S);
  for (int32_t s = 0; s < S; ++s)
    for (int f = 0; f < 8; ++f)
      EXPECT(first[8 * s + f] == (slots[s] < slots[s + 1] ? items[8 * slots[s] + f] : 0),
             "first-item table, slot %d field %d", s, f);

  const int32_t rows_total = c.shared ? c.qo_indptr[c.batch] : c.batch;
  const int32_t tq = c.shared ? 128 / (c.Hq / c.Hkv) : 1;
  const int32_t heads = c.shared ? c.Hkv : 1;
  const int64_t alpha = c.alpha < 0 ? 1 : c.alpha, beta = c.beta <= 0 ? 1 : c.beta;
  // Items of each (row, row block, KV head) unit, in page order: they must
  // cover the row's pages exactly once.  Chunk j of a split row writes
  // partial id base_r + j (base_r counting the partial states of the split
  // rows before it: k per request of the row); an unsplit row writes -1.
  struct Rec {
    int64_t unit;
    int32_t r, pb, np, ll, len, out;
  };
  std::vector<Rec> recs;
  std::vector<int64_t> unit0(c.batch, 0), blocks_of(c.batch, 0);
  int64_t units = 0;
  for (int32_t r = 0; r < c.batch; ++r) {
    const int64_t rows = c.shared ? c.qo_indptr[r + 1] - c.qo_indptr[r] : 1;
    unit0[r] = units;
    blocks_of[r] = ceil_div(rows, tq);
    units += blocks_of[r] * heads;
  }
  std::vector<int64_t> slot_load(S, 0);
  int64_t max_cost = 0, sum_cost = 0;
  for (int32_t s = 0; s < S; ++s) {
    for (int32_t x = slots[s]; x < slots[s + 1]; ++x) {
      const int32_t* it = items + 8 * int64_t(x);
      const int32_t r = it[0];
      EXPECT(r >= 0 && r < c.batch, "item %d row %d", x, r);
      const int32_t b = c.shared ? it[6] : 0, hd = c.shared ? it[7] : 0;
      EXPECT(b >= 0 && b < blocks_of[r] && hd >= 0 && hd < heads, "item %d block/head", x);
      recs.push_back({unit0[r] + int64_t(b) * heads + hd, r, it[1], it[2], it[3], it[5], it[4]});
      const int64_t rows = c.shared ? c.qo_indptr[r + 1] - c.qo_indptr[r] : 1;
      const int64_t lq = std::min<int64_t>(tq, rows - int64_t(b) * tq);
      const int64_t cost = alpha * lq + beta * it[5];
      slot_load[s] = slot_load[s] > INT64_MAX - cost ? INT64_MAX : slot_load[s] + cost;
      sum_cost = sum_cost > INT64_MAX - cost ? INT64_MAX : sum_cost + cost;
      max_cost = std::max(max_cost, cost);
    }
  }
  std::sort(recs.begin(), recs.end(), [](const Rec& a, const Rec& b) {
    return a.unit != b.unit ? a.unit < b.unit : a.pb < b.pb;
  });
  std::vector<int32_t> chunks_of(c.batch, 0);
  for (const Rec& e : recs)
    if (e.unit == unit0[e.r]) ++chunks_of[e.r];
  std::vector<int64_t> base_of(c.batch, -1);
  int64_t next_id = 0;
  for (int32_t r = 0; r < c.batch; ++r) {
    if (chunks_of[r] > 1 || all_partials) {
      base_of[r] = next_id;
      next_id += (c.shared ? c.qo_indptr[r + 1] - c.qo_indptr[r] : 1) * int64_t(chunks_of[r]);
    }
  }
  EXPECT(next_id == L.n_partials, "partial states %lld, plan says %d", (long long)next_id,
         L.n_partials);
  size_t e = 0;
  for (int32_t r = 0; r < c.batch; ++r) {
    for (int64_t u = unit0[r]; u < unit0[r] + blocks_of[r] * heads; ++u) {
      int64_t next = c.indptr[r];
      int32_t j = 0;
      for (; e < recs.size() && recs[e].unit == u; ++e, ++j) {
        const Rec& q = recs[e];
        EXPECT(q.np >= 1 && q.pb == next, "row %d chunk %d begins at page %d, expected %lld", r,
               j, q.pb, (long long)next);
        next += q.np;
        EXPECT(next <= c.indptr[r + 1], "row %d chunk %d runs past its pages", r, j);
        const bool last_chunk = next == c.indptr[r + 1];
        EXPECT(q.ll == (last_chunk ? c.last[r] : P), "row %d chunk %d last_len %d", r, j, q.ll);
        EXPECT(q.len == int64_t(q.np - 1) * P + q.ll, "row %d chunk %d length", r, j);
        if (c.fixed > 0) EXPECT(q.np <= c.fixed, "row %d chunk %d above the forced size", r, j);
        EXPECT(q.out == (base_of[r] >= 0 ? base_of[r] + j : -1), "row %d chunk %d out %d", r, j,
               q.out);
      }
      EXPECT(next == c.indptr[r + 1], "row %d unit %lld covers pages up to %lld of %d", r,
             (long long)(u - unit0[r]), (long long)next, c.indptr[r + 1]);
      EXPECT(j == chunks_of[r], "row %d: a unit has %d chunks, the first %d", r, j, chunks_of[r]);
    }
  }
  EXPECT(e == recs.size(), "items left over");
  // merge list: each request of a split row once, ascending, with its ids
  const int32_t* merge = img + L.off_merge;
  int32_t prev = -1, split = 0;
  for (int32_t r = 0; r < c.batch; ++r) {
    if (base_of[r] >= 0) {
      const int32_t rows = c.shared ? c.qo_indptr[r + 1] - c.qo_indptr[r] : 1;
      const int32_t row0 = c.shared ? c.qo_indptr[r] : r;
      for (int32_t q = 0; q < rows; ++q, ++split) {
        EXPECT(split < L.n_split, "merge list too short");
        const int32_t* m = merge + 4 * split;
        EXPECT(m[0] == row0 + q && m[0] > prev, "merge entry %d request %d", split, m[0]);
        EXPECT(m[1] == base_of[r] + int64_t(q) * chunks_of[r] && m[2] == chunks_of[r],
               "merge entry %d ids %d k %d", split, m[1], m[2]);
        prev = m[0];
      }
    }
  }
  EXPECT(split == L.n_split, "merge list %d of %d", split, L.n_split);
  EXPECT(L.off_indices <= int64_t(1) << 40 && rows_total >= c.batch, "layout");
  if (!c.shared && c.fixed == 0)
    EXPECT(I <= int64_t(S) + 2 * c.batch, "I = %d above S + 2B = %d", I, S + 2 * c.batch);
  int64_t max_load = 0;
  for (int64_t v : slot_load) max_load = std::max(max_load, v);
  EXPECT(max_load * S <= sum_cost + max_cost * S, "LPT bound: max load %lld, mean %lld, max cost %lld",
         (long long)max_load, (long long)(sum_cost / S), (long long)max_cost);
}

void run_case(const Case& c, std::mt19937_64& rng) {
  pkd::PlanInput in = input_of(c);
  pkd::PlanScratch scratch;
  pkd::PlanLayout layout;
  std::string err;
  int rc = pkd::plan_measure(in, scratch, &layout, &err);
  if (c.expect != PKD_OK) {
    EXPECT(rc == c.expect, "plan_measure returned %d for a case that must give %d (%s)", rc,
           c.expect, err.c_str());
    std::vector<int32_t> img(64);
    rc = pkd::plan_build(in, scratch, img.data(), int64_t(img.size()), &layout, &err);
    EXPECT(rc == c.expect, "plan_build returned %d, expected %d", rc, c.expect);
    return;
  }
  if (rc == PKD_ERR_INVALID_ARG && err == "too many partial states") return;
  EXPECT(rc == PKD_OK, "plan_measure failed on a valid case: %d %s", rc, err.c_str());
  const int64_t need = layout.off_indices;
  // too small by a random margin: refused, nothing written past the buffer
  {
    const int64_t cap = std::uniform_int_distribution<int64_t>(0, need - 1)(rng);
    std::vector<int32_t> small(cap);
    pkd::PlanLayout l2;
    rc = pkd::plan_build(in, scratch, small.empty() ? nullptr : small.data(), cap, &l2, &err);
    EXPECT(rc == PKD_ERR_WORKSPACE_TOO_SMALL, "capacity %lld of %lld gave %d", (long long)cap,
           (long long)need, rc);
  }
  std::vector<int32_t> img(need);
  rc = pkd::plan_build(in, scratch, img.data(), need, &layout, &err);
  EXPECT(rc == PKD_OK, "plan_build failed: %d %s", rc, err.c_str());
  check_image(c, layout, img.data());
  // the workspace-size bound holds for derived chunks
  if (c.fixed == 0 && !c.shared) {
    EXPECT(layout.num_items <= pkd::max_items(c.batch, c.S), "max_items");
    EXPECT(need <= pkd::plan_image_ints(c.S, pkd::max_items(c.batch, c.S), c.batch),
           "plan_image_ints bound");
  }
  if (c.fixed == 0 && c.shared) {
    const int64_t Imax = pkd::max_items_shared(c.batch, c.qo_indptr[c.batch], c.S, c.Hq, c.Hkv);
    EXPECT(layout.num_items <= Imax, "max_items_shared %d > %lld", layout.num_items,
           (long long)Imax);
    EXPECT(layout.n_partials <= pkd::max_partials_shared(c.qo_indptr[c.batch], c.S, c.Hkv),
           "max_partials_shared");
  }
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const int cases = argc > 2 ? std::atoi(argv[2]) : 2000;
  std::mt19937_64 rng(seed);
  int valid = 0, refused = 0;
  for (int n = 0; n < cases; ++n) {
    const Case c = make_case(rng, n);
    try {
      run_case(c, rng);
    } catch (const Failure& f) {
      std::printf("FAIL case %d (seed %llu, batch %d, P %d, S %d, Hq %d, Hkv %d, fixed %d, "
                  "shared %d): %s\n",
                  n, (unsigned long long)seed, c.batch, c.P, c.S, c.Hq, c.Hkv, c.fixed,
                  int(c.shared), f.what.c_str());
      return 1;
    }
    (c.expect == PKD_OK ? valid : refused) += 1;
  }
  std::printf("ok %d cases (%d planned, %d refused)\n", cases, valid, refused);
  return 0;
}
