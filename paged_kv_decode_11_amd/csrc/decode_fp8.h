// Device code of the paged GQA decode kernel over an FP8 (E4M3) KV cache
// (decode_fp8_kernel in decode_fp8.hip), as a function of the slot a
// workgroup serves, so that another kernel can run it on part of its grid
// (the composable kernel in composable.hip).  Internal to the library.
//
// Same work items and outputs as the bf16 kernels (pinghaoyang FlashInfer
// page, sections "从推理形状出发" and "在线 Softmax 为什么允许任意切块"); the
// cache holds E4M3 codes and one scale per tensor, a stored K code c standing
// for e4m3(c) * k_scale (pinghaoyang page, table of customisable hooks in
// "可定制注意力模板：把变化留给 JIT": dequantisation is a key/value transform
// with a scale contract).  k_scale is folded into the logit scale and v_scale
// into the final normalisation, so the kernel works on the codes' values.
//
// Halving the bytes per token halves the time HBM allows per token, so both
// products go to the matrix cores and the vector ALUs are left with the
// conversions and the softmax.  A step covers 32 tokens of one KV head:
//
// * S^T = K Q^T: two v_mfma_f32_16x16x32_bf16 chains (tokens 0..15 and
//   16..31), K as the A operand straight from the cache (lane l holds 32
//   bytes of token l & 15's row), Q^T as the B operand (rows g..15 zero).
//   Every E4M3 value is exact in bf16 and bf16 x bf16 products are exact in
//   fp32, so the logits carry only fp32 summation error.  The contraction
//   order over head_dim is permuted the same way in both operands so that
//   each lane's K bytes are 2 x 16 contiguous bytes.
// * The result leaves lane l with row l & 15 and tokens 4 (l >> 4) + v of
//   each half: the row maximum is an in-lane max over 8 values and a swap
//   across the four 16-lane groups; the 8 probabilities of a lane, as fp16
//   pairs, are exactly the B operands of the P V products, so they never
//   leave the registers.
// * O^T += V^T P^T: sixteen v_mfma_f32_16x16x32_f16 (two per 16 head dims).
//   V rows are written to LDS in token order permuted to match P's layout
//   and read back transposed with ds_read_b64_tr_b8, 8 tokens of one head
//   dim per lane, then widened to fp16 (exact).  Each probability enters as
//   an fp16 high part plus the fp16 rounding of its remainder (two products
//   with the same V operand): their sum is p to about 2^-22 relative, where
//   fp16 alone keeps 2^-11, so the output error does not grow with the
//   magnitude of V (E4M3 values reach 448 times v_scale).  Every fp16 x fp16
//   product is exact in the fp32 accumulator.  The probabilities are scaled
//   by 2^15 before the split (folded into the exponent), which keeps the
//   high part in fp16's normal range down to 2^-29; the scale cancels in
//   o = acc / l.
//
// K and V of the next two steps stream into registers while the current one
// is computed (two steps in a ring, each refilled with the step two ahead
// once its V is in LDS and its K consumed), one wave per KV head as in the bf16
// matrix-core kernel; Q waits in LDS.  The two waves that share a SIMD keep
// pace through issue priority (see the steady-state loop).  Page sizes 16,
// 32 and 64 keep each 16-token half of a step in one page, addressed through
// a buffer descriptor over that page; smaller pages (1, 2, 4, 8 tokens) give
// each lane the address of each of its rows (two K rows and four V rows per
// step).

#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"
#include "pkd.h"
#include "plan_layout.h"

namespace pkd {
namespace fp8 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

constexpr int kStep = 32;
// probabilities enter fp16 as p * 2^kPShift
constexpr float kPShift = 15.f;

// 8 E4M3 codes to 8 fp16 (exact).
__device__ __forceinline__ uint4 fp8x8_to_f16(uint32_t w0, uint32_t w1) {
  return make_uint4(
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, true)));
}

// Two probabilities as fp16 pairs: `hi` their fp16 roundings, `lo` the
// fp16 roundings of what those leave over (a - fp16(a) is exact in fp32).
__device__ __forceinline__ void split_f16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  f16x2_t h;
  h.x = (_Float16)a;
  h.y = (_Float16)b;
  f16x2_t r;
  r.x = (_Float16)(a - (float)h.x);
  r.y = (_Float16)(b - (float)h.y);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ floatx4_t mfma_bf16(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx4_t mfma_f16(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// LDS row (slot) of step token t.  P^T's B operand gives lane group kg the
// tokens 4 kg .. 4 kg + 3 of both halves as its 8 contraction slots
// 8 kg .. 8 kg + 7; V rows are stored in that slot order.
__device__ __forceinline__ int v_slot(int t) {
  const int u = t & 15;
  return 8 * (u >> 2) + 4 * (t >> 4) + (u & 3);
}

// V rows sit 144 bytes apart in LDS: the 16 rows that two lane groups read
// at the same head dims then fall on 16 distinct 4-bank groups, and every
// lane's read and write addresses are one base plus constant offsets.
constexpr int kVRowBytes = 144;

struct FShared {
  uint4 v[kStep * kVRowBytes / 16];  // V rows of the step by slot, kVRowBytes apart
  uint4 q[4][64];                    // Q^T operand of MFMA j for lane l (see the kernel)
};

struct FStep {
  uint4 k[2][2];  // half h, load i: K[token 16 h + (l & 15)] bytes 64 i + 16 (l >> 4) .. + 16
  uint4 v[4];     // load i: V[token 8 i + (l >> 3)] bytes 16 (l & 7) .. + 16
};

// Where this lane's rows of one step are.  Pages of 16 or more tokens:
// buffers over the pages of the two halves and the byte offset of each
// half's first token row within its page.  Smaller pages: the range-checked
// page id of each of this lane's rows (K rows of both halves, V rows of the
// four V loads), the step and the item length; each address is formed at
// its load (six 64-bit addresses held across the step would spill).
template <int P, bool kWhole = (P % 16 == 0)>
struct FRef;

template <int P>
struct FRef<P, true> {
  __amdgpu_buffer_rsrc_t page[2];
  uint32_t off[2];
};

template <int P>
struct FRef<P, false> {
  int32_t k[2];
  int32_t v[4];
  int32_t step;
  int32_t len;
};

// Page ids of one step, read a step ahead of their use: one wave-uniform id
// per half for whole-half pages, else the id of each of this lane's rows.
template <int P, bool kWhole = (P % 16 == 0)>
struct FIds;

template <int P>
struct FIds<P, true> {
  int32_t id[2];
};

template <int P>
struct FIds<P, false> {
  int32_t k[2];
  int32_t v[4];
};

struct FCtx {
  const char* __restrict__ kv;
  int64_t num_pages;
  uint32_t row_bytes;   // one token's K (or V) codes of all KV heads
  uint32_t v_bytes;     // K half of a page
  uint32_t page_bytes;
  uint32_t k_lane;      // this lane's K offset in a half: (l & 15) rows + head + 16 (l >> 4)
  uint32_t v_lane;      // this lane's V offset in a load: (l >> 3) rows + head + 16 (l & 7)
  uint32_t k_col;       // this lane's K offset in a row: head + 16 (l >> 4)
  uint32_t v_col;       // this lane's V offset in a row: head + 16 (l & 7)
};

// Step tokens of this lane's rows, clamped into the item (rows past its end
// re-read its last token; their logits are masked and their V zeroed): K
// row of half h is token 16 h + (l & 15), V load i holds token 8 i + (l >> 3).
__device__ __forceinline__ int f_k_token(int s, int h, int lane, int len) {
  return min(kStep * s + 16 * h + (lane & 15), len - 1);
}
__device__ __forceinline__ int f_v_token(int s, int i, int lane, int len) {
  return min(kStep * s + 8 * i + (lane >> 3), len - 1);
}

// Page ids of step s.  Whole-half pages: the id of each half; a half past
// the item's last page (possible when P = 16) reads that last page and is
// masked.  Smaller pages: the id of each of this lane's rows.
template <int P>
__device__ __forceinline__ FIds<P> f_read_ids(const int32_t* idx, int len, int s, int lane) {
  FIds<P> ids;
  if constexpr (P % 16 == 0) {
    const int last = (len - 1) / P;
    ids.id[0] = idx[min((kStep * s) / P, last)];
    if constexpr (P == 16) {
      ids.id[1] = idx[min((kStep * s + 16) / P, last)];
    } else {
      ids.id[1] = ids.id[0];
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) ids.k[h] = idx[f_k_token(s, h, lane, len) / P];
#pragma unroll
    for (int i = 0; i < 4; ++i) ids.v[i] = idx[f_v_token(s, i, lane, len) / P];
  }
  return ids;
}

template <int P>
__device__ __forceinline__ FRef<P> f_ref(const FCtx& c, FIds<P> ids, int s, int lane, int len,
                                         int& bad) {
  FRef<P> r;
  if constexpr (P % 16 != 0) {
    // (the ids were requested a step earlier; the empty asm keeps each range
    // check here instead of next to its load)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      asm volatile("" : "+v"(ids.k[h]));
      r.k[h] = int32_t(safe_page(ids.k[h], c.num_pages, bad));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      asm volatile("" : "+v"(ids.v[i]));
      r.v[i] = int32_t(safe_page(ids.v[i], c.num_pages, bad));
    }
    r.step = s;
    r.len = len;
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // The id was requested a step earlier.  Passing it through an empty asm
      // here keeps its range check from being hoisted next to the load, where
      // it would make the step wait for the scalar load before its prefetch.
      // (wave-uniform by construction; readfirstlane keeps it in a scalar
      // register whatever the loop structure)
      int32_t id = __builtin_amdgcn_readfirstlane(ids.id[h]);
      asm volatile("" : "+s"(id));
      const int64_t pg = safe_page(id, c.num_pages, bad);
      // raw buffer over one page (32-bit data format word as raw loads need);
      // offsets past the page read zeros
      r.page[h] = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(c.kv + pg * c.page_bytes),
                                                    0, int(c.page_bytes), 0x00020000);
      r.off[h] = uint32_t((kStep * s + 16 * h) % P) * c.row_bytes;
    }
  }
  return r;
}

template <int P>
__device__ __forceinline__ void f_load_k(FStep& d, const FCtx& c, const FRef<P>& r) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (P % 16 == 0) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b128(r.page[h], c.k_lane,
                                                             r.off[h] + 64 * i, kBufferNontemporal);
        d.k[h][i] = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        const int lane = threadIdx.x & 63;
        const uint32_t slot = uint32_t(f_k_token(r.step, h, lane, r.len) % P);
        d.k[h][i] = load_stream16(c.kv + int64_t(r.k[h]) * c.page_bytes + slot * c.row_bytes +
                                  c.k_col + 64 * i);
      }
    }
}

template <int P>
__device__ __forceinline__ void f_load_v(FStep& d, const FCtx& c, const FRef<P>& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (P % 16 == 0) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b128(
          r.page[i >> 1], c.v_lane, r.off[i >> 1] + c.v_bytes + 8 * (i & 1) * c.row_bytes,
          kBufferNontemporal);
      d.v[i] = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      const int lane = threadIdx.x & 63;
      const uint32_t slot = uint32_t(f_v_token(r.step, i, lane, r.len) % P);
      d.v[i] = load_stream16(c.kv + int64_t(r.v[i]) * c.page_bytes + c.v_bytes +
                             slot * c.row_bytes + c.v_col);
    }
  }
}

template <int P>
__device__ __forceinline__ void f_load(FStep& d, const FCtx& c, const FRef<P>& r) {
  f_load_k<P>(d, c, r);
  f_load_v<P>(d, c, r);
}

template <int G>
struct FState {
  float m;          // running max (base 2) of row l & 15
  float lp;         // this lane's share of the row's sum of 2^15 p
  floatx4_t o[8];   // O^T block b: dims 16 b + 4 (l >> 4) + v of row l & 15, scaled by 2^15
};

// One 32-token step.  With kPrefetch a later step's loads are issued into
// `nxt`, its V once this step's V is in LDS and its K once this step's K has
// gone through the matrix cores, so `nxt` may be `cur` (the two-step ring);
// the last step (kLast)
// masks tokens >= valid: their logits to -inf and their V rows to zero (a
// slot past the sequence may hold any code).
template <int G, int P, bool kPrefetch, bool kLast>
__device__ __forceinline__ void f_step(FState<G>& st, const FStep& cur, FStep& nxt,
                                       const FCtx& c, const FRef<P>& next,
                                       int valid, int lane, float scale_log2, FShared& sh,
                                       uint32_t v_wr, uint32_t v_rd) {
  const int kg = lane >> 4;

  // V rows to LDS in slot order (the previous step's transposed reads come
  // first in program order, and one wave's LDS accesses complete in order).
  // Load i of lane l holds token 8 i + (l >> 3), whose slot is
  // 16 (i & 1) + 4 (i >> 1) + v_slot(l >> 3).
  {
    char* vb = reinterpret_cast<char*>(sh.v) + v_wr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 w = cur.v[i];
      if constexpr (kLast) {
        if (8 * i + (lane >> 3) >= valid) w = make_uint4(0u, 0u, 0u, 0u);
      }
      *reinterpret_cast<uint4*>(vb + (16 * (i & 1) + 4 * (i >> 1)) * kVRowBytes) = w;
    }
  }
  if constexpr (kPrefetch) {
    __builtin_amdgcn_sched_barrier(0);
    f_load_v<P>(nxt, c, next);
    __builtin_amdgcn_sched_barrier(0);
  }

  // S^T for both halves: A = K rows, B = Q^T; MFMA j takes head dims
  // 64 (j >> 1) + 16 kg + 8 (j & 1) .. + 7 at contraction slots 8 kg ..
  floatx4_t s[2] = {floatx4_t{0.f, 0.f, 0.f, 0.f}, floatx4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // Q stays in LDS so that it holds no registers across the step
    const uint4 qj = sh.q[j][lane];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 kw = cur.k[h][j >> 1];
      const uint4 ka = (j & 1) ? fp8x8_to_bf16(kw.z, kw.w) : fp8x8_to_bf16(kw.x, kw.y);
      s[h] = mfma_bf16(ka, qj, s[h]);
    }
  }
  if constexpr (kPrefetch) {
    __builtin_amdgcn_sched_barrier(0);
    f_load_k<P>(nxt, c, next);
    __builtin_amdgcn_sched_barrier(0);
  }

  // online softmax on row l & 15, tokens 16 h + 4 kg + v
  float x[2][4];
  float mx = kNegInf;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float sv = s[h][v] * scale_log2;
      if constexpr (kLast) {
        if (16 * h + 4 * kg + v >= valid) sv = kNegInf;
      }
      x[h][v] = sv;
      mx = fmaxf(mx, sv);
    }
  const float mn = fmaxf(st.m, rows_max(mx));
  const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
  const float base = mn - kPShift;
  float p[2][4];
  float psum = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[h][v] = __builtin_amdgcn_exp2f(x[h][v] - base);
      psum += p[h][v];
    }
  st.lp = fmaf(st.lp, alpha, psum);
  st.m = mn;
  uint4 pb, pr;
  split_f16x2(p[0][0], p[0][1], pb.x, pr.x);
  split_f16x2(p[0][2], p[0][3], pb.y, pr.y);
  split_f16x2(p[1][0], p[1][1], pb.z, pr.z);
  split_f16x2(p[1][2], p[1][3], pb.w, pr.w);
#pragma unroll
  for (int b = 0; b < 8; ++b) st.o[b] *= alpha;

  __builtin_amdgcn_wave_barrier();
  // O^T block b += V^T[16 b .. 16 b + 15][slots] P^T[slots][rows].  In the
  // transposed read, lane j of each 16-lane group names an 8-byte piece:
  // slot 8 kg + (j >> 1), head dims 16 b + 8 (j & 1) .. + 7 (v_rd + 16 b);
  // lane i then receives byte i & 7 of the pieces of lanes i >> 3,
  // 2 + (i >> 3), ..., that is head dim 16 b + i at slots 8 kg .. 8 kg + 7.
  char* vr = reinterpret_cast<char*>(sh.v) + v_rd;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const i32x2_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_i32x2_t*)((__attribute__((address_space(3))) char*)vr + 16 * b));
    const uint4 vt = fp8x8_to_f16(uint32_t(w[0]), uint32_t(w[1]));
    st.o[b] = mfma_f16(vt, pb, st.o[b]);
    st.o[b] = mfma_f16(vt, pr, st.o[b]);
  }
  __builtin_amdgcn_wave_barrier();
}

// One workgroup's work: the items of slot `slot` of `num_slots`, with
// `shared` its per-wave LDS areas and `progress` one counter per wave
// (steps each wave has completed; see the steady-state loop).
template <int G, int P>
__device__ __forceinline__ void decode_fp8_body(
    const uint16_t* __restrict__ q_ptr, const uint8_t* __restrict__ kv_ptr,
    uint16_t* __restrict__ o_ptr, float* __restrict__ lse_ptr, const int32_t* __restrict__ ws,
    float* __restrict__ fws, int32_t* __restrict__ err, int64_t num_pages, float scale_log2,
    float out_scale, int num_qo_heads, int num_kv_heads, int slot, int num_slots,
    FShared* shared, int* progress) {
  static_assert(G >= 1 && G <= 8, "group size");
  static_assert(P == 1 || P == 2 || P == 4 || P == 8 || P == 16 || P == 32 || P == 64,
                "page size");

  // The slot's bounds, its first item (with the ids of that item's first two
  // pages) and the header fields sit at offsets fixed by the slot count (the
  // slot count): requested together, waited for at once (the empty asm), one
  // round trip to memory before the first loads of K and V (two for pages
  // below 16 tokens, whose ids come from the page table).
  const int32_t* hdr = ws + PKD_HEADER_BASE;
  const int32_t* slot_indptr = ws + plan_off_slots();
  const int32_t* first = ws + plan_off_first(num_slots) + 8 * int64_t(slot);
  const int it_begin = slot_indptr[slot];
  const int it_end = slot_indptr[slot + 1];
  const int first_req = first[0], first_page = first[1], first_out = first[4],
            first_len = first[5], first_id0 = first[6], first_id1 = first[7];
  const int off_indices = hdr[PKD_H_OFF_INDICES];
  const int partials = hdr[PKD_H_PARTIALS];
  const int off_items = hdr[PKD_H_OFF_ITEMS];
  asm volatile("" ::"s"(it_begin), "s"(it_end), "s"(first_req), "s"(first_page), "s"(first_out),
               "s"(first_len), "s"(first_id0), "s"(first_id1), "s"(off_indices), "s"(partials),
               "s"(off_items));
  const int32_t* items = ws + off_items;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (lane == 0) progress[wave] = 0;
  __syncthreads();
  int done_steps = 0;
  const int nwaves = blockDim.x >> 6;
  // every wave runs the same number of steps when the heads divide evenly
  const bool lockstep = num_kv_heads % nwaves == 0;
  const int row16 = lane & 15;
  const int kg = lane >> 4;
  FShared& sh = shared[wave];
  // this lane's LDS write base (slot of token l >> 3, piece l & 7) and
  // transposed-read base (slot 8 kg + ((l & 15) >> 1), byte 8 (l & 1))
  const uint32_t v_wr = uint32_t(v_slot(lane >> 3)) * kVRowBytes + 16 * uint32_t(lane & 7);
  const uint32_t v_rd = uint32_t(8 * kg + (row16 >> 1)) * kVRowBytes + 8 * uint32_t(lane & 1);

  const int32_t* kv_idx = ws + off_indices;
  const int64_t n_partials = partials;
  const int Hq = num_qo_heads;
  float* o_part = fws;
  float* lse_part = fws + n_partials * Hq * kHeadDim;

  FCtx c;
  c.kv = reinterpret_cast<const char*>(kv_ptr);
  c.num_pages = num_pages;
  c.row_bytes = uint32_t(num_kv_heads) * kHeadDim;
  c.v_bytes = uint32_t(P) * c.row_bytes;
  c.page_bytes = 2 * c.v_bytes;

  for (int it = it_begin; it < it_end; ++it) {
    // an item row carries the ids of the item's first two pages
    int req = first_req, page_begin = first_page, out = first_out, len = first_len,
        id0 = first_id0, id1 = first_id1;
    if (it != it_begin) {
      const int32_t* item = items + 8 * it;
      req = item[0];
      page_begin = item[1];
      out = item[4];
      len = item[5];
      id0 = item[6];
      id1 = item[7];
    }
    const int32_t* idx = kv_idx + page_begin;
    const int nsteps = (len + kStep - 1) / kStep;

    for (int kh = wave; kh < num_kv_heads; kh += nwaves) {
      const uint32_t head = uint32_t(kh) * kHeadDim;
      c.k_lane = uint32_t(row16) * c.row_bytes + head + 16 * uint32_t(kg);
      c.v_lane = uint32_t(lane >> 3) * c.row_bytes + head + 16 * uint32_t(lane & 7);
      c.k_col = head + 16 * uint32_t(kg);
      c.v_col = head + 16 * uint32_t(lane & 7);

      // Q^T operand: lane (row l & 15, kg) holds head dims
      // 64 (j >> 1) + 16 kg + 8 (j & 1) .. + 7 for MFMA j; rows >= g are zero.
      // Loaded first, staged in LDS after the first steps' loads are issued.
      uint4 qop[4];
      {
        const uint16_t* qrow = q_ptr + (int64_t(req) * Hq + kh * G + row16) * kHeadDim + 16 * kg;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          qop[j] = row16 < G
                       ? *reinterpret_cast<const uint4*>(qrow + 64 * (j >> 1) + 8 * (j & 1))
                       : make_uint4(0u, 0u, 0u, 0u);
      }
      __builtin_amdgcn_sched_barrier(0);
      FState<G> st;
      st.m = kNegInf;
      st.lp = 0.f;
#pragma unroll
      for (int b = 0; b < 8; ++b) st.o[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};

      int bad = 0;
      FStep ta, tb;
      // both loads unconditional (a one-step item reads its step twice): with
      // the same loads in flight on every path, the wait counts stay exact
      // Step 0 lies in the item's first two pages (one, for P >= 32), whose
      // ids the item row holds; so does step 1 for P >= 32 (page 1 for
      // P = 32: the first page again when the item has one page, as then it
      // has one step).  For P = 16 step 1 needs the page table.  Smaller
      // pages read the ids of both steps from the page table, together.
      FIds<P> ids0, ids1;
      if constexpr (P % 16 == 0) {
        ids0.id[0] = id0;
        ids0.id[1] = P == 16 ? id1 : id0;
      } else {
        ids0 = f_read_ids<P>(idx, len, 0, lane);
        ids1 = f_read_ids<P>(idx, len, min(1, nsteps - 1), lane);
      }
      f_load<P>(ta, c, f_ref<P>(c, ids0, 0, lane, len, bad));
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (P == 16) {
        ids1 = f_read_ids<P>(idx, len, min(1, nsteps - 1), lane);
      } else if constexpr (P % 16 == 0) {
        ids1.id[0] = ids1.id[1] = P == 32 ? id1 : id0;
      }
      f_load<P>(tb, c, f_ref<P>(c, ids1, min(1, nsteps - 1), lane, len, bad));
      FIds<P> ids_next = f_read_ids<P>(idx, len, min(2, nsteps - 1), lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) sh.q[j][lane] = qop[j];
      __builtin_amdgcn_wave_barrier();
      const int last_valid = len - kStep * (nsteps - 1);
      const FRef<P> none = {};
      int n = 0;
      // Two steps form the ring; each is refilled with the step two ahead as
      // soon as its V is in LDS and its K consumed, so while a step is
      // computed the next two are in flight.  Two steps per straight-line
      // trip.
      auto step2 = [&](FStep& cur) -> bool {
        if (n == nsteps - 1) {
          f_step<G, P, false, true>(st, cur, cur, c, none, last_valid, lane, scale_log2, sh,
                                    v_wr, v_rd);
          return true;
        }
        if (n + 2 < nsteps) {
          const FRef<P> ref = f_ref<P>(c, ids_next, n + 2, lane, len, bad);
          ids_next = f_read_ids<P>(idx, len, min(n + 3, nsteps - 1), lane);
          f_step<G, P, true, false>(st, cur, cur, c, ref, kStep, lane, scale_log2, sh, v_wr,
                                    v_rd);
        } else {
          f_step<G, P, false, false>(st, cur, cur, c, none, kStep, lane, scale_log2, sh, v_wr,
                                     v_rd);
        }
        ++n;
        return false;
      };
      while (n + 3 < nsteps) {
        // keep the waves of the workgroup together, once per trip (left alone,
        // waves 4-7 finished their heads at ~1.75x the time of waves 0-3)
        keep_pace<kMaxWavesPerBlock>(progress, wave, nwaves, lockstep, done_steps + n);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          FStep& cur = k == 0 ? ta : tb;
          const FRef<P> ref = f_ref<P>(c, ids_next, n + 2, lane, len, bad);
          ids_next = f_read_ids<P>(idx, len, min(n + 3, nsteps - 1), lane);
          f_step<G, P, true, false>(st, cur, cur, c, ref, kStep, lane, scale_log2, sh, v_wr,
                                    v_rd);
          ++n;
        }
      }
      for (;;) {
        if (step2(ta)) break;
        if (step2(tb)) break;
      }
      report_bad_pages(bad, lane, err, PKD_DEVERR_PAGE_ID);
      __builtin_amdgcn_s_setprio(0);
      done_steps += nsteps;

      // lane (row l & 15, kg) holds head dims 16 b + 4 kg + v of its row
      const float l_row = rows_sum(st.lp);
      if (row16 < G) {
        const float inv = out_scale / l_row;
        const float lse_nat = (st.m + __log2f(l_row) - kPShift) * kLn2;
        const int64_t qh = int64_t(kh) * G + row16;
        if (out < 0) {
          uint16_t* orow = o_ptr + (int64_t(req) * Hq + qh) * kHeadDim + 4 * kg;
#pragma unroll
          for (int b = 0; b < 8; ++b)
            *reinterpret_cast<uint2*>(orow + 16 * b) =
                make_uint2(pack_bf16x2(st.o[b][0] * inv, st.o[b][1] * inv),
                           pack_bf16x2(st.o[b][2] * inv, st.o[b][3] * inv));
          if (lse_ptr && kg == 0) lse_ptr[int64_t(req) * Hq + qh] = lse_nat;
        } else {
          float* orow = o_part + (int64_t(out) * Hq + qh) * kHeadDim + 4 * kg;
#pragma unroll
          for (int b = 0; b < 8; ++b)
            *reinterpret_cast<float4*>(orow + 16 * b) =
                make_float4(st.o[b][0] * inv, st.o[b][1] * inv, st.o[b][2] * inv,
                            st.o[b][3] * inv);
          if (kg == 0) lse_part[int64_t(out) * Hq + qh] = lse_nat;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

}  // namespace
}  // namespace fp8
}  // namespace pkd
