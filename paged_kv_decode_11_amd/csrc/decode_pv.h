// Device code of the paged GQA decode kernel with both products on the
// matrix cores (decode_pv_kernel in decode_pv.hip), as a function of the
// slot a workgroup serves, so that another kernel can run it on part of its
// grid (the composable kernel in composable.hip).  Internal to the library.
//
// Same work items and outputs as the other decode kernels (pinghaoyang
// FlashInfer page, sections "从推理形状出发" and "在线 Softmax 为什么允许任意切块").
// In decode_mfma.hip P V runs on the vector ALUs, at a cost proportional to
// the GQA group size g; here it runs on the matrix cores, so the work per
// tile is the same for g = 1 .. 8.  Per 16-token tile of one KV head:
//
// * K and V rows are loaded row-major (16 lanes per 256-byte head row, four
//   rows per instruction) and staged in per-wave LDS tiles whose 16-byte
//   pieces of row r are rotated by XOR r.
// * S^T = K Q^T: four v_mfma_f32_16x16x32_bf16, K as the A operand from LDS,
//   Q^T as the B operand (the g query rows of the group, rows g..15 zero).
//   The result leaves lane l with query row l & 15 and tokens 4 (l >> 4) + v.
// * Online softmax on those registers: the row maximum is an in-lane max over
//   4 values and a swap across the four 16-lane groups.  The 4 probabilities
//   of a lane are, in bf16, exactly the B operand of a 16x16x16 product; p is
//   split into a bf16 high part and a bf16 remainder, so the product keeps
//   about 16 bits of each probability (the vector-ALU kernel keeps fp32).
// * O^T += V^T P^T: for each block of 16 head dims, one transposing LDS read
//   (ds_read_b64_tr_b16) gives each lane 4 tokens of its head dim as the A
//   operand, and two v_mfma_f32_16x16x16_bf16 (high and low part of P)
//   accumulate.  Lane l ends with query row l & 15, so rescale factors and
//   the final max and sum never cross lanes.
//
// Streaming: two tiles in a register ring, each refilled with the tile two
// ahead as soon as it has been staged in LDS, so while one tile is computed
// the next two are in flight; a straight-line steady state of two tiles per
// trip, and a workgroup barrier plus issue priority per trip keeping the two
// waves of each SIMD together.  Page sizes that are multiples of 16 keep each tile
// in one page, addressed through a buffer descriptor over the page; smaller
// pages (1, 2, 4, 8 tokens) give each lane the address of each of its rows.

#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"
#include "pkd.h"
#include "plan_layout.h"

namespace pkd {
namespace pv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4_t mfma32(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx4_t mfma16(uint2 a, uint2 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a),
                                                   __builtin_bit_cast(short4_t, b), c, 0, 0, 0);
}

// Transposing LDS read: for the 16 lanes of a row group, lane i receives
// element i % 4 of the 8-byte piece addressed by lane 4 r + i / 4 of its
// group, for r = 0..3.
__device__ __forceinline__ uint2 lds_read_tr(const void* p) {
  typedef __attribute__((address_space(3))) short4_t lds_short4;
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p));
  return __builtin_bit_cast(uint2, v);
}

struct VShared {
  uint4 kt[16][16];  // K tile, row r's 16-byte piece c at [r][c ^ r]
  uint4 vt[16][16];  // V tile, same layout
  uint4 qa[4][64];   // B operand (Q^T) of MFMA j for lane l
};

struct VTile {
  uint4 k[4];  // load j: K row 4 j + (l >> 4), 16-byte piece l & 15
  uint4 v[4];  // load j: V row 4 j + (l >> 4), 16-byte piece l & 15
};

// Where this lane's rows of one tile are.  Page sizes that are multiples of
// 16 keep a tile in one page: a buffer over that page and the tile's offset
// in it.  Smaller pages spread a tile over 16 / P pages: the lane carries the
// address of each of its 4 K rows (V rows sit v_bytes further).
template <int P, bool kWhole = (P % 16 == 0)>
struct VRef;

template <int P>
struct VRef<P, true> {
  __amdgpu_buffer_rsrc_t page;  // buffer over the tile's page
  uint32_t tile_off;            // byte offset of the tile's first K row in the page
};

template <int P>
struct VRef<P, false> {
  const char* row[4];  // K row 4 j + (l >> 4) of the tile, this lane's 16-byte piece
};

// Page ids of one tile, read a tile ahead of their use: one wave-uniform id
// for whole-tile pages, else the id of each of this lane's 4 rows.
template <int P, bool kWhole = (P % 16 == 0)>
struct VIds;

template <int P>
struct VIds<P, true> {
  int32_t id;
};

template <int P>
struct VIds<P, false> {
  int32_t id[4];
};

struct VCtx {
  const char* __restrict__ kv;
  int64_t num_pages;
  uint32_t row_bytes;  // one token's K (or V) rows of all KV heads
  uint32_t v_bytes;    // K half of a page
  uint32_t page_bytes;
  uint32_t lane_off;   // (l >> 4) rows + this wave's head + 16 (l & 15)
  uint32_t col_off;    // this wave's head + 16 (l & 15)
};

// Row 4 j + kg of tile t, clamped into the chunk: rows past its end re-read
// its last token (their logits are masked and their V zeroed), so no slot
// past last_page_len and no page past the chunk's is touched.
__device__ __forceinline__ int v_row(int j, int kg, int len, int t) {
  return 16 * t + min(4 * j + kg, len - 16 * t - 1);
}

template <int P>
__device__ __forceinline__ VIds<P> v_read_ids(const int32_t* idx, int len, int t, int kg) {
  VIds<P> ids;
  if constexpr (P % 16 == 0) {
    ids.id = idx[(16 * t) / P];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) ids.id[j] = idx[v_row(j, kg, len, t) / P];
  }
  return ids;
}

template <int P>
__device__ __forceinline__ VRef<P> v_ref(const VCtx& c, VIds<P> ids, int len, int t, int kg,
                                         int& bad) {
  VRef<P> r;
  if constexpr (P % 16 == 0) {
    // The id was requested a tile earlier; the empty asm keeps its range
    // check here instead of next to the load.
    asm volatile("" : "+s"(ids.id));
    const int64_t pg = safe_page(ids.id, c.num_pages, bad);
    // raw buffer over one page (32-bit data format word as raw loads need)
    r.page = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(c.kv + pg * c.page_bytes), 0,
                                               int(c.page_bytes), 0x00020000);
    r.tile_off = uint32_t((16 * t) % P) * c.row_bytes;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      asm volatile("" : "+v"(ids.id[j]));
      const int64_t pg = safe_page(ids.id[j], c.num_pages, bad);
      const uint32_t slot = uint32_t(v_row(j, kg, len, t) % P);
      r.row[j] = c.kv + pg * c.page_bytes + slot * c.row_bytes + c.col_off;
    }
  }
  return r;
}

template <int P>
__device__ __forceinline__ void v_load(VTile& d, const VCtx& c, const VRef<P>& r) {
  if constexpr (P % 16 == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b128(
          r.page, c.lane_off, r.tile_off + uint32_t(4 * j) * c.row_bytes, kBufferNontemporal);
      d.k[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b128(
          r.page, c.lane_off, r.tile_off + c.v_bytes + uint32_t(4 * j) * c.row_bytes,
          kBufferNontemporal);
      d.v[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) d.k[j] = load_stream16(r.row[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) d.v[j] = load_stream16(r.row[j] + c.v_bytes);
  }
}

struct VState {
  float m;           // running max (base 2) of row l & 15
  float lp;          // this lane's share of the row's sum of p
  floatx4_t o[8];    // O^T block b: head dims 16 b + 4 (l >> 4) + v of row l & 15
};

// One tile.  With kPrefetch a later tile's loads are issued first; the last
// tile (kLast) masks tokens >= valid: logits to -inf, V rows to zero (a slot
// past the sequence may hold any value).
// With kPrefetch the later tile is requested into `nxt` once this tile has
// been staged in LDS, so `nxt` may be `cur` (the two-tile ring).
template <bool kPrefetch, bool kLast, int P>
__device__ __forceinline__ void v_step(VState& st, const VTile& cur, VTile& nxt, const VCtx& c,
                                       const VRef<P>& next, int valid, int lane, float scale_log2,
                                       VShared& sh) {
  const int row16 = lane & 15;
  const int kg = lane >> 4;
  // stage the tile (the previous tile's reads come first in program order,
  // and one wave's LDS accesses complete in order)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * j + kg;
    sh.kt[r][row16 ^ r] = cur.k[j];
    uint4 w = cur.v[j];
    if constexpr (kLast) {
      if (r >= valid) w = make_uint4(0u, 0u, 0u, 0u);
    }
    sh.vt[r][row16 ^ r] = w;
  }
  if constexpr (kPrefetch) {
    __builtin_amdgcn_sched_barrier(0);
    v_load(nxt, c, next);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_wave_barrier();

  // S^T = K Q^T: A = K row l & 15, head dims 32 j + 8 kg .. + 7
  floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) s = mfma32(sh.kt[row16][(4 * j + kg) ^ row16], sh.qa[j][lane], s);

  // online softmax on query row l & 15, tokens 4 kg + v
  float x[4];
  float mx = kNegInf;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float sv = s[v] * scale_log2;
    if constexpr (kLast) {
      if (4 * kg + v >= valid) sv = kNegInf;
    }
    x[v] = sv;
    mx = fmaxf(mx, sv);
  }
  const float mn = fmaxf(st.m, rows_max(mx));
  const float alpha = __builtin_amdgcn_exp2f(st.m - mn);  // 0 while m = -inf
  float p[4];
  float psum = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    p[v] = __builtin_amdgcn_exp2f(x[v] - mn);
    psum += p[v];
  }
  st.lp = fmaf(st.lp, alpha, psum);
  st.m = mn;
  // P^T as the B operand, high and low bf16 parts
  const uint2 ph = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
  const uint2 pl = make_uint2(pack_bf16x2(p[0] - bf16_lo(ph.x), p[1] - bf16_hi(ph.x)),
                              pack_bf16x2(p[2] - bf16_lo(ph.y), p[3] - bf16_hi(ph.y)));
#pragma unroll
  for (int b = 0; b < 8; ++b) st.o[b] *= alpha;

  // V^T as the A operand of head-dim block b: lane j of each 16-lane group
  // points the transposing read at row 4 kg + (j >> 2), head dims
  // 16 b + 4 (j & 3) .. + 3; lane i then receives head dim 16 b + i of
  // tokens 4 kg .. 4 kg + 3
  const int tr_row = 4 * kg + (row16 >> 2);
  const int tr_q = row16 & 3;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const char* a = reinterpret_cast<const char*>(&sh.vt[tr_row][(2 * b + (tr_q >> 1)) ^ tr_row]) +
                    8 * (tr_q & 1);
    const uint2 va = lds_read_tr(a);
    st.o[b] = mfma16(va, ph, st.o[b]);
    st.o[b] = mfma16(va, pl, st.o[b]);
  }
  __builtin_amdgcn_wave_barrier();
}

// One workgroup's work: the items of slot `slot` of `num_slots`.  `shared`
// holds kMaxWavesPerBlock per-wave areas and `progress` as many ints (tiles
// each wave has completed; see the steady-state loop), both in LDS.
template <int G, int P>
__device__ __forceinline__ void decode_pv_body(
    const uint16_t* __restrict__ q_ptr, const uint16_t* __restrict__ kv_ptr,
    uint16_t* __restrict__ o_ptr, float* __restrict__ lse_ptr, const int32_t* __restrict__ ws,
    float* __restrict__ fws, int32_t* __restrict__ err, int64_t num_pages, float scale_log2,
    int num_qo_heads, int num_kv_heads, int slot, int num_slots, VShared* shared,
    int* progress) {
  static_assert(G >= 1 && G <= 8, "group size");

  // The slot's bounds, its first item (with the ids of that item's first two
  // pages) and the header fields sit at offsets fixed by the slot count (the
  // slot count): requested together, waited for at once (the empty asm), one
  // round trip to memory before the first K and V loads.
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
  const int nwaves = blockDim.x >> 6;
  // every wave walks the same tiles when the heads divide evenly
  const bool lockstep = num_kv_heads % nwaves == 0;
  if (lane == 0) progress[wave] = 0;
  __syncthreads();
  int done_tiles = 0;
  const int row16 = lane & 15;
  const int kg = lane >> 4;
  VShared& sh = shared[wave];

  const int32_t* kv_idx = ws + off_indices;
  const int64_t n_partials = partials;
  const int Hq = num_qo_heads;
  float* o_part = fws;
  float* lse_part = fws + n_partials * Hq * kHeadDim;

  VCtx c;
  c.kv = reinterpret_cast<const char*>(kv_ptr);
  c.num_pages = num_pages;
  c.row_bytes = uint32_t(num_kv_heads) * kHeadDim * 2;
  c.v_bytes = uint32_t(P) * c.row_bytes;
  c.page_bytes = 2 * c.v_bytes;

  for (int it = it_begin; it < it_end; ++it) {
    // an item row carries the ids of the item's first two pages, which hold
    // its first two tiles
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
    const int ntiles = (len + 15) >> 4;

    for (int kh = wave; kh < num_kv_heads; kh += nwaves) {
      const uint32_t head_bytes = uint32_t(kh) * kHeadDim * 2;
      c.col_off = head_bytes + 16 * uint32_t(row16);
      c.lane_off = uint32_t(kg) * c.row_bytes + c.col_off;
      // Q^T operand: lane (row l & 15, kg) holds head dims 32 j + 8 kg .. + 7
      // for MFMA j; rows >= g are zero.  Loaded first, staged in LDS after
      // the first tiles' loads are issued.
      uint4 qv[4];
      {
        const uint16_t* qrow = q_ptr + (int64_t(req) * Hq + kh * G + row16) * kHeadDim + kg * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          qv[j] = row16 < G ? *reinterpret_cast<const uint4*>(qrow + 32 * j)
                            : make_uint4(0u, 0u, 0u, 0u);
      }
      __builtin_amdgcn_sched_barrier(0);
      VState st;
      st.m = kNegInf;
      st.lp = 0.f;
#pragma unroll
      for (int b = 0; b < 8; ++b) st.o[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};

      int bad = 0;
      VTile ta, tb;
      // both loads unconditional (a one-tile item reads its tile twice), so
      // the same loads are in flight on every path and the waits stay exact
      VIds<P> ids0, ids1;
      if constexpr (P % 16 == 0) {
        ids0.id = id0;
        ids1.id = P == 16 ? id1 : id0;
      } else {
        // the item row's two ids cover 2 P tokens here; read the tiles' own
        ids0 = v_read_ids<P>(idx, len, 0, kg);
        ids1 = v_read_ids<P>(idx, len, min(1, ntiles - 1), kg);
      }
      v_load(ta, c, v_ref<P>(c, ids0, len, 0, kg, bad));
      v_load(tb, c, v_ref<P>(c, ids1, len, min(1, ntiles - 1), kg, bad));
      VIds<P> id_next = v_read_ids<P>(idx, len, min(2, ntiles - 1), kg);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) sh.qa[j][lane] = qv[j];
      __builtin_amdgcn_wave_barrier();
      const int last_valid = len - 16 * (ntiles - 1);
      const VRef<P> none = {};
      int n = 0;
      // Two tiles form the ring; each is refilled as soon as it is staged in
      // LDS (its registers are free from then on), so while a tile is
      // computed the next one and the one after it are in flight.  Two tiles
      // per straight-line trip.
      auto step2 = [&](VTile& cur) -> bool {
        if (n == ntiles - 1) {
          v_step<false, true, P>(st, cur, cur, c, none, last_valid, lane, scale_log2, sh);
          return true;
        }
        if (n + 2 < ntiles) {
          const VRef<P> ref = v_ref<P>(c, id_next, len, n + 2, kg, bad);
          id_next = v_read_ids<P>(idx, len, min(n + 3, ntiles - 1), kg);
          v_step<true, false, P>(st, cur, cur, c, ref, 16, lane, scale_log2, sh);
        } else {
          v_step<false, false, P>(st, cur, cur, c, none, 16, lane, scale_log2, sh);
        }
        ++n;
        return false;
      };
      while (n + 3 < ntiles) {
        keep_pace<kMaxWavesPerBlock>(progress, wave, nwaves, lockstep, done_tiles + n);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          VTile& cur = k == 0 ? ta : tb;
          const VRef<P> ref = v_ref<P>(c, id_next, len, n + 2, kg, bad);
          id_next = v_read_ids<P>(idx, len, min(n + 3, ntiles - 1), kg);
          v_step<true, false, P>(st, cur, cur, c, ref, 16, lane, scale_log2, sh);
          ++n;
        }
      }
      for (;;) {
        if (step2(ta)) break;
        if (step2(tb)) break;
      }
      report_bad_pages(bad, lane, err, PKD_DEVERR_PAGE_ID);
      __builtin_amdgcn_s_setprio(0);
      done_tiles += ntiles;

      // lane (row l & 15, kg) holds head dims 16 b + 4 kg + v of its row
      const float l_row = rows_sum(st.lp);
      if (row16 < G) {
        const float inv = 1.f / l_row;
        const float lse_nat = (st.m + __log2f(l_row)) * kLn2;
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
}  // namespace pv
}  // namespace pkd
