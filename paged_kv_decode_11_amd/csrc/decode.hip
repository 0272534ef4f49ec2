// Paged GQA decode kernel for gfx950.
//
// What it computes (pinghaoyang FlashInfer page, sections "从推理形状出发" and
// "在线 Softmax 为什么允许任意切块"): for each work item of the plan -- one
// request, a page-aligned chunk of its KV -- and each KV head, the attention
// state (o, lse) of the g query heads of that group over the chunk's tokens,
// with logits scaled by sm_scale.  Unsplit requests write the final bf16
// output and lse directly; chunks of split requests write fp32 partial
// states to the float workspace for the merge kernel.
//
// Mapping to the hardware.  A workgroup is one persistent slot of the plan;
// it walks its item list.  Each wave takes one KV head of the item.  The
// wave's 64 lanes are 4 rows of 16: lane (R, c) holds elements 8c..8c+7 of
// head_dim, so one 16-byte load per lane reads 4 whole 256-byte K (or V)
// head rows, tokens R, R+4, R+8, R+12 of a 16-token tile over four loads
// (gather: the page of every tile comes from kv_indices; head rows are
// contiguous, aicassindra "The block-sparse page table" / NHD layout).
// The g query rows of the group stay in registers as packed bf16 (GQA fold,
// aicassindra "GQA, tensor cores and MLA").  q.k partial sums use
// v_dot2_f32_bf16 on the packed pairs and are reduced over the 16 lanes of a
// row with DPP; the online softmax runs in base 2 (v_exp_f32) with the tile
// maximum taken across rows with permlane swaps; V accumulates in fp32.
// The next tile's K is requested as soon as the current logits are formed,
// its V as soon as the current V is consumed.
//
// The data path is HBM-bound (aicassindra "Why serving attention is a
// different problem": decode streams every cached key and value once), so no
// matrix cores: a g x 16 logit tile would fill a 16-row MFMA tile only at
// g = 16.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"
#include "pkd.h"
#include "plan_layout.h"

namespace pkd {
namespace {

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

struct Ctx {
  const uint16_t* __restrict__ q;
  const char* __restrict__ kv;  // cache base, bytes
  uint16_t* __restrict__ o;
  float* __restrict__ lse;
  float* __restrict__ o_part;
  float* __restrict__ lse_part;
  int64_t num_pages;
  float scale_log2;
  int Hq;
  int Hkv;
  uint32_t row_bytes;   // one token's K (or V) rows of all KV heads
  uint64_t v_bytes;     // K half of a page; V starts this far in
  uint64_t page_bytes;
};

// Running attention state of one (item, KV head) for the G query rows.
template <int G>
struct State {
  uint4 q[G];       // packed bf16, elements 8c..8c+7 of each query row
  float m[G];       // running max of the base-2 logits
  float l[G];       // running sum of exp2(logit - m), this lane's token rows only
  float acc[G][8];  // running sum of exp2(logit - m) * v, this lane's token rows only
};

// Where the 4 rows of one tile are.  Page sizes that are multiples of 16 keep
// a tile inside one page: one wave-uniform base address plus a 32-bit lane
// offset per row.  Smaller page sizes spread a tile over 16 / P pages: each
// lane carries the full address of each of its rows.
template <int P, bool kWhole = (P % 16 == 0)>
struct TileRef;

template <int P>
struct TileRef<P, true> {
  const char* kbase;  // K rows of the tile (wave-uniform)
  const char* vbase;  // V rows of the tile (wave-uniform)
  uint32_t off[4];    // this lane's byte offset of row i from either base
  __device__ __forceinline__ const uint4* k(int i) const {
    return reinterpret_cast<const uint4*>(kbase + off[i]);
  }
  __device__ __forceinline__ const uint4* v(int i) const {
    return reinterpret_cast<const uint4*>(vbase + off[i]);
  }
};

template <int P>
struct TileRef<P, false> {
  const char* row[4];
  uint64_t v_bytes;
  __device__ __forceinline__ const uint4* k(int i) const {
    return reinterpret_cast<const uint4*>(row[i]);
  }
  __device__ __forceinline__ const uint4* v(int i) const {
    return reinterpret_cast<const uint4*>(row[i] + v_bytes);
  }
};

// Page ids the next tiles need, read ahead of their use.  For whole-tile
// pages one wave-uniform id; otherwise one per row of this lane.
template <int P, bool kWhole = (P % 16 == 0)>
struct TileIds;

template <int P>
struct TileIds<P, true> {
  int32_t id;
};

template <int P>
struct TileIds<P, false> {
  int32_t id[4];
};

// Rows past the end of a chunk re-read its last token: their logits are
// masked, so the values never matter, and no slot past last_page_len (or past
// the request's pages) is read.
__device__ __forceinline__ int clamp_row(int i, int R, int valid) { return min(4 * i + R, valid - 1); }

template <int P>
__device__ __forceinline__ TileIds<P> read_ids(const int32_t* idx, int len, int t, int R) {
  TileIds<P> ids;
  const int valid = min(16, len - 16 * t);
  if constexpr (P % 16 == 0) {
    ids.id = idx[(16 * t) / P];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) ids.id[i] = idx[(16 * t + clamp_row(i, R, valid)) / P];
  }
  return ids;
}

template <int P>
__device__ __forceinline__ TileRef<P> tile_ref(const Ctx& p, const TileIds<P>& ids, int len, int t,
                                               int R, uint32_t col, int& bad) {
  TileRef<P> ref;
  const int valid = min(16, len - 16 * t);
  if constexpr (P % 16 == 0) {
    const int64_t pg = safe_page(ids.id, p.num_pages, bad);
    ref.kbase = p.kv + pg * p.page_bytes + uint64_t((16 * t) % P) * p.row_bytes;
    ref.vbase = ref.kbase + p.v_bytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) ref.off[i] = uint32_t(clamp_row(i, R, valid)) * p.row_bytes + col;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t pg = safe_page(ids.id[i], p.num_pages, bad);
      const int slot = clamp_row(i, R, valid) % P;
      ref.row[i] = p.kv + pg * p.page_bytes + uint64_t(slot) * p.row_bytes + col;
    }
    ref.v_bytes = p.v_bytes;
  }
  return ref;
}

template <int P>
__device__ __forceinline__ void load_k(uint4 (&dst)[4], const TileRef<P>& ref) {
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = load_stream16(ref.k(i));
}

template <int P>
__device__ __forceinline__ void load_v(uint4 (&dst)[4], const TileRef<P>& ref) {
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = load_stream16(ref.v(i));
}

// K and V rows of one 16-token tile held by this lane.
struct TileRegs {
  uint4 k[4];
  uint4 v[4];
};

// One 16-token tile: logits from t.k, online-softmax update, V from t.v.
// With kNext, the next tile's K is requested into t.k as soon as the logits
// are formed and its V into t.v as soon as this tile's V is consumed, so
// loads stream while the rest of the tile is computed; the last tile masks
// rows >= valid.
template <int G, int P, bool kNext>
__device__ __forceinline__ void tile_step(State<G>& st, TileRegs& t, const TileRef<P>& next,
                                          int valid, int R, float scale_log2, uint64_t v_bytes) {
  const TileRegs& cur = t;
  float s[4][G];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < G; ++r) {
      float a = dot2_bf16(st.q[r].x, cur.k[i].x, 0.f);
      a = dot2_bf16(st.q[r].y, cur.k[i].y, a);
      a = dot2_bf16(st.q[r].z, cur.k[i].z, a);
      a = dot2_bf16(st.q[r].w, cur.k[i].w, a);
      s[i][r] = row_sum16(a) * scale_log2;
    }
  }
  // The scheduling barriers keep each prefetch where it is written: left
  // alone, the scheduler sinks the loads to the end of the iteration to
  // shorten register live ranges, and the next tile is then waited on as
  // soon as it is requested.
  if constexpr (kNext) {
    __builtin_amdgcn_sched_barrier(0);
    load_k<P>(t.k, next);
    __builtin_amdgcn_sched_barrier(0);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * i + R >= valid) {
#pragma unroll
        for (int r = 0; r < G; ++r) s[i][r] = kNegInf;
      }
  }

  float mt[G];
  bool grow = false;
#pragma unroll
  for (int r = 0; r < G; ++r) {
    mt[r] = rows_max(fmaxf(fmaxf(s[0][r], s[1][r]), fmaxf(s[2][r], s[3][r])));
    grow |= mt[r] > st.m[r];
  }
  // m and mt hold the same value in every lane, so the branch is uniform
  if (__builtin_amdgcn_readfirstlane(int(grow))) {
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const float mn = fmaxf(st.m[r], mt[r]);
      const float scale = __builtin_amdgcn_exp2f(st.m[r] - mn);
      st.m[r] = mn;
      st.l[r] *= scale;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[r][e] *= scale;
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float vf[8];
    vf[0] = bf16_lo(cur.v[i].x);
    vf[1] = bf16_hi(cur.v[i].x);
    vf[2] = bf16_lo(cur.v[i].y);
    vf[3] = bf16_hi(cur.v[i].y);
    vf[4] = bf16_lo(cur.v[i].z);
    vf[5] = bf16_hi(cur.v[i].z);
    vf[6] = bf16_lo(cur.v[i].w);
    vf[7] = bf16_hi(cur.v[i].w);
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const float pr = __builtin_amdgcn_exp2f(s[i][r] - st.m[r]);
      st.l[r] += pr;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[r][e] = fmaf(pr, vf[e], st.acc[r][e]);
    }
  }
  if constexpr (kNext) {
    __builtin_amdgcn_sched_barrier(0);
    load_v<P>(t.v, next);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Pointers are separate __restrict__ arguments so the compiler knows the
// plan and kv_indices are not written by this kernel and reads them through
// the scalar cache.
template <int G, int P>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 8)))
void decode_kernel(
    const uint16_t* __restrict__ q_ptr, const uint16_t* __restrict__ kv_ptr,
    uint16_t* __restrict__ o_ptr, float* __restrict__ lse_ptr, const int32_t* __restrict__ ws,
    float* __restrict__ fws, int32_t* __restrict__ err, int64_t num_pages, float scale_log2,
    int num_qo_heads, int num_kv_heads) {
  const int lane = threadIdx.x & 63;
  // wave-uniform by construction; saying so keeps the item and page reads
  // in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int R = lane >> 4;
  const int c = lane & 15;

  // The slot's bounds, its first item and the header fields sit at offsets
  // fixed by the slot count (the grid size): requested together and waited
  // for at once (the empty asm), one round trip before the page ids.
  const int32_t* hdr = ws + PKD_HEADER_BASE;
  const int num_slots = gridDim.x;
  const int32_t* slot_indptr = ws + plan_off_slots();
  const int32_t* first = ws + plan_off_first(num_slots) + 8 * int64_t(blockIdx.x);
  const int it_begin = slot_indptr[blockIdx.x];
  const int it_end = slot_indptr[blockIdx.x + 1];
  const int first_req = first[0], first_page = first[1], first_out = first[4],
            first_len = first[5];
  const int off_indices = hdr[PKD_H_OFF_INDICES];
  const int partials = hdr[PKD_H_PARTIALS];
  const int off_items = hdr[PKD_H_OFF_ITEMS];
  asm volatile("" ::"s"(it_begin), "s"(it_end), "s"(first_req), "s"(first_page), "s"(first_out),
               "s"(first_len), "s"(off_indices), "s"(partials),
               "s"(off_items));
  const int32_t* items = ws + off_items;
  const int32_t* kv_idx = ws + off_indices;
  const int64_t n_partials = partials;

  Ctx p;
  p.q = q_ptr;
  p.kv = reinterpret_cast<const char*>(kv_ptr);
  p.o = o_ptr;
  p.lse = lse_ptr;
  p.o_part = fws;
  p.lse_part = fws + n_partials * num_qo_heads * kHeadDim;
  p.num_pages = num_pages;
  p.scale_log2 = scale_log2;
  p.Hq = num_qo_heads;
  p.Hkv = num_kv_heads;
  p.row_bytes = uint32_t(num_kv_heads) * kHeadDim * 2;
  p.v_bytes = uint64_t(P) * p.row_bytes;
  p.page_bytes = 2 * p.v_bytes;

  for (int it = it_begin; it < it_end; ++it) {
    int req = first_req, page_begin = first_page, out = first_out, len = first_len;
    if (it != it_begin) {
      const int32_t* item = items + 8 * it;
      req = item[0];
      page_begin = item[1];
      out = item[4];
      len = item[5];
    }
    const int32_t* idx = kv_idx + page_begin;
    const int ntiles = (len + 15) >> 4;

    for (int kh = wave; kh < p.Hkv; kh += nwaves) {
      const uint32_t col = uint32_t(kh * kHeadDim + c * 8) * 2;
      State<G> st;
      const uint16_t* qrow = p.q + (int64_t(req) * p.Hq + kh * G) * kHeadDim + c * 8;
#pragma unroll
      for (int r = 0; r < G; ++r) {
        st.q[r] = *reinterpret_cast<const uint4*>(qrow + r * kHeadDim);
        st.m[r] = kNegInf;
        st.l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[r][e] = 0.f;
      }

      int bad = 0;
      if constexpr (G > 4) {
        // g = 8 holds twice the query rows and accumulators; a second tile
        // in registers would spill, so one tile is in flight.  Page ids run
        // one tile ahead of the loads that use them.
        TileRegs t;
        {
          const TileRef<P> t0 = tile_ref<P>(p, read_ids<P>(idx, len, 0, R), len, 0, R, col, bad);
          load_k<P>(t.k, t0);
          load_v<P>(t.v, t0);
        }
        TileIds<P> ids_next = read_ids<P>(idx, len, ntiles > 1 ? 1 : 0, R);
        for (int n = 0; n + 1 < ntiles; ++n) {
          const TileRef<P> ref = tile_ref<P>(p, ids_next, len, n + 1, R, col, bad);
          ids_next = read_ids<P>(idx, len, min(n + 2, ntiles - 1), R);
          tile_step<G, P, true>(st, t, ref, 16, R, p.scale_log2, p.v_bytes);
        }
        const TileRef<P> none = {};
        tile_step<G, P, false>(st, t, none, len - 16 * (ntiles - 1), R, p.scale_log2, p.v_bytes);
      } else {
        // Two tiles in a register ring: while tile n is computed, tile n + 1
        // is in flight and tile n + 2 is requested into n's registers as they
        // free up.  Page ids run one tile ahead of the loads that use them.
        TileRegs ta, tb;
        {
          const TileRef<P> r0 = tile_ref<P>(p, read_ids<P>(idx, len, 0, R), len, 0, R, col, bad);
          load_k<P>(ta.k, r0);
          load_v<P>(ta.v, r0);
        }
        if (ntiles > 1) {
          const TileRef<P> r1 = tile_ref<P>(p, read_ids<P>(idx, len, 1, R), len, 1, R, col, bad);
          load_k<P>(tb.k, r1);
          load_v<P>(tb.v, r1);
        }
        TileIds<P> ids_next = read_ids<P>(idx, len, min(2, ntiles - 1), R);
        int n = 0;
        for (; n + 3 < ntiles; n += 2) {
          {
            const TileRef<P> ref = tile_ref<P>(p, ids_next, len, n + 2, R, col, bad);
            ids_next = read_ids<P>(idx, len, n + 3, R);
            tile_step<G, P, true>(st, ta, ref, 16, R, p.scale_log2, p.v_bytes);
          }
          {
            const TileRef<P> ref = tile_ref<P>(p, ids_next, len, n + 3, R, col, bad);
            ids_next = read_ids<P>(idx, len, min(n + 4, ntiles - 1), R);
            tile_step<G, P, true>(st, tb, ref, 16, R, p.scale_log2, p.v_bytes);
          }
        }
        // 1, 2 or 3 tiles remain; only the last one masks
        {
          const TileRef<P> none = {};
          const int last_valid = len - 16 * (ntiles - 1);
          if (ntiles - n == 3) {
            const TileRef<P> ref = tile_ref<P>(p, ids_next, len, n + 2, R, col, bad);
            tile_step<G, P, true>(st, ta, ref, 16, R, p.scale_log2, p.v_bytes);
            tile_step<G, P, false>(st, tb, none, 16, R, p.scale_log2, p.v_bytes);
            tile_step<G, P, false>(st, ta, none, last_valid, R, p.scale_log2, p.v_bytes);
          } else if (ntiles - n == 2) {
            tile_step<G, P, false>(st, ta, none, 16, R, p.scale_log2, p.v_bytes);
            tile_step<G, P, false>(st, tb, none, last_valid, R, p.scale_log2, p.v_bytes);
          } else {
            tile_step<G, P, false>(st, ta, none, last_valid, R, p.scale_log2, p.v_bytes);
          }
        }
      }
      report_bad_pages(bad, lane, err, PKD_DEVERR_PAGE_ID);

      // totals over the 4 token rows; every lane then holds the full state
#pragma unroll
      for (int r = 0; r < G; ++r) {
        st.l[r] = rows_sum(st.l[r]);
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[r][e] = rows_sum(st.acc[r][e]);
      }

#pragma unroll
      for (int r = 0; r < G; ++r) {
        if ((r & 3) != R) continue;
        const float inv = 1.f / st.l[r];
        const float lse_nat = (st.m[r] + __log2f(st.l[r])) * kLn2;
        const int64_t qh = kh * G + r;
        if (out < 0) {
          uint4 w;
          w.x = pack_bf16x2(st.acc[r][0] * inv, st.acc[r][1] * inv);
          w.y = pack_bf16x2(st.acc[r][2] * inv, st.acc[r][3] * inv);
          w.z = pack_bf16x2(st.acc[r][4] * inv, st.acc[r][5] * inv);
          w.w = pack_bf16x2(st.acc[r][6] * inv, st.acc[r][7] * inv);
          *reinterpret_cast<uint4*>(p.o + (int64_t(req) * p.Hq + qh) * kHeadDim + c * 8) = w;
          if (p.lse && c == 0) p.lse[int64_t(req) * p.Hq + qh] = lse_nat;
        } else {
          float* dst = p.o_part + (int64_t(out) * p.Hq + qh) * kHeadDim + c * 8;
          *reinterpret_cast<float4*>(dst) =
              make_float4(st.acc[r][0] * inv, st.acc[r][1] * inv, st.acc[r][2] * inv,
                          st.acc[r][3] * inv);
          *reinterpret_cast<float4*>(dst + 4) =
              make_float4(st.acc[r][4] * inv, st.acc[r][5] * inv, st.acc[r][6] * inv,
                          st.acc[r][7] * inv);
          if (c == 0) p.lse_part[int64_t(out) * p.Hq + qh] = lse_nat;
        }
      }
    }
  }
}

template <int G, int P>
hipError_t launch_one(const DecodeParams& p, int num_slots, hipStream_t stream) {
  const int waves = p.num_kv_heads < kMaxWavesPerBlock ? p.num_kv_heads : kMaxWavesPerBlock;
  hipLaunchKernelGGL((decode_kernel<G, P>), dim3(num_slots), dim3(64 * waves), 0, stream, p.q,
                     p.kv, p.o, p.lse, p.ws, p.fws, p.err, p.num_pages, p.scale_log2,
                     p.num_qo_heads, p.num_kv_heads);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(const DecodeParams& p, int page_size, int num_slots, hipStream_t stream) {
  switch (page_size) {
    case 1: return launch_one<G, 1>(p, num_slots, stream);
    case 2: return launch_one<G, 2>(p, num_slots, stream);
    case 4: return launch_one<G, 4>(p, num_slots, stream);
    case 8: return launch_one<G, 8>(p, num_slots, stream);
    case 16: return launch_one<G, 16>(p, num_slots, stream);
    case 32: return launch_one<G, 32>(p, num_slots, stream);
    case 64: return launch_one<G, 64>(p, num_slots, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_variant_built(int g, int page_size) {
  const bool g_ok = g == 1 || g == 2 || g == 4 || g == 8;
  const bool p_ok = page_size == 1 || page_size == 2 || page_size == 4 || page_size == 8 ||
                    page_size == 16 || page_size == 32 || page_size == 64;
  return g_ok && p_ok;
}

hipError_t launch_decode(const DecodeParams& p, int g, int page_size, int num_slots,
                         hipStream_t stream) {
  switch (g) {
    case 1: return launch_g<1>(p, page_size, num_slots, stream);
    case 2: return launch_g<2>(p, page_size, num_slots, stream);
    case 4: return launch_g<4>(p, page_size, num_slots, stream);
    case 8: return launch_g<8>(p, page_size, num_slots, stream);
    default: return hipErrorInvalidValue;
  }
}

int decode_blocks_per_cu_dot2(int waves_per_block) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_kernel<4, 16>,
                                                   64 * waves_per_block, 0) != hipSuccess)
    return 1;
  return blocks < 1 ? 1 : blocks;
}

}  // namespace pkd
