// Paged GQA decode kernel for gfx950 with the logits on the matrix cores.
//
// Same contract as decode_kernel (decode.hip): for each work item of the
// plan and each KV head, the attention state of the group's g query rows
// over the chunk's tokens (pinghaoyang FlashInfer page, sections
// "从推理形状出发" and "在线 Softmax 为什么允许任意切块"), written as the final
// bf16 output or as an fp32 partial state.
//
// What differs is how a 16-token tile is computed.  The GQA group is folded
// into the rows of a 16 x 16 logit tile (aicassindra "GQA, tensor cores and
// MLA": the g queries of a group form a small matrix), S = Q K^T, computed by
// four v_mfma_f32_16x16x32_bf16 over head_dim 128.  Rows g..15 of Q are zero.
// The B operand gives lane l 8 elements of token (l & 15)'s row per 32-wide
// step.  With pages of 16 tokens or more each lane loads 16-byte pieces of
// K row-major (whole 256-byte head rows per instruction) and the tile is
// transposed into operand layout through a per-wave LDS area whose pieces
// are XOR-rotated by row; smaller pages load the operand layout directly
// (16 bytes of each of the 16 rows per instruction).  The
// result leaves lane l with S[4 (l >> 4) + v][l & 15], v = 0..3: the online
// softmax needs only a 16-lane row maximum per register (DPP) and 8
// exponentials per tile.  The probabilities and the rescale factors go
// through a small per-wave LDS area to every lane, and P V runs in fp32 on
// the vector ALUs: lane l owns output elements 2l and 2l + 1 of every query
// row and reads one dword of each V row, so the 16 V loads of a tile each
// read one whole 256-byte row.
//
// K and V of the next two tiles stream into registers while the current
// tile is computed (three register tiles used in a ring).  One workgroup per
// compute unit, each wave with two tiles in flight, reads faster than more
// workgroups with less in flight each.  The path stays bound by
// HBM: the matrix cores do 4 instructions per 8 KiB tile, and the vector ALU
// work per tile is about half that of the dot-product kernel.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"
#include "pkd.h"
#include "plan_layout.h"

namespace pkd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4_t mfma_qk(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

struct MCtx {
  const char* __restrict__ kv;  // cache base, bytes
  int64_t num_pages;
  uint32_t row_bytes;  // one token's K (or V) rows of all KV heads
  uint64_t v_bytes;    // K half of a page; V starts this far in
  uint64_t page_bytes;
  uint32_t head_bytes;  // this wave's KV head offset within a token row
};

// Running state of one (item, KV head).
template <int G>
struct MState {
  float m[4];       // running max (base 2) of rows 4 (lane >> 4) + v
  float lp[4];      // sum of exp2(s - m) over this lane's tokens (column lane & 15), same rows
  float acc[G][2];  // unnormalised o[r][2 lane], o[r][2 lane + 1]
};

struct MTile {
  uint4 k[4];      // K: see MRef (row-major pieces, or the B operand directly)
  uint32_t v[16];  // V[token t][2 lane .. 2 lane + 1]
};

// Addresses of one tile.  Page sizes that are multiples of 16 keep the tile
// in one page: wave-uniform bases plus lane offsets.  Smaller ones give each
// lane its own K row address and each token its own (wave-uniform) V row.
template <int P, bool kWhole = (P % 16 == 0)>
struct MRef;

template <int P>
struct MRef<P, true> {
  __amdgpu_buffer_rsrc_t page;  // buffer over the tile's page
  uint32_t tile_off;            // byte offset of the tile's first K row in the page
  uint32_t koff;                // this lane's row (lane >> 4) and 16-byte piece (lane & 15)
  uint32_t row_bytes;           // token stride
  uint32_t v_off;               // tile_off + size of the page's K half
  int vlast;                    // last valid row of the tile
};

template <int P>
struct MRef<P, false> {
  const char* krow;      // this lane's K row, 8-element group included
  const char* vrow[16];  // V row of each token (clamped)
};

// Page ids of a tile, read one tile ahead of the loads that use them.
template <int P, bool kWhole = (P % 16 == 0)>
struct MIds;

template <int P>
struct MIds<P, true> {
  int32_t id;
};

template <int P>
struct MIds<P, false> {
  int32_t krow_id;   // page of this lane's K row
  int32_t tok[16];   // page of each token's V row
};

template <int P>
__device__ __forceinline__ MIds<P> m_read_ids(const int32_t* idx, int len, int t, int row16) {
  MIds<P> ids;
  const int valid = min(16, len - 16 * t);
  if constexpr (P % 16 == 0) {
    ids.id = idx[(16 * t) / P];
  } else {
    ids.krow_id = idx[(16 * t + min(row16, valid - 1)) / P];
#pragma unroll
    for (int i = 0; i < 16; ++i) ids.tok[i] = idx[(16 * t + min(i, valid - 1)) / P];
  }
  return ids;
}

// Ids of tile t (0 or 1) of an item.  With pages of 16 tokens or more both
// tiles lie in the item's first two pages, whose ids the item row carries
// (`id`): no read of the page table stands between an item's row and its
// first loads.
template <int P>
__device__ __forceinline__ MIds<P> m_start_ids(int32_t id, const int32_t* idx, int len, int t,
                                               int row16) {
  if constexpr (P % 16 == 0) {
    MIds<P> ids;
    ids.id = id;
    return ids;
  } else {
    return m_read_ids<P>(idx, len, t, row16);
  }
}

template <int P>
__device__ __forceinline__ MRef<P> m_tile_ref(const MCtx& c, const MIds<P>& ids, int len, int t,
                                              int row16, int kg, int& bad) {
  MRef<P> ref;
  const int valid = min(16, len - 16 * t);
  if constexpr (P % 16 == 0) {
    const int64_t pg = safe_page(ids.id, c.num_pages, bad);
    // raw buffer (stride 0) over one page; 0x00020000 in the last word selects
    // 32-bit data, as raw loads need; reads past the page return zeros
    ref.page = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(c.kv + pg * c.page_bytes),
                                                 0, int(c.page_bytes), 0x00020000);
    ref.tile_off = uint32_t((16 * t) % P) * c.row_bytes;
    // rows past the valid ones are still inside the page; their logits are
    // masked before use, so K needs no clamping here
    ref.koff = uint32_t(kg) * c.row_bytes + c.head_bytes + uint32_t(row16) * 16;
    ref.row_bytes = c.row_bytes;
    ref.v_off = ref.tile_off + uint32_t(c.v_bytes);
    ref.vlast = valid - 1;
  } else {
    const int krow = min(row16, valid - 1);
    const int64_t kp = safe_page(ids.krow_id, c.num_pages, bad);
    ref.krow = c.kv + kp * c.page_bytes + uint64_t(krow % P) * c.row_bytes + c.head_bytes + kg * 16;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t vp = safe_page(ids.tok[i], c.num_pages, bad);
      ref.vrow[i] = c.kv + vp * c.page_bytes + c.v_bytes +
                    uint64_t(min(i, valid - 1) % P) * c.row_bytes + c.head_bytes;
    }
  }
  return ref;
}

template <int P>
__device__ __forceinline__ void m_load(MTile& dst, const MRef<P>& ref, int lane,
                                       uint32_t head_bytes) {
  if constexpr (P % 16 == 0) {
    // K row-major: load j reads rows 4 j .. 4 j + 3, each whole 256-byte head
    // row by 16 lanes; the transpose to the operand layout goes through LDS
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b128(
          ref.page, ref.koff, ref.tile_off + uint32_t(4 * j) * ref.row_bytes, kBufferNontemporal);
      dst.k[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    const uint32_t voff = head_bytes + uint32_t(lane) * 4;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      dst.v[i] = __builtin_amdgcn_raw_buffer_load_b32(
          ref.page, voff, ref.v_off + uint32_t(min(i, ref.vlast)) * ref.row_bytes,
          kBufferNontemporal);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) dst.k[j] = load_stream16(ref.krow + 64 * j);
#pragma unroll
    for (int i = 0; i < 16; ++i) dst.v[i] = load_stream4(ref.vrow[i] + uint32_t(lane) * 4);
  }
}

// Per-wave LDS used to hand the tile's probabilities and rescale factors to
// every lane of the wave.
struct MShared {
  uint4 kt[16][16];  // K tile, row r's 16-byte piece c at [r][c ^ r]
  uint4 qa[4][64];  // A operand of step j for lane l: q row (l & 15), zero for rows >= g
  float4 p[64];     // lane l's p[v] for rows 4 (l >> 4) + v, token l & 15
  float4 scale[4];  // per 16-lane row group: rescale factors (then m at the end)
  float4 sum[4];    // per 16-lane row group: final l
};

// One tile: S from the matrix cores, online-softmax update, P V on the
// vector ALUs.  With kPrefetch a later tile's K and V are requested into `nxt`
// first, so they stream in while this one is computed; the last tile (kLast)
// masks tokens >= valid.
template <int G, int P, bool kPrefetch, bool kLast>
__device__ __forceinline__ void m_tile_step(MState<G>& st, const MTile& cur, MTile& nxt,
                                            const MRef<P>& next, int valid, int lane,
                                            uint32_t head_bytes, float scale_log2,
                                            MShared& sh) {
  const int row16 = lane & 15;
  const int kg = lane >> 4;
  if constexpr (kPrefetch) {
    // keep the prefetch where it is written (see decode.hip)
    __builtin_amdgcn_sched_barrier(0);
    m_load<P>(nxt, next, lane, head_bytes);
    __builtin_amdgcn_sched_barrier(0);
  }
  floatx4_t s = {0.f, 0.f, 0.f, 0.f};
  if constexpr (P % 16 == 0) {
    // Row-major K to the B operand (token lane & 15, 8 elements per lane):
    // through LDS, with the 16-byte pieces of row r rotated by XOR r so that
    // both the row writes and the column reads hit 16 distinct bank groups.
#pragma unroll
    for (int j = 0; j < 4; ++j) sh.kt[4 * j + kg][row16 ^ (4 * j + kg)] = cur.k[j];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 4; ++j) s = mfma_qk(sh.qa[j][lane], sh.kt[row16][(4 * j + kg) ^ row16], s);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) s = mfma_qk(sh.qa[j][lane], cur.k[j], s);
  }

  float p[4], alpha[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float sv = s[v] * scale_log2;
    if constexpr (kLast) {
      if (row16 >= valid) sv = kNegInf;
    }
    const float mn = fmaxf(st.m[v], row_max16(sv));
    alpha[v] = __builtin_amdgcn_exp2f(st.m[v] - mn);
    p[v] = __builtin_amdgcn_exp2f(sv - mn);
    st.lp[v] = fmaf(st.lp[v], alpha[v], p[v]);
    st.m[v] = mn;
  }
  sh.p[lane] = make_float4(p[0], p[1], p[2], p[3]);
  if (row16 == 0) sh.scale[kg] = make_float4(alpha[0], alpha[1], alpha[2], alpha[3]);
  // LDS accesses of one wave complete in order; the barrier only stops the
  // compiler from moving the reads above the writes of other lanes.
  __builtin_amdgcn_wave_barrier();

  {
    const float4 a0 = sh.scale[0];
    const float a03[4] = {a0.x, a0.y, a0.z, a0.w};
#pragma unroll
    for (int r = 0; r < (G < 4 ? G : 4); ++r) {
      st.acc[r][0] *= a03[r];
      st.acc[r][1] *= a03[r];
    }
    if constexpr (G > 4) {
      const float4 a1 = sh.scale[1];
      const float a47[4] = {a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int r = 4; r < G; ++r) {
        st.acc[r][0] *= a47[r - 4];
        st.acc[r][1] *= a47[r - 4];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    // a few tokens at a time, so the LDS reads of p are not all hoisted
    // into registers at once
    if (t % 4 == 0) __builtin_amdgcn_sched_barrier(0);
    const float lo = bf16_lo(cur.v[t]);
    const float hi = bf16_hi(cur.v[t]);
    const float4 p0 = sh.p[t];
    const float p03[4] = {p0.x, p0.y, p0.z, p0.w};
#pragma unroll
    for (int r = 0; r < (G < 4 ? G : 4); ++r) {
      st.acc[r][0] = fmaf(p03[r], lo, st.acc[r][0]);
      st.acc[r][1] = fmaf(p03[r], hi, st.acc[r][1]);
    }
    if constexpr (G > 4) {
      const float4 p1 = sh.p[16 + t];
      const float p47[4] = {p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int r = 4; r < G; ++r) {
        st.acc[r][0] = fmaf(p47[r - 4], lo, st.acc[r][0]);
        st.acc[r][1] = fmaf(p47[r - 4], hi, st.acc[r][1]);
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
}

template <int G, int P>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 8)))
void decode_mfma_kernel(const uint16_t* __restrict__ q_ptr, const uint16_t* __restrict__ kv_ptr,
                        uint16_t* __restrict__ o_ptr, float* __restrict__ lse_ptr,
                        const int32_t* __restrict__ ws, float* __restrict__ fws,
                        int32_t* __restrict__ err, int64_t num_pages, float scale_log2,
                        int num_qo_heads, int num_kv_heads) {
  static_assert(G >= 1 && G <= 8, "group size");
  __shared__ MShared shared[kMaxWavesPerBlock];
  // tiles each wave has completed; see the tile loop
  __shared__ int progress[kMaxWavesPerBlock];

  // The slot's bounds, its first item (with the ids of that item's first two
  // pages) and the header fields sit at offsets fixed by the slot count (the
  // grid size).  They are requested together, and the empty asm below makes
  // the kernel wait for them all at once: one round trip to memory before the
  // first K and V loads are issued.
  const int32_t* hdr = ws + PKD_HEADER_BASE;
  const int num_slots = gridDim.x;
  const int32_t* slot_indptr = ws + plan_off_slots();
  const int32_t* first = ws + plan_off_first(num_slots) + 8 * int64_t(blockIdx.x);
  const int it_begin = slot_indptr[blockIdx.x];
  const int it_end = slot_indptr[blockIdx.x + 1];
  const int first_req = first[0], first_page = first[1], first_out = first[4],
            first_len = first[5], first_id0 = first[6], first_id1 = first[7];
  const int off_indices = hdr[PKD_H_OFF_INDICES];
  const int partials = hdr[PKD_H_PARTIALS];
  const int off_items = hdr[PKD_H_OFF_ITEMS];

  asm volatile("" ::"s"(it_begin), "s"(it_end), "s"(first_req), "s"(first_page), "s"(first_out),
               "s"(first_len), "s"(first_id0), "s"(first_id1), "s"(off_indices), "s"(partials),
               "s"(off_items));
  const int32_t* items = ws + off_items;
  if ((threadIdx.x & 63) == 0) progress[threadIdx.x >> 6] = 0;
  __syncthreads();
  int done_tiles = 0;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  // every wave walks the same tiles when the heads divide evenly
  const bool lockstep = num_kv_heads % nwaves == 0;
  const int row16 = lane & 15;
  const int kg = lane >> 4;
  MShared& sh = shared[wave];

  const int32_t* kv_idx = ws + off_indices;
  const int64_t n_partials = partials;
  const int Hq = num_qo_heads;
  float* o_part = fws;
  float* lse_part = fws + n_partials * Hq * kHeadDim;

  MCtx c;
  c.kv = reinterpret_cast<const char*>(kv_ptr);
  c.num_pages = num_pages;
  c.row_bytes = uint32_t(num_kv_heads) * kHeadDim * 2;
  c.v_bytes = uint64_t(P) * c.row_bytes;
  c.page_bytes = 2 * c.v_bytes;

  for (int it = it_begin; it < it_end; ++it) {
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
      c.head_bytes = uint32_t(kh) * kHeadDim * 2;
      MState<G> st;
      // q stays in LDS in operand layout and is re-read for each tile, so it
      // holds no registers while V is accumulated.  It is loaded first and
      // staged after the first tiles' loads are issued, which do not wait
      // for it.
      uint4 qv[4];
      {
        const uint16_t* qrow = q_ptr + (int64_t(req) * Hq + kh * G + row16) * kHeadDim + kg * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          qv[j] = row16 < G ? *reinterpret_cast<const uint4*>(qrow + 32 * j)
                            : make_uint4(0u, 0u, 0u, 0u);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        st.m[v] = kNegInf;
        st.lp[v] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < G; ++r) st.acc[r][0] = st.acc[r][1] = 0.f;

      int bad = 0;
      // Three register tiles used in a ring: while tile n is computed, tiles
      // n + 1 and n + 2 stream in.  Page ids run one tile further ahead.
      MTile ta, tb, tc;
      m_load<P>(ta, m_tile_ref<P>(c, m_start_ids<P>(id0, idx, len, 0, row16), len, 0, row16, kg, bad),
                lane, c.head_bytes);
      if (ntiles > 1)
        m_load<P>(tb,
                  m_tile_ref<P>(c, m_start_ids<P>(P == 16 ? id1 : id0, idx, len, 1, row16), len,
                                1, row16, kg, bad),
                  lane, c.head_bytes);
      MIds<P> ids_next = m_read_ids<P>(idx, len, min(2, ntiles - 1), row16);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) sh.qa[j][lane] = qv[j];
      __builtin_amdgcn_wave_barrier();
      const int last_valid = len - 16 * (ntiles - 1);
      const MRef<P> none = {};
      int n = 0;
      // returns true once the last tile is done
      auto step = [&](MTile& cur, MTile& nxt) -> bool {
        if (n == ntiles - 1) {
          m_tile_step<G, P, false, true>(st, cur, nxt, none, last_valid, lane, c.head_bytes,
                                         scale_log2, sh);
          return true;
        }
        if (n + 2 < ntiles) {
          const MRef<P> ref = m_tile_ref<P>(c, ids_next, len, n + 2, row16, kg, bad);
          ids_next = m_read_ids<P>(idx, len, min(n + 3, ntiles - 1), row16);
          m_tile_step<G, P, true, false>(st, cur, nxt, ref, 16, lane, c.head_bytes, scale_log2,
                                         sh);
        } else {
          m_tile_step<G, P, false, false>(st, cur, nxt, none, 16, lane, c.head_bytes,
                                          scale_log2, sh);
        }
        ++n;
        return false;
      };
      for (;;) {
        // keep the waves of the workgroup together, every three tiles (all
        // waves walk the same items, so they meet the same barriers)
        keep_pace<kMaxWavesPerBlock>(progress, wave, nwaves, lockstep, done_tiles + n);
        if (step(ta, tc)) break;
        if (step(tb, ta)) break;
        if (step(tc, tb)) break;
      }
      report_bad_pages(bad, lane, err, PKD_DEVERR_PAGE_ID);
      __builtin_amdgcn_s_setprio(0);
      done_tiles += ntiles;

      // final l per row: sum over the 16 token columns; rows 4 kg + v
      float lt[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) lt[v] = row_sum16(st.lp[v]);
      if (row16 == 0) {
        sh.scale[kg] = make_float4(st.m[0], st.m[1], st.m[2], st.m[3]);
        sh.sum[kg] = make_float4(lt[0], lt[1], lt[2], lt[3]);
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const float4 mv = sh.scale[r >> 2];
        const float4 lv = sh.sum[r >> 2];
        const float mr = (r & 3) == 0 ? mv.x : (r & 3) == 1 ? mv.y : (r & 3) == 2 ? mv.z : mv.w;
        const float lr = (r & 3) == 0 ? lv.x : (r & 3) == 1 ? lv.y : (r & 3) == 2 ? lv.z : lv.w;
        const float inv = 1.f / lr;
        const float lse_nat = (mr + __log2f(lr)) * kLn2;
        const int64_t qh = kh * G + r;
        if (out < 0) {
          *reinterpret_cast<uint32_t*>(o_ptr + (int64_t(req) * Hq + qh) * kHeadDim + 2 * lane) =
              pack_bf16x2(st.acc[r][0] * inv, st.acc[r][1] * inv);
          if (lse_ptr && lane == 0) lse_ptr[int64_t(req) * Hq + qh] = lse_nat;
        } else {
          *reinterpret_cast<float2*>(o_part + (int64_t(out) * Hq + qh) * kHeadDim + 2 * lane) =
              make_float2(st.acc[r][0] * inv, st.acc[r][1] * inv);
          if (lane == 0) lse_part[int64_t(out) * Hq + qh] = lse_nat;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

template <int G, int P>
hipError_t launch_m(const DecodeParams& p, int num_slots, hipStream_t stream) {
  const int waves = p.num_kv_heads < kMaxWavesPerBlock ? p.num_kv_heads : kMaxWavesPerBlock;
  hipLaunchKernelGGL((decode_mfma_kernel<G, P>), dim3(num_slots), dim3(64 * waves), 0, stream,
                     p.q, p.kv, p.o, p.lse, p.ws, p.fws, p.err, p.num_pages, p.scale_log2,
                     p.num_qo_heads, p.num_kv_heads);
  return hipGetLastError();
}

template <int G>
hipError_t launch_mg(const DecodeParams& p, int page_size, int num_slots, hipStream_t stream) {
  switch (page_size) {
    case 1: return launch_m<G, 1>(p, num_slots, stream);
    case 2: return launch_m<G, 2>(p, num_slots, stream);
    case 4: return launch_m<G, 4>(p, num_slots, stream);
    case 8: return launch_m<G, 8>(p, num_slots, stream);
    case 16: return launch_m<G, 16>(p, num_slots, stream);
    case 32: return launch_m<G, 32>(p, num_slots, stream);
    case 64: return launch_m<G, 64>(p, num_slots, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int decode_blocks_per_cu(int waves_per_block) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_mfma_kernel<4, 16>,
                                                   64 * waves_per_block, 0) != hipSuccess)
    return 1;
  return blocks < 1 ? 1 : blocks;
}

hipError_t launch_decode_mfma(const DecodeParams& p, int g, int page_size, int num_slots,
                              hipStream_t stream) {
  switch (g) {
    case 1: return launch_mg<1>(p, page_size, num_slots, stream);
    case 2: return launch_mg<2>(p, page_size, num_slots, stream);
    case 4: return launch_mg<4>(p, page_size, num_slots, stream);
    case 8: return launch_mg<8>(p, page_size, num_slots, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkd
