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
// K of the next tile is requested as soon as the current tile's logits are
// formed, V of the next tile as soon as the current V is consumed.
//
// The data path is HBM-bound (aicassindra "Why serving attention is a
// different problem": decode streams every cached key and value once), so no
// matrix cores: a g x 16 logit tile would fill a 16-row MFMA tile only at
// g = 16.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"
#include "pkd.h"

namespace pkd {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a row: swap neighbours, swap pairs, mirror
// halves, mirror the row.  Every lane of the row ends with the same bits.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

// Combine the 4 rows of a wave: exchange with the row 32 lanes away, then
// with the neighbouring row.  Each swap returns both halves, so lane L sees
// its own value and the one at L ^ 32 (then L ^ 16).
__device__ __forceinline__ float rows_max(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  v = fmaxf(__builtin_bit_cast(float, a[0]), __builtin_bit_cast(float, a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  return fmaxf(__builtin_bit_cast(float, b[0]), __builtin_bit_cast(float, b[1]));
}

__device__ __forceinline__ float rows_sum(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  v = __builtin_bit_cast(float, a[0]) + __builtin_bit_cast(float, a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  return __builtin_bit_cast(float, b[0]) + __builtin_bit_cast(float, b[1]);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Page ids of one 16-token tile.  Page sizes that are multiples of 16 keep a
// tile inside one page (one id for the wave); smaller ones spread a tile over
// 16/P pages, so each lane looks up the page of each of its 4 rows.
template <int P, bool kWholeTile = (P % 16 == 0)>
struct TileIds;

template <int P>
struct TileIds<P, true> {
  int64_t page;
};

template <int P>
struct TileIds<P, false> {
  int32_t page[4];
};

struct Chunk {
  const int32_t* idx;  // kv_indices of the chunk (first page)
  int len;             // tokens in the chunk
  int ntiles;
};

__device__ __forceinline__ int tile_row(const Chunk& ch, int n, int i, int R) {
  // Rows past the end of the chunk re-read its last token; their logits are
  // masked, so the values never matter, and no slot past last_page_len (or
  // past the request's pages) is touched.
  const int valid = min(16, ch.len - 16 * n);
  return min(4 * i + R, valid - 1);
}

__device__ __forceinline__ int64_t checked_page(int32_t pg, int64_t num_pages, int32_t* err,
                                                int lane) {
  if (pg < 0 || pg >= num_pages) {
    if (lane == 0) err[0] = PKD_DEVERR_PAGE_ID;
    return 0;
  }
  return pg;
}

template <int P>
__device__ __forceinline__ TileIds<P> tile_ids(const Chunk& ch, int n, int R, int lane,
                                               const DecodeParams& p) {
  TileIds<P> t;
  if constexpr (P % 16 == 0) {
    t.page = checked_page(ch.idx[(16 * n) / P], p.num_pages, p.err, lane);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 16 * n + tile_row(ch, n, i, R);
      int32_t pg = ch.idx[tok / P];
      if (pg < 0 || pg >= p.num_pages) {
        p.err[0] = PKD_DEVERR_PAGE_ID;
        pg = 0;
      }
      t.page[i] = pg;
    }
  }
  return t;
}

// Element offset of row i of tile n (K half; V is v_off further).
template <int P>
__device__ __forceinline__ int64_t row_offset(const TileIds<P>& t, const Chunk& ch, int n, int i,
                                              int R, int64_t page_stride, int64_t row_stride) {
  const int row = tile_row(ch, n, i, R);
  if constexpr (P % 16 == 0) {
    return t.page * page_stride + int64_t((16 * n) % P + row) * row_stride;
  } else {
    return int64_t(t.page[i]) * page_stride + int64_t(row % P) * row_stride;
  }
}

template <int G, int P>
__global__ __launch_bounds__(512) void decode_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int R = lane >> 4;
  const int c = lane & 15;
  const int Hq = p.num_qo_heads;
  const int Hkv = p.num_kv_heads;

  const int32_t* hdr = p.ws + PKD_HEADER_BASE;
  const int32_t* slot_indptr = p.ws + hdr[PKD_H_OFF_SLOTS];
  const int32_t* items = p.ws + hdr[PKD_H_OFF_ITEMS];
  const int32_t* kv_idx = p.ws + hdr[PKD_H_OFF_INDICES];
  const int64_t n_partials = hdr[PKD_H_PARTIALS];
  float* o_part = p.fws;
  float* lse_part = p.fws + n_partials * Hq * kHeadDim;

  const int64_t row_stride = int64_t(Hkv) * kHeadDim;
  const int64_t v_off = int64_t(P) * row_stride;
  const int64_t page_stride = 2 * v_off;

  const int it_end = slot_indptr[blockIdx.x + 1];
  for (int it = slot_indptr[blockIdx.x]; it < it_end; ++it) {
    const int32_t* item = items + 8 * it;
    const int req = item[0];
    const int out = item[4];
    Chunk ch;
    ch.idx = kv_idx + item[1];
    ch.len = item[5];
    ch.ntiles = (ch.len + 15) >> 4;

    for (int kh = wave; kh < Hkv; kh += nwaves) {
      const uint16_t* head = p.kv + int64_t(kh) * kHeadDim + c * 8;

      uint4 qv[G];
      const uint16_t* qrow = p.q + (int64_t(req) * Hq + kh * G) * kHeadDim + c * 8;
#pragma unroll
      for (int r = 0; r < G; ++r) qv[r] = *reinterpret_cast<const uint4*>(qrow + r * kHeadDim);

      float m[G], l[G], acc[G][8];
#pragma unroll
      for (int r = 0; r < G; ++r) {
        m[r] = kNegInf;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
      }

      uint4 kr[4], vr[4];
      {
        const TileIds<P> t0 = tile_ids<P>(ch, 0, R, lane, p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t off = row_offset<P>(t0, ch, 0, i, R, page_stride, row_stride);
          kr[i] = *reinterpret_cast<const uint4*>(head + off);
          vr[i] = *reinterpret_cast<const uint4*>(head + off + v_off);
        }
      }
      TileIds<P> next = tile_ids<P>(ch, min(1, ch.ntiles - 1), R, lane, p);

      for (int n = 0; n < ch.ntiles; ++n) {
        const bool more = n + 1 < ch.ntiles;
        const TileIds<P> after = tile_ids<P>(ch, min(n + 2, ch.ntiles - 1), R, lane, p);

        // logits of the 4 rows of this lane's token row, scaled to base 2
        float s[4][G];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int r = 0; r < G; ++r) {
            float a = dot2_bf16(qv[r].x, kr[i].x, 0.f);
            a = dot2_bf16(qv[r].y, kr[i].y, a);
            a = dot2_bf16(qv[r].z, kr[i].z, a);
            a = dot2_bf16(qv[r].w, kr[i].w, a);
            s[i][r] = row_sum16(a) * p.scale_log2;
          }
        }
        if (n == ch.ntiles - 1) {
          const int valid = ch.len - 16 * n;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * i + R >= valid) {
#pragma unroll
              for (int r = 0; r < G; ++r) s[i][r] = kNegInf;
            }
        }
        if (more) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            kr[i] = *reinterpret_cast<const uint4*>(
                head + row_offset<P>(next, ch, n + 1, i, R, page_stride, row_stride));
        }

        // online softmax: rescale the running state when the maximum grows
        float mt[G];
        bool grow = false;
#pragma unroll
        for (int r = 0; r < G; ++r) {
          mt[r] = rows_max(fmaxf(fmaxf(s[0][r], s[1][r]), fmaxf(s[2][r], s[3][r])));
          grow |= mt[r] > m[r];
        }
        if (grow) {
#pragma unroll
          for (int r = 0; r < G; ++r) {
            const float mn = fmaxf(m[r], mt[r]);
            const float scale = __builtin_amdgcn_exp2f(m[r] - mn);
            m[r] = mn;
            l[r] *= scale;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] *= scale;
          }
        }

#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float vf[8];
          vf[0] = bf16_lo(vr[i].x);
          vf[1] = bf16_hi(vr[i].x);
          vf[2] = bf16_lo(vr[i].y);
          vf[3] = bf16_hi(vr[i].y);
          vf[4] = bf16_lo(vr[i].z);
          vf[5] = bf16_hi(vr[i].z);
          vf[6] = bf16_lo(vr[i].w);
          vf[7] = bf16_hi(vr[i].w);
#pragma unroll
          for (int r = 0; r < G; ++r) {
            const float pr = __builtin_amdgcn_exp2f(s[i][r] - m[r]);
            l[r] += pr;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(pr, vf[e], acc[r][e]);
          }
        }
        if (more) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vr[i] = *reinterpret_cast<const uint4*>(
                head + row_offset<P>(next, ch, n + 1, i, R, page_stride, row_stride) + v_off);
        }
        next = after;
      }

      // totals over the 4 token rows; every lane then holds the full state
#pragma unroll
      for (int r = 0; r < G; ++r) {
        l[r] = rows_sum(l[r]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = rows_sum(acc[r][e]);
      }

#pragma unroll
      for (int r = 0; r < G; ++r) {
        if ((r & 3) != R) continue;
        const float inv = 1.f / l[r];
        const float lse_nat = (m[r] + __log2f(l[r])) * kLn2;
        const int64_t qh = kh * G + r;
        if (out < 0) {
          uint4 w;
          w.x = pack_bf16x2(acc[r][0] * inv, acc[r][1] * inv);
          w.y = pack_bf16x2(acc[r][2] * inv, acc[r][3] * inv);
          w.z = pack_bf16x2(acc[r][4] * inv, acc[r][5] * inv);
          w.w = pack_bf16x2(acc[r][6] * inv, acc[r][7] * inv);
          *reinterpret_cast<uint4*>(p.o + (int64_t(req) * Hq + qh) * kHeadDim + c * 8) = w;
          if (p.lse && c == 0) p.lse[int64_t(req) * Hq + qh] = lse_nat;
        } else {
          float* dst = o_part + (int64_t(out) * Hq + qh) * kHeadDim + c * 8;
          *reinterpret_cast<float4*>(dst) =
              make_float4(acc[r][0] * inv, acc[r][1] * inv, acc[r][2] * inv, acc[r][3] * inv);
          *reinterpret_cast<float4*>(dst + 4) =
              make_float4(acc[r][4] * inv, acc[r][5] * inv, acc[r][6] * inv, acc[r][7] * inv);
          if (c == 0) lse_part[int64_t(out) * Hq + qh] = lse_nat;
        }
      }
    }
  }
}

template <int G, int P>
hipError_t launch_one(const DecodeParams& p, int num_slots, hipStream_t stream) {
  const int waves = p.num_kv_heads < kMaxWavesPerBlock ? p.num_kv_heads : kMaxWavesPerBlock;
  hipLaunchKernelGGL((decode_kernel<G, P>), dim3(num_slots), dim3(64 * waves), 0, stream, p);
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

int decode_blocks_per_cu(int waves_per_block) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_kernel<4, 16>,
                                                   64 * waves_per_block, 0) != hipSuccess)
    return 1;
  return blocks < 1 ? 1 : blocks;
}

}  // namespace pkd
