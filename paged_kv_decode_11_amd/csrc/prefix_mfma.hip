// Shared-prefix (composable) attention kernel for gfx950.
//
// A group of requests that share a prefix is one block row of the KV
// matrix (pinghaoyang FlashInfer page, section "Composable Format：共享前缀与
// 独有后缀分开算"): one workgroup reads each K/V tile of the prefix once and
// applies it to every query row of the group's row block, instead of each
// request reading the prefix for itself.  The result is the attention state
// of every (request, query head) over the group's tokens, written as the
// final bf16 output or, when the group's pages are split into chunks, as fp32
// partial states that the merge kernel combines exactly (same page, section
// "在线 Softmax 为什么允许任意切块").
//
// One workgroup (8 waves) takes one item: one KV head of one (group, row
// block, chunk).  Wave w owns 16 query rows, 16 / g requests times the g
// query heads of the KV head, so the workgroup covers 128 / g requests.
// Per 16-token tile:
//   * the 512 lanes load the head's K and V rows of the tile (16 rows x 256
//     bytes each, one 16-byte piece per lane) into registers, kDepth tiles
//     ahead, and stage them in LDS: K row-major with its 16-byte pieces
//     rotated by XOR of the row, V transposed to [d][token];
//   * S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16, K from LDS
//     as the A operand, the wave's q rows as B), which leaves lane l with the
//     logits of query row l & 15 for tokens 4 (l >> 4) .. +3;
//   * the online softmax per query row: a max over those 4 tokens and over
//     the 4 lanes holding the same row (permlane swaps), exponentials in base
//     2;
//   * O += P V on the matrix cores (v_mfma_f32_16x16x16_bf16, P as bf16
//     straight from the softmax registers as the A operand, V^T from LDS as
//     B), 8 column blocks of 16 elements of head_dim.
// The rescale factors and the final max and sum move from "row l & 15" to the
// accumulator's "rows 4 (l >> 4) + v" layout through a per-wave LDS row.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"
#include "pkd.h"
#include "plan_layout.h"

namespace pkd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kDepth = 8;       // tiles in flight per workgroup
constexpr int kVtStride = 20;   // bf16 per head_dim row of the transposed V tile (16 + pad)

struct PShared {
  uint4 kt[2][16][16];                   // K tile: row r's 16-byte piece c at [r][c ^ r]
  uint16_t vt[2][kHeadDim * kVtStride];  // V tile transposed: [d][token]
  float xa[kWaves][16];                  // per wave, per query row: rescale factor, then max
  float xl[kWaves][16];                  // per wave, per query row: final sum
};

__device__ __forceinline__ floatx4_t mfma_kq(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx4_t mfma_pv(uint2 a, uint2 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a),
                                                   __builtin_bit_cast(short4_t, b), c, 0, 0, 0);
}

template <int G, int P>
__global__ __launch_bounds__(kThreads) void prefix_mfma_kernel(
    const uint16_t* __restrict__ q_ptr, const uint16_t* __restrict__ kv_ptr,
    uint16_t* __restrict__ o_ptr, float* __restrict__ lse_ptr, const int32_t* __restrict__ ws,
    float* __restrict__ fws, int32_t* __restrict__ err, int64_t num_pages, float scale_log2,
    int num_qo_heads, int num_kv_heads) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  static_assert(P % 16 == 0, "a 16-token tile must lie in one page");
  constexpr int kReqPerWave = 16 / G;
  __shared__ PShared sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row16 = lane & 15;
  const int kg = lane >> 4;
  // load role: half of the lanes move K, half V; 16 lanes per 256-byte row
  const int ld_v = tid >> 8;
  const int ld_row = (tid >> 4) & 15;
  const int ld_piece = tid & 15;

  const int32_t* hdr = ws + PKD_HEADER_BASE;
  const int num_slots = gridDim.x;
  const int32_t* slot_indptr = ws + plan_off_slots();
  const int32_t* items = ws + plan_off_items(num_slots);
  const int32_t* kv_idx = ws + hdr[PKD_H_OFF_INDICES];
  const int32_t* groups = ws + hdr[PKD_H_OFF_GROUPS];
  const int rows_per_block = hdr[PKD_H_ROWS_PER_BLOCK];
  const int64_t n_partials = hdr[PKD_H_PARTIALS];
  const int Hq = num_qo_heads;
  float* o_part = fws;
  float* lse_part = fws + n_partials * Hq * kHeadDim;

  const uint32_t row_bytes = uint32_t(num_kv_heads) * kHeadDim * 2;
  const uint64_t v_bytes = uint64_t(P) * row_bytes;
  const uint64_t page_bytes = 2 * v_bytes;
  const char* kv = reinterpret_cast<const char*>(kv_ptr);
  int bad = 0;

  const int it_end = slot_indptr[blockIdx.x + 1];
  for (int it = slot_indptr[blockIdx.x]; it < it_end; ++it) {
    const int32_t* item = items + 8 * it;
    const int grp = item[0];
    const int32_t* idx = kv_idx + item[1];
    const int out = item[4];
    const int len = item[5];
    const int block = item[6];
    const int kh = item[7];
    const int row0 = groups[4 * grp + 0];
    const int rows = groups[4 * grp + 1];
    const int kchunks = groups[4 * grp + 2];
    const int ntiles = (len + 15) >> 4;
    const int last_valid = len - 16 * (ntiles - 1);

    // this wave's requests: first row (group-relative) and count
    const int wrow = block * rows_per_block + wave * kReqPerWave;
    const int nreq = min(kReqPerWave, rows - wrow);  // <= 0: the wave only loads
    const bool compute = nreq > 0;

    // q as the B operand: lane l holds query row l & 15 (request (l & 15) / g,
    // head kh g + (l & 15) % g), head_dim elements 32 j + 8 kg .. + 8
    uint4 qv[4];
    {
      const int i = row16 / G;
      const bool have = compute && i < nreq;
      const uint16_t* qrow =
          q_ptr + ((int64_t(row0) + wrow + (have ? i : 0)) * Hq + kh * G + row16 % G) * kHeadDim +
          kg * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        qv[j] = have ? *reinterpret_cast<const uint4*>(qrow + 32 * j) : make_uint4(0u, 0u, 0u, 0u);
    }

    float m = kNegInf, lsum = 0.f;
    floatx4_t acc[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) acc[cb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // this lane's piece of tile t
    auto tile_addr = [&](int t) -> const uint4* {
      const int64_t pg = safe_page(idx[(16 * t) / P], num_pages, bad);
      const uint64_t off = uint64_t(pg) * page_bytes + (ld_v ? v_bytes : 0) +
                           uint64_t((16 * t) % P + ld_row) * row_bytes +
                           uint64_t(kh) * kHeadDim * 2 + uint64_t(ld_piece) * 16;
      return reinterpret_cast<const uint4*>(kv + off);
    };

    uint4 ring[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (d < ntiles) ring[d] = load_stream16(tile_addr(d));

    for (int n0 = 0; n0 < ntiles; n0 += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int n = n0 + d;
        if (n >= ntiles) break;
        const int stage = n & 1;
        const bool last = n == ntiles - 1;
        const int valid = last ? last_valid : 16;
        // stage tile n in LDS; rows past the valid ones hold zeros in V (a
        // zero probability must not meet a stale or NaN value)
        if (!ld_v) {
          sh.kt[stage][ld_row][ld_piece ^ ld_row] = ring[d];
        } else {
          const uint4 w = ld_row < valid ? ring[d] : make_uint4(0u, 0u, 0u, 0u);
          const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
          uint16_t* col = sh.vt[stage] + (ld_piece * 8) * kVtStride + ld_row;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            col[(2 * e) * kVtStride] = uint16_t(ww[e] & 0xffffu);
            col[(2 * e + 1) * kVtStride] = uint16_t(ww[e] >> 16);
          }
        }
        __syncthreads();
        if (n + kDepth < ntiles) ring[d] = load_stream16(tile_addr(n + kDepth));
        if (!compute) continue;

        // S^T = K Q^T: lane l gets query row l & 15, tokens 4 kg + v
        floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          s = mfma_kq(sh.kt[stage][row16][(4 * j + kg) ^ row16], qv[j], s);
        float sv[4];
        float mx = kNegInf;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          sv[v] = (4 * kg + v < valid) ? s[v] * scale_log2 : kNegInf;
          mx = fmaxf(mx, sv[v]);
        }
        const float mn = fmaxf(m, rows_max(mx));
        const float alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 while m = -inf
        float p[4];
        float ps = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          p[v] = __builtin_amdgcn_exp2f(sv[v] - mn);
          ps += p[v];
        }
        lsum = fmaf(lsum, alpha, ps);
        m = mn;
        // rescale factors to the accumulator's row layout (rows 4 kg + v)
        if (kg == 0) sh.xa[wave][row16] = alpha;
        __builtin_amdgcn_wave_barrier();
        const float4 a4 = *reinterpret_cast<const float4*>(&sh.xa[wave][4 * kg]);
        __builtin_amdgcn_wave_barrier();
        const uint2 pa = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
        const uint16_t* vcol = sh.vt[stage] + row16 * kVtStride + 4 * kg;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          acc[cb][0] *= a4.x;
          acc[cb][1] *= a4.y;
          acc[cb][2] *= a4.z;
          acc[cb][3] *= a4.w;
          const uint2 vb = *reinterpret_cast<const uint2*>(vcol + cb * 16 * kVtStride);
          acc[cb] = mfma_pv(pa, vb, acc[cb]);
        }
      }
    }

    if (compute) {
      // final per-row max and sum, to the accumulator's row layout
      const float lt = rows_sum(lsum);
      if (kg == 0) {
        sh.xa[wave][row16] = m;
        sh.xl[wave][row16] = lt;
      }
      __builtin_amdgcn_wave_barrier();
      const float4 m4 = *reinterpret_cast<const float4*>(&sh.xa[wave][4 * kg]);
      const float4 l4 = *reinterpret_cast<const float4*>(&sh.xl[wave][4 * kg]);
      __builtin_amdgcn_wave_barrier();
      const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 4 * kg + v;  // query row of the wave
        const int i = r / G;
        if (i >= nreq) continue;
        const int req_in_group = wrow + i;
        const int64_t qh = int64_t(kh) * G + r % G;
        const float inv = 1.f / lv[v];
        const float lse_nat = (mv[v] + __log2f(lv[v])) * kLn2;
        if (out < 0) {
          uint16_t* orow = o_ptr + ((int64_t(row0) + req_in_group) * Hq + qh) * kHeadDim + row16;
#pragma unroll
          for (int cb = 0; cb < 8; ++cb)
            orow[cb * 16] = uint16_t(pack_bf16x2(acc[cb][v] * inv, 0.f) & 0xffffu);
          if (lse_ptr && row16 == 0) lse_ptr[(int64_t(row0) + req_in_group) * Hq + qh] = lse_nat;
        } else {
          const int64_t pid = int64_t(out) + int64_t(req_in_group) * kchunks;
          float* prow = o_part + (pid * Hq + qh) * kHeadDim + row16;
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) prow[cb * 16] = acc[cb][v] * inv;
          if (row16 == 0) lse_part[pid * Hq + qh] = lse_nat;
        }
      }
    }
    // the next item's first tile reuses LDS stage 0
    __syncthreads();
  }
  if (bad && lane == 0) err[0] = PKD_DEVERR_PAGE_ID;
}

template <int G, int P>
hipError_t launch_p(const DecodeParams& p, int num_slots, hipStream_t stream) {
  hipLaunchKernelGGL((prefix_mfma_kernel<G, P>), dim3(num_slots), dim3(kThreads), 0, stream, p.q,
                     p.kv, p.o, p.lse, p.ws, p.fws, p.err, p.num_pages, p.scale_log2,
                     p.num_qo_heads, p.num_kv_heads);
  return hipGetLastError();
}

template <int G>
hipError_t launch_pg(const DecodeParams& p, int page_size, int num_slots, hipStream_t stream) {
  switch (page_size) {
    case 16: return launch_p<G, 16>(p, num_slots, stream);
    case 32: return launch_p<G, 32>(p, num_slots, stream);
    case 64: return launch_p<G, 64>(p, num_slots, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool prefix_variant_built(int g, int page_size) {
  return (g == 1 || g == 2 || g == 4 || g == 8) &&
         (page_size == 16 || page_size == 32 || page_size == 64);
}

hipError_t launch_prefix_mfma(const DecodeParams& p, int g, int page_size, int num_slots,
                              hipStream_t stream) {
  switch (g) {
    case 1: return launch_pg<1>(p, page_size, num_slots, stream);
    case 2: return launch_pg<2>(p, page_size, num_slots, stream);
    case 4: return launch_pg<4>(p, page_size, num_slots, stream);
    case 8: return launch_pg<8>(p, page_size, num_slots, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkd
