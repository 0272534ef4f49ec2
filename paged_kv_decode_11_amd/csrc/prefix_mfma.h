// Device code of the shared-prefix (composable) attention kernel
// (prefix_mfma_kernel in prefix_mfma.hip), as a function of the slot a
// workgroup serves, so that another kernel can run it on part of its grid
// (the composable kernel in composable.hip).  Internal to the library.
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
// Per 64-token tile (four 16-token quarters, each within one page):
//   * every lane loads one 16-byte piece of two K rows and of two V rows of
//     the head (64 rows x 256 bytes each), kDepth tiles ahead, and stages
//     them in LDS row-major, the 16-byte pieces of row r rotated by XOR r;
//   * S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16 per quarter,
//     K from LDS as the A operand, the wave's q rows as B), which leaves lane
//     l with the logits of query row l & 15 for tokens 4 (l >> 4) .. +3 of
//     each quarter;
//   * the online softmax per query row: a max over those 16 tokens and over
//     the 4 lanes holding the same row (permlane swaps), exponentials in base
//     2;
//   * O^T += V^T P^T on the matrix cores (v_mfma_f32_16x16x32_bf16, 32 tokens
//     -- two quarters -- per instruction, 8 blocks of 16 elements of
//     head_dim): the transposing LDS read (ds_read_b64_tr_b16) gives each
//     lane the A operand of its head dim, 4 consecutive tokens of each
//     quarter, and P as bf16 straight from the softmax registers is the B
//     operand.  The product leaves lane l with
//     query row l & 15 (head dims 16 b + 4 (l >> 4) + v), the row the
//     softmax keeps in that lane, so rescale factors and the final max and
//     sum never move between lanes.
//
// Over an FP8 E4M3 cache (kFp8) a head row is 128 bytes of codes: every lane
// loads one 16-byte piece of one K row and of one V row per tile and
// stages it as two bf16 pieces (every E4M3 value is exact in bf16), so the
// LDS tiles and the products are those of the bf16 cache.  P enters P V as
// a bf16 high part and the bf16 rounding of its remainder (two products),
// about 16 bits of each probability, so the output error does not grow
// with the values' magnitude (up to 448 v_scale).  k_scale is folded into
// the logit scale and v_scale into the final normalisation.

#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"
#include "pkd.h"
#include "plan_layout.h"

namespace pkd {
namespace prefix {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;   // tokens per tile (four quarters of 16)
constexpr int kDepth = 4;   // tiles in flight per workgroup

// A wave's 16 fp32 output rows, staged in LDS at the end of an item so that
// each store instruction writes two whole 512-byte rows: rows 528 bytes apart
// (512 + 16), so the 16 rows one wave writes per instruction start 4 banks
// apart.
constexpr int kEpiRowBytes = 528;
constexpr int kEpiWaveBytes = 16 * kEpiRowBytes;

struct PTiles {
  uint4 k[2][kTile][16];  // K tile, row r's 16-byte piece c at [r][c ^ (r & 15)]
  uint4 v[2][kTile][16];  // V tile, same layout
};

union PShared {
  PTiles t;
  char epi[kWaves * kEpiWaveBytes];  // partial-state rows of each wave, after the last tile
};

__device__ __forceinline__ floatx4_t mfma32(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Transposing LDS read: for the 16 lanes of a row group, lane i receives
// element i % 4 of the 8-byte piece addressed by lane 4 r + i / 4 of its
// group, for r = 0..3.
__device__ __forceinline__ uint2 lds_read_tr(const void* p) {
  typedef __attribute__((address_space(3))) short4_t lds_short4;
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// One workgroup's work: the items of slot `slot` of `num_slots`, with `sh`
// its LDS.  Needs kThreads lanes.  kFp8: the cache holds E4M3 codes;
// out_scale multiplies every output (v_scale; 1 for a bf16 cache).
template <int G, int P, bool kFp8>
__device__ __forceinline__ void prefix_body(
    const uint16_t* __restrict__ q_ptr, const uint16_t* __restrict__ kv_ptr,
    uint16_t* __restrict__ o_ptr, float* __restrict__ lse_ptr, const int32_t* __restrict__ ws,
    float* __restrict__ fws, int32_t* __restrict__ err, int64_t num_pages, float scale_log2,
    float out_scale, int num_qo_heads, int num_kv_heads, int slot, int num_slots, PShared& sh) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  static_assert(P % 16 == 0, "a 16-token half tile must lie in one page");
  constexpr int kReqPerWave = 16 / G;
  // bytes per cached element; 16-byte pieces per head row; tile rows one
  // pass of the workgroup's lanes loads; passes per tile
  constexpr int kElem = kFp8 ? 1 : 2;
  constexpr int kPieces = kHeadDim * kElem / 16;
  constexpr int kRowsPerPass = kThreads / kPieces;
  constexpr int kLdRows = kTile / kRowsPerPass;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row16 = lane & 15;
  const int kg = lane >> 4;
  // load role: tile rows ld_row + kRowsPerPass i, 16-byte piece ld_piece
  // (its LDS slot in a row, rotated by the row; an E4M3 piece fills the two
  // bf16 slots 2 ld_piece and 2 ld_piece + 1)
  const int ld_row = tid / kPieces;
  const int ld_piece = tid % kPieces;
  const int ld_slot = ld_piece ^ (ld_row & 15);
  const int ld_slot2 = (2 * ld_piece) ^ (ld_row & 15);
  const int ld_slot2b = (2 * ld_piece + 1) ^ (ld_row & 15);

  const int32_t* hdr = ws + PKD_HEADER_BASE;
  const int32_t* slot_indptr = ws + plan_off_slots();
  const int off_indices = hdr[PKD_H_OFF_INDICES];
  const int off_groups = hdr[PKD_H_OFF_GROUPS];
  const int rows_per_block = hdr[PKD_H_ROWS_PER_BLOCK];
  const int partials = hdr[PKD_H_PARTIALS];
  const int32_t* items = ws + hdr[PKD_H_OFF_ITEMS];
  const int32_t* kv_idx = ws + off_indices;
  const int32_t* groups = ws + off_groups;
  const int Hq = num_qo_heads;

  const uint32_t row_bytes = uint32_t(num_kv_heads) * kHeadDim * kElem;
  const uint64_t v_bytes = uint64_t(P) * row_bytes;
  const uint64_t page_bytes = 2 * v_bytes;
  const char* kv = reinterpret_cast<const char*>(kv_ptr);
  int bad = 0;

  // The slot's bounds and its first item sit at offsets fixed by the slot
  // count, so they are read together with the header: the first tile loads
  // wait for two round trips (item, then page ids), not four.
  const int32_t* first = ws + plan_off_first(num_slots) + 8 * int64_t(slot);
  const int it_begin = slot_indptr[slot];
  const int it_end = slot_indptr[slot + 1];
  int32_t fi[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) fi[f] = first[f];
  // keep the loads next to the bounds' (not sunk past the empty-slot test)
  asm volatile("" ::"s"(fi[0]), "s"(fi[1]), "s"(fi[2]), "s"(fi[3]), "s"(fi[4]), "s"(fi[5]),
               "s"(fi[6]), "s"(fi[7]), "s"(off_indices), "s"(off_groups), "s"(rows_per_block),
               "s"(partials));
  float* o_part = fws;
  float* lse_part = fws + int64_t(partials) * Hq * kHeadDim;
  for (int it = it_begin; it < it_end; ++it) {
    int32_t itm[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) itm[f] = it == it_begin ? fi[f] : items[8 * it + f];
    const int grp = itm[0];
    const int32_t* idx = kv_idx + itm[1];
    const int out = itm[4];
    const int len = itm[5];
    const int block = itm[6];
    const int kh = itm[7];
    const int ntiles = (len + kTile - 1) / kTile;
    const int last_valid = len - kTile * (ntiles - 1);
    const int last_token = len - 1;
    floatx4_t acc[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) acc[cb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // This lane's token of row ld_row + 32 i of tile t (clamped to the
    // chunk: rows past its end repeat the last token; they are masked, and V
    // of those rows is zeroed when staged) and the page id of that token.
    auto token_of = [&](int t, int i) {
      return min(kTile * t + kRowsPerPass * i + ld_row, last_token);
    };
    // (threadIdx.y is 0 in this one-dimensional launch; adding it makes the
    // page-id load a per-lane one, so its wait sits where the id is used)
    auto page_of = [&](int t, int i) -> int32_t {
      return idx[token_of(t, i) / P + int(threadIdx.y)];
    };
    auto piece_addr = [&](int t, int i, int32_t id) -> const uint4* {
      const int64_t pg = safe_page(id, num_pages, bad);
      const uint64_t off = uint64_t(pg) * page_bytes + uint64_t(token_of(t, i) % P) * row_bytes +
                           uint64_t(kh) * kHeadDim * kElem + uint64_t(ld_piece) * 16;
      return reinterpret_cast<const uint4*>(kv + off);
    };

    // Ring of kDepth tiles in registers (K and V pieces of kLdRows rows per
    // lane) and the page ids of the tiles each slot loads next.  Loads are
    // issued unconditionally and in the same order in the prologue and the
    // loop (tile, then its page ids), so every wait is for one specific
    // older load.
    uint4 rk[kDepth][kLdRows], rv[kDepth][kLdRows];
    int32_t pid[kDepth][kLdRows];
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
#pragma unroll
      for (int i = 0; i < kLdRows; ++i) pid[d][i] = page_of(min(d, ntiles - 1), i);
    // the group's rows are needed only for q, which is loaded after the
    // first tile
    const int row0 = groups[4 * grp + 0];
    const int rows = groups[4 * grp + 1];
    const int kchunks = groups[4 * grp + 2];
    // this wave's requests: first row (group-relative) and count
    const int wrow = block * rows_per_block + wave * kReqPerWave;
    int nreq = 0;
    bool compute = false;
    // q as the B operand: lane l holds query row l & 15 (request (l & 15) / g,
    // head kh g + (l & 15) % g), head_dim elements 32 j + 8 kg .. + 8
    uint4 qv[4];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
#pragma unroll
      for (int i = 0; i < kLdRows; ++i) {
        const uint4* a = piece_addr(min(d, ntiles - 1), i, pid[d][i]);
        rk[d][i] = load_stream16(a);
        rv[d][i] = load_stream16(reinterpret_cast<const char*>(a) + v_bytes);
      }
#pragma unroll
      for (int i = 0; i < kLdRows; ++i) pid[d][i] = page_of(min(d + kDepth, ntiles - 1), i);
      __builtin_amdgcn_sched_barrier(0);
      if (d == 0) {
        nreq = min(kReqPerWave, rows - wrow);  // <= 0: the wave only loads
        compute = nreq > 0;
        const int i = row16 / G;
        const bool have = compute && i < nreq;
        const uint16_t* qrow = q_ptr +
                               ((int64_t(row0) + wrow + (have ? i : 0)) * Hq + kh * G + row16 % G) *
                                   kHeadDim +
                               kg * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          qv[j] =
              have ? *reinterpret_cast<const uint4*>(qrow + 32 * j) : make_uint4(0u, 0u, 0u, 0u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    float m = kNegInf, lsum = 0.f;
    auto step = [&](uint4 (&sk)[kLdRows], uint4 (&sv)[kLdRows], int32_t (&next_page)[kLdRows],
                    int n, bool reload) {
      const int stage = n & 1;
      const bool last = n == ntiles - 1;
      const int valid = last ? last_valid : kTile;
      // stage tile n; V rows past the valid ones are zero (a zero probability
      // must not meet a repeated or NaN value)
#pragma unroll
      for (int i = 0; i < kLdRows; ++i) {
        const int r = kRowsPerPass * i + ld_row;
        if constexpr (kFp8) {
          const uint4 kc = sk[i];
          const uint4 vc = r < valid ? sv[i] : make_uint4(0u, 0u, 0u, 0u);
          sh.t.k[stage][r][ld_slot2] = fp8x8_to_bf16(kc.x, kc.y);
          sh.t.k[stage][r][ld_slot2b] = fp8x8_to_bf16(kc.z, kc.w);
          sh.t.v[stage][r][ld_slot2] = fp8x8_to_bf16(vc.x, vc.y);
          sh.t.v[stage][r][ld_slot2b] = fp8x8_to_bf16(vc.z, vc.w);
        } else {
          sh.t.k[stage][r][ld_slot] = sk[i];
          sh.t.v[stage][r][ld_slot] = r < valid ? sv[i] : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      lds_barrier();
      if (reload) {
#pragma unroll
        for (int i = 0; i < kLdRows; ++i) {
          const uint4* a = piece_addr(min(n + kDepth, ntiles - 1), i, next_page[i]);
          sk[i] = load_stream16(a);
          sv[i] = load_stream16(reinterpret_cast<const char*>(a) + v_bytes);
        }
#pragma unroll
        for (int i = 0; i < kLdRows; ++i)
          next_page[i] = page_of(min(n + 2 * kDepth, ntiles - 1), i);
      }
      if (!compute) return;

      // S^T = K Q^T per quarter h: lane l gets query row l & 15, tokens
      // 16 h + 4 kg + v
      floatx4_t sq[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) sq[h] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < 4; ++h)
          sq[h] = mfma32(sh.t.k[stage][16 * h + row16][(4 * j + kg) ^ row16], qv[j], sq[h]);
      float sc[16];
      float mx = kNegInf;
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          sc[4 * h + v] = (16 * h + 4 * kg + v < valid) ? sq[h][v] * scale_log2 : kNegInf;
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[v]);
      const float mn = fmaxf(m, rows_max(mx));
      const float alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 while m = -inf
      float p[16];
      float ps = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        p[v] = __builtin_amdgcn_exp2f(sc[v] - mn);
        ps += p[v];
      }
      lsum = fmaf(lsum, alpha, ps);
      m = mn;
      // P^T as the B operand of the product over quarters 2 e and 2 e + 1:
      // k = 8 kg + j <-> token 4 kg + j (j < 4) of the first quarter and
      // 16 + 4 kg + j - 4 of the second
      uint4 pb[2];
      [[maybe_unused]] uint4 pr[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float* pe = p + 8 * e;
        const uint4 h = make_uint4(pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3]),
                                   pack_bf16x2(pe[4], pe[5]), pack_bf16x2(pe[6], pe[7]));
        pb[e] = h;
        if constexpr (kFp8) {
          // what the bf16 high parts leave over (exact in fp32), in bf16
          pr[e] = make_uint4(pack_bf16x2(pe[0] - bf16_lo(h.x), pe[1] - bf16_hi(h.x)),
                             pack_bf16x2(pe[2] - bf16_lo(h.y), pe[3] - bf16_hi(h.y)),
                             pack_bf16x2(pe[4] - bf16_lo(h.z), pe[5] - bf16_hi(h.z)),
                             pack_bf16x2(pe[6] - bf16_lo(h.w), pe[7] - bf16_hi(h.w)));
        }
      }
      // V^T as the A operand of head-dim block cb: lane (kg, i = 4 r + q)
      // points the transposing read at row 4 kg + r of each quarter,
      // elements cb 16 + 4 q .. + 3
      const int tr_row = 4 * kg + (row16 >> 2);
      const int tr_q = row16 & 3;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const int piece = 2 * cb + (tr_q >> 1);
        uint2 b[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
          b[h] = lds_read_tr(
              reinterpret_cast<const char*>(&sh.t.v[stage][16 * h + tr_row][piece ^ tr_row]) +
              8 * (tr_q & 1));
        acc[cb] *= alpha;
        const uint4 va = make_uint4(b[0].x, b[0].y, b[1].x, b[1].y);
        const uint4 vb = make_uint4(b[2].x, b[2].y, b[3].x, b[3].y);
        acc[cb] = mfma32(va, pb[0], acc[cb]);
        acc[cb] = mfma32(vb, pb[1], acc[cb]);
        if constexpr (kFp8) {
          acc[cb] = mfma32(va, pr[0], acc[cb]);
          acc[cb] = mfma32(vb, pr[1], acc[cb]);
        }
      }
    };

    // Whole rounds of kDepth tiles always reload (past the end, the last
    // tile again), so every round leaves the same loads in flight; the
    // partial round after them does not reload.
    const int full = ntiles / kDepth;
    for (int r = 0; r < full; ++r) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) step(rk[d], rv[d], pid[d], r * kDepth + d, true);
    }
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (full * kDepth + d < ntiles) step(rk[d], rv[d], pid[d], full * kDepth + d, false);

    // a chunk's state goes out as fp32 rows staged through LDS: wait until
    // every wave is done with the last tile's K and V there (out is the
    // same for all waves of the item)
    if (out >= 0) lds_barrier();
    if (compute) {
      // lane l: query row l & 15, head dims 16 cb + 4 kg + v
      const float lt = rows_sum(lsum);
      const int i = row16 / G;
      const float inv = out_scale / lt;
      if (out >= 0) {
        char* epi = sh.epi + wave * kEpiWaveBytes;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
          *reinterpret_cast<float4*>(epi + row16 * kEpiRowBytes + 64 * cb + 16 * kg) =
              make_float4(acc[cb][0] * inv, acc[cb][1] * inv, acc[cb][2] * inv,
                          acc[cb][3] * inv);
        // one wave's LDS accesses complete in order: its reads below see
        // every lane's writes
        __builtin_amdgcn_wave_barrier();
        // store s: rows 2 s and 2 s + 1, 16 bytes of a row per lane
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const int r = 2 * st + (lane >> 5);
          const float4 v = *reinterpret_cast<const float4*>(epi + r * kEpiRowBytes +
                                                             16 * (lane & 31));
          const int ri = r / G;
          if (ri < nreq) {
            const int64_t pid_out = int64_t(out) + int64_t(wrow + ri) * kchunks;
            const int64_t qh_r = int64_t(kh) * G + r % G;
            *reinterpret_cast<float4*>(o_part + (pid_out * Hq + qh_r) * kHeadDim +
                                       4 * (lane & 31)) = v;
          }
        }
      }
      if (i < nreq) {
        const int req_in_group = wrow + i;
        const int64_t qh = int64_t(kh) * G + row16 % G;
        const float lse_nat = (m + __log2f(lt)) * kLn2;
        if (out < 0) {
          uint16_t* orow =
              o_ptr + ((int64_t(row0) + req_in_group) * Hq + qh) * kHeadDim + 4 * kg;
#pragma unroll
          for (int cb = 0; cb < 8; ++cb)
            *reinterpret_cast<uint2*>(orow + 16 * cb) =
                make_uint2(pack_bf16x2(acc[cb][0] * inv, acc[cb][1] * inv),
                           pack_bf16x2(acc[cb][2] * inv, acc[cb][3] * inv));
          if (lse_ptr && kg == 0) lse_ptr[(int64_t(row0) + req_in_group) * Hq + qh] = lse_nat;
        } else {
          const int64_t pid_out = int64_t(out) + int64_t(req_in_group) * kchunks;
          if (kg == 0) lse_part[pid_out * Hq + qh] = lse_nat;
        }
      }
    }
    // the next item's first tile reuses LDS stage 0
    lds_barrier();
  }
  report_bad_pages(bad, lane, err, PKD_DEVERR_PAGE_ID);
}

}  // namespace
}  // namespace prefix
}  // namespace pkd
