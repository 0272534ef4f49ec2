// Appending new tokens to the paged KV cache, for gfx950.
//
// The pyshine FlashInfer tour, section "The Paged KV Cache Layer": after
// every generated token the engine copies the new K and V rows into their
// page slots, given the page table that already covers them, and a helper
// derives each new token's request and sequence position from the page
// indirection.  Token t of a request lives in page indices[indptr[i] + t / P],
// slot t % P (aicassindra "FlashInfer, in depth", section "The block-sparse
// page table"), so a run of new tokens that crosses into a fresh page just
// continues on the next page of the request's list.
//
// append_positions_kernel: one workgroup per request writes the request and
// the position L_i - a_i + j of its j-th new token (L_i its length after the
// append, a_i its new-token count).
// append_kv_kernel: one workgroup per new token (grid-stride), 16-byte pieces:
// the K row and the V row of the token (num_kv_heads x 128 bf16 each) go to
// the same slot of the K and V halves of their page.  Indices outside the
// request, its pages or the cache are not written; they set a flag.
// append_kv_fp8_kernel: the same into an FP8 E4M3 cache, quantising on the
// way (the pyshine page fuses quantisation with the append): each thread
// turns 16 bf16 values into 16 codes e4m3(x * (1 / scale)), the product in
// fp32, rounded to nearest even and saturated to +-448 (the hardware
// conversion does not saturate, so values are clamped first; NaN stays NaN).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"
#include "pkd.h"

namespace pkd {
namespace {

constexpr int kAppendThreads = 256;

__global__ __launch_bounds__(kAppendThreads) void append_positions_kernel(
    const int32_t* __restrict__ append_indptr, const int32_t* __restrict__ kv_indptr,
    const int32_t* __restrict__ kv_last_page_len, int page_size,
    int32_t* __restrict__ batch_indices, int32_t* __restrict__ positions) {
  const int i = blockIdx.x;
  const int64_t a0 = append_indptr[i];
  const int a = append_indptr[i + 1] - append_indptr[i];
  const int64_t length =
      int64_t(page_size) * (kv_indptr[i + 1] - kv_indptr[i] - 1) + kv_last_page_len[i];
  for (int j = threadIdx.x; j < a; j += kAppendThreads) {
    batch_indices[a0 + j] = i;
    positions[a0 + j] = int32_t(length - a + j);
  }
}

__global__ __launch_bounds__(kAppendThreads) void append_kv_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int32_t* __restrict__ batch_indices, const int32_t* __restrict__ positions,
    int64_t nnz, const int32_t* __restrict__ kv_indptr, const int32_t* __restrict__ kv_indices,
    int batch, int row_pieces, int page_size, char* __restrict__ cache, int64_t num_pages,
    int32_t* __restrict__ err) {
  const uint64_t row_bytes = uint64_t(row_pieces) * 16;
  const uint64_t v_bytes = uint64_t(page_size) * row_bytes;
  int bad = 0;
  for (int64_t t = blockIdx.x; t < nnz; t += gridDim.x) {
    const int b = batch_indices[t];
    const int pos = positions[t];
    bool ok = b >= 0 && b < batch && pos >= 0;
    int64_t page = 0;
    if (ok) {
      const int first = kv_indptr[b];
      const int n = kv_indptr[b + 1] - first;
      ok = pos / page_size < n;
      if (ok) {
        page = kv_indices[first + pos / page_size];
        ok = page >= 0 && page < num_pages;
      }
    }
    if (!ok) {
      bad = 1;
      continue;
    }
    char* slot = cache + uint64_t(page) * 2 * v_bytes + uint64_t(pos % page_size) * row_bytes;
    const uint4* ks = k_new + t * row_pieces;
    const uint4* vs = v_new + t * row_pieces;
    for (int p = threadIdx.x; p < 2 * row_pieces; p += kAppendThreads) {
      const bool is_v = p >= row_pieces;
      const int q = is_v ? p - row_pieces : p;
      reinterpret_cast<uint4*>(slot + (is_v ? v_bytes : 0))[q] = load_stream16(is_v ? vs + q : ks + q);
    }
  }
  if (bad && err && threadIdx.x == 0) err[0] = PKD_DEVERR_PAGE_ID;
}

__device__ __forceinline__ float sat_e4m3(float x) {
  return x != x ? __builtin_nanf("") : fminf(fmaxf(x, -448.f), 448.f);
}

// Codes of two bf16 pairs (a dword each) times inv, as 4 bytes.  The
// hardware writes NaN as 0xFF; NaN codes are given as 0x7F (sign cleared):
// after saturation a byte whose low 7 bits are all ones can only be NaN, and
// adding 1 to the low 7 bits of each byte carries into bit 7 exactly there.
__device__ __forceinline__ uint32_t e4m3x4(uint32_t w0, uint32_t w1, float inv) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(bf16_lo(w0) * inv),
                                          sat_e4m3(bf16_hi(w0) * inv), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(bf16_lo(w1) * inv), sat_e4m3(bf16_hi(w1) * inv),
                                      r, true);
  const uint32_t u = uint32_t(r);
  const uint32_t nan_sign = ((u & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
  return u & ~nan_sign;
}

__global__ __launch_bounds__(kAppendThreads) void append_kv_fp8_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int32_t* __restrict__ batch_indices, const int32_t* __restrict__ positions,
    int64_t nnz, const int32_t* __restrict__ kv_indptr, const int32_t* __restrict__ kv_indices,
    int batch, int row_pieces, int page_size, char* __restrict__ cache, int64_t num_pages,
    float k_inv, float v_inv, int32_t* __restrict__ err) {
  // row_pieces: 16-byte pieces of one token's codes (num_kv_heads x 128 bytes);
  // the bf16 input row is twice as long
  const uint64_t row_bytes = uint64_t(row_pieces) * 16;
  const uint64_t v_bytes = uint64_t(page_size) * row_bytes;
  int bad = 0;
  for (int64_t t = blockIdx.x; t < nnz; t += gridDim.x) {
    const int b = batch_indices[t];
    const int pos = positions[t];
    bool ok = b >= 0 && b < batch && pos >= 0;
    int64_t page = 0;
    if (ok) {
      const int first = kv_indptr[b];
      const int n = kv_indptr[b + 1] - first;
      ok = pos / page_size < n;
      if (ok) {
        page = kv_indices[first + pos / page_size];
        ok = page >= 0 && page < num_pages;
      }
    }
    if (!ok) {
      bad = 1;
      continue;
    }
    char* slot = cache + uint64_t(page) * 2 * v_bytes + uint64_t(pos % page_size) * row_bytes;
    const uint4* ks = k_new + t * 2 * row_pieces;
    const uint4* vs = v_new + t * 2 * row_pieces;
    for (int p = threadIdx.x; p < 2 * row_pieces; p += kAppendThreads) {
      const bool is_v = p >= row_pieces;
      const int q = is_v ? p - row_pieces : p;
      const uint4* src = (is_v ? vs : ks) + 2 * q;
      const float inv = is_v ? v_inv : k_inv;
      const uint4 a = load_stream16(src);
      const uint4 c = load_stream16(src + 1);
      reinterpret_cast<uint4*>(slot + (is_v ? v_bytes : 0))[q] =
          make_uint4(e4m3x4(a.x, a.y, inv), e4m3x4(a.z, a.w, inv), e4m3x4(c.x, c.y, inv),
                     e4m3x4(c.z, c.w, inv));
    }
  }
  if (bad && err && threadIdx.x == 0) err[0] = PKD_DEVERR_PAGE_ID;
}

}  // namespace

hipError_t launch_append_positions(const int32_t* append_indptr, const int32_t* kv_indptr,
                                   const int32_t* kv_last_page_len, int batch, int page_size,
                                   int32_t* batch_indices, int32_t* positions,
                                   hipStream_t stream) {
  if (batch < 1) return hipSuccess;
  hipLaunchKernelGGL(append_positions_kernel, dim3(batch), dim3(kAppendThreads), 0, stream,
                     append_indptr, kv_indptr, kv_last_page_len, page_size, batch_indices,
                     positions);
  return hipGetLastError();
}

hipError_t launch_append_kv(const void* k_new, const void* v_new, const int32_t* batch_indices,
                            const int32_t* positions, int64_t nnz, const int32_t* kv_indptr,
                            const int32_t* kv_indices, int batch, int num_kv_heads,
                            int page_size, void* cache, int64_t num_pages, int32_t* err,
                            int grid_cap, hipStream_t stream) {
  if (nnz < 1) return hipSuccess;
  const int64_t grid = nnz < grid_cap ? nnz : grid_cap;
  hipLaunchKernelGGL(append_kv_kernel, dim3(unsigned(grid)), dim3(kAppendThreads), 0, stream,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     batch_indices, positions, nnz, kv_indptr, kv_indices, batch,
                     num_kv_heads * kHeadDim * 2 / 16, page_size, static_cast<char*>(cache),
                     num_pages, err);
  return hipGetLastError();
}

hipError_t launch_append_kv_fp8(const void* k_new, const void* v_new,
                                const int32_t* batch_indices, const int32_t* positions,
                                int64_t nnz, const int32_t* kv_indptr, const int32_t* kv_indices,
                                int batch, int num_kv_heads, int page_size, void* cache,
                                int64_t num_pages, float k_inv_scale, float v_inv_scale,
                                int32_t* err, int grid_cap, hipStream_t stream) {
  if (nnz < 1) return hipSuccess;
  const int64_t grid = nnz < grid_cap ? nnz : grid_cap;
  hipLaunchKernelGGL(append_kv_fp8_kernel, dim3(unsigned(grid)), dim3(kAppendThreads), 0, stream,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     batch_indices, positions, nnz, kv_indptr, kv_indices, batch,
                     num_kv_heads * kHeadDim / 16, page_size, static_cast<char*>(cache),
                     num_pages, k_inv_scale, v_inv_scale, err);
  return hipGetLastError();
}

}  // namespace pkd
