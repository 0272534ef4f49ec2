// Kernel parameter blocks and launchers shared by the C ABI (api.cpp) and
// the HIP kernels (decode.hip, merge.hip).  Internal to the library.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace pkd {

constexpr int kHeadDim = 128;
constexpr int kMaxWavesPerBlock = 8;

struct DecodeParams {
  const uint16_t* q;   // bf16 [B, Hq, 128]
  const uint16_t* kv;  // [num_pages, 2, P, Hkv, 128]: bf16, or E4M3 codes (fp8 kernel)
  uint16_t* o;         // bf16 [B, Hq, 128]
  float* lse;          // fp32 [B, Hq] or null
  const int32_t* ws;   // int workspace (plan image + kv_indices copy)
  float* fws;          // float workspace (partial states)
  int32_t* err;        // device error word
  int64_t num_pages;
  float scale_log2;    // sm_scale * log2(e) (times k_scale for an E4M3 cache)
  float out_scale;     // E4M3 cache: v_scale, applied to o; unused by the bf16 kernels
  int32_t num_qo_heads;
  int32_t num_kv_heads;
};

struct MergeParams {
  // task t = (row r = t / H, head h = t % H); state c of a task:
  //   o at  o_in + (row_base(r) + c) * o_stride_c + h * 128   (fp32 or bf16)
  //   lse at lse_in + (row_base(r) + c) * lse_stride_c + h
  const void* o_in;
  const float* lse_in;
  int64_t o_stride_c;
  int64_t lse_stride_c;
  const int32_t* ws;   // plan image (partials mode) or null (uniform mode)
  int32_t rows;        // uniform mode: number of rows
  int32_t k;           // uniform mode: states per row
  int32_t H;
  uint16_t* o_out;     // bf16 [.., H, 128]
  float* lse_out;      // fp32 [.., H] or null
  // partials mode: the plan's slot count (which fixes the merge list's
  // offset) and how many merge-list entries the int workspace can hold
  int32_t num_slots;
  int32_t merge_cap;
};

// Decode kernel for group size g and page size P (both must be built):
// q.k with packed bf16 dot products on the vector ALUs (decode.hip) ...
hipError_t launch_decode(const DecodeParams& p, int g, int page_size, int num_slots,
                         hipStream_t stream);
// ... or with the logit tile on the matrix cores (decode_mfma.hip).
hipError_t launch_decode_mfma(const DecodeParams& p, int g, int page_size, int num_slots,
                              hipStream_t stream);
bool decode_variant_built(int g, int page_size);
// ... or with both products on the matrix cores (decode_pv.hip).
hipError_t launch_decode_pv(const DecodeParams& p, int g, int page_size, int num_slots,
                            hipStream_t stream);
bool pv_variant_built(int g, int page_size);
// Decode over an E4M3 cache (decode_fp8.hip): both products on the matrix
// cores, V transposed through LDS.
hipError_t launch_decode_fp8(const DecodeParams& p, int g, int page_size, int num_slots,
                             hipStream_t stream);
bool fp8_variant_built(int g, int page_size);
// Shared-prefix kernel (prefix_mfma.hip): one KV head of one (group, row
// block, chunk) item per workgroup, 128 query rows sharing each K/V tile;
// fp8: the cache holds E4M3 codes (p.out_scale = v_scale).
hipError_t launch_prefix_mfma(const DecodeParams& p, int g, int page_size, int num_slots,
                              bool fp8, hipStream_t stream);
bool prefix_variant_built(int g, int page_size);
// The shared-prefix kernel on a prefix plan (workgroups [0, prefix_slots))
// and the matrix-core P.V decode kernel on a suffix plan (the next
// suffix_slots workgroups) in one launch (composable.hip); page sizes 16,
// 32, 64.  fp8: an E4M3 cache, the suffix on the FP8 decode kernel's code
// (pre.out_scale = v_scale).
hipError_t launch_composable(const DecodeParams& pre, const DecodeParams& suf, int g,
                             int page_size, int prefix_slots, int suffix_slots, bool fp8,
                             hipStream_t stream);
// Occupancy (workgroups per CU) of the matrix-core decode kernel at g=4,
// P=16 (the default kernel), and of the dot-product kernel.
int decode_blocks_per_cu(int waves_per_block);
int decode_blocks_per_cu_dot2(int waves_per_block);

// Copy `image_ints` ints (a multiple of 4, 16-byte aligned ends) of a plan
// image from pinned host memory (device-visible pointer) to the workspace,
// and `nnz` page ids from `indices` to `dst_indices`, in one kernel.  Words
// 6 and 7 of each 8-int item row -- `first_rows` of them from image int
// `first_off` on and `item_rows` from `items_off` on (both multiples of 8) --
// receive the page ids of that item's first two pages (its first twice for a
// one-page item; a row with no pages is left as it is).
hipError_t launch_plan_upload(const int32_t* image, int32_t* dst, int64_t image_ints,
                              const int32_t* indices, int32_t* dst_indices, int64_t nnz,
                              int64_t first_off, int64_t first_rows, int64_t items_off,
                              int64_t item_rows, hipStream_t stream);

// New tokens' requests and positions, and their K/V rows into the paged
// cache (append.hip).
hipError_t launch_append_positions(const int32_t* append_indptr, const int32_t* kv_indptr,
                                   const int32_t* kv_last_page_len, int batch, int page_size,
                                   int32_t* batch_indices, int32_t* positions,
                                   hipStream_t stream);
hipError_t launch_append_kv(const void* k_new, const void* v_new, const int32_t* batch_indices,
                            const int32_t* positions, int64_t nnz, const int32_t* kv_indptr,
                            const int32_t* kv_indices, int batch, int num_kv_heads,
                            int page_size, void* cache, int64_t num_pages, int32_t* err,
                            int grid_cap, hipStream_t stream);
// The same into an E4M3 cache: code = e4m3(x * inv_scale), saturated.
hipError_t launch_append_kv_fp8(const void* k_new, const void* v_new,
                                const int32_t* batch_indices, const int32_t* positions,
                                int64_t nnz, const int32_t* kv_indptr, const int32_t* kv_indices,
                                int batch, int num_kv_heads, int page_size, void* cache,
                                int64_t num_pages, float k_inv_scale, float v_inv_scale,
                                int32_t* err, int grid_cap, hipStream_t stream);

// Merge of the split requests of the current plan (reads the plan image).
hipError_t launch_merge_partials(const MergeParams& p, int grid, hipStream_t stream);
// Merge of two all-partials plans' states per request (plan A's first):
// the composable format's one merge (merge.hip).
// (slots_x: plan x's slot count; cap_x: merge-list entries its int
// workspace can hold)
hipError_t launch_merge_composable(const int32_t* ws_a, const float* fws_a, int slots_a, int cap_a,
                                   const int32_t* ws_b, const float* fws_b, int slots_b, int cap_b,
                                   int H, uint16_t* o_out, float* lse_out, int grid,
                                   hipStream_t stream);
// Merge of `k` bf16 states per row, rows laid out uniformly.
hipError_t launch_merge_states_bf16(const MergeParams& p, hipStream_t stream);
// Row-wise merge of two bf16 states.
hipError_t launch_merge_two_bf16(const uint16_t* o_a, const float* lse_a, const uint16_t* o_b,
                                 const float* lse_b, int64_t rows, uint16_t* o_out,
                                 float* lse_out, hipStream_t stream);

// The library's device scratch array (static_scratch.hip): its address on
// `device` is taken once, with that device current; until then, and after a
// failure, static_scratch_ptr returns null.
hipError_t static_scratch_init(int device);
void* static_scratch_ptr(int device);
// The handle whose plan the array on `device` holds (set by pkd_plan_static).
void static_scratch_claim(int device, const void* owner);
void static_scratch_release(int device, const void* owner);  // if `owner` holds it
const void* static_scratch_owner(int device);

// Read-ceiling kernels (read_ceiling.hip): `grid` workgroups of
// read_ceiling_threads() lanes, one 32-bit XOR per lane into `sink`.
int read_ceiling_threads();
hipError_t launch_read_stream(const void* buf, int64_t n16, uint32_t* sink, int grid,
                              hipStream_t stream);
hipError_t launch_read_pages(const void* base, const int32_t* ids, int64_t n_ids,
                             int64_t num_pages, int64_t page_bytes, uint32_t* sink, int grid,
                             hipStream_t stream);

}  // namespace pkd
