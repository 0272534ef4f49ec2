// C ABI of the paged GQA decode library (declared in include/pkd.h).
//
// pkd_plan (and pkd_plan_shared) run the host scheduler into a pinned
// staging buffer and queue one kernel that uploads it, with the kv_indices
// snapshot, into the caller's int workspace (pinghaoyang FlashInfer page,
// "固定指针比固定内容更重要": the plan is built in page-locked host memory and
// copied asynchronously into a workspace at fixed offsets, so the run sees
// the same addresses with new contents).  pkd_run launches the decode (or
// shared-prefix) kernel on the handle's S slots and the merge kernel on a
// fixed grid; neither launch depends on the plan's contents, only on its
// kind and head configuration, so a captured run stays valid across plans of
// the same kind and configuration on the same workspaces.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <exception>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "pkd.h"
#include "plan.h"
#include "plan_layout.h"

struct pkd_handle {
  int device = 0;
  int num_slots = 0;
  int cu_count = 0;
  int merge_grid = 0;
  int waves_per_block = 0;
  int64_t plan_counter = 0;

  // current plan
  bool planned = false;
  int32_t batch = 0, Hq = 0, Hkv = 0, D = 0, P = 0, q_dtype = 0, kv_dtype = 0;
  int32_t variant = PKD_VARIANT_MFMA;
  pkd::PlanLayout layout;
  void* int_ws = nullptr;
  size_t int_bytes = 0;
  void* float_ws = nullptr;
  size_t float_bytes = 0;
  void* host_ws = nullptr;
  void* host_view_for = nullptr;  // host workspace whose device view is host_view
  int32_t* host_view = nullptr;   // device-visible address of the host workspace
  size_t host_bytes = 0;
  void* err_cleared_for = nullptr;

  // staging halves
  int staging_next = 0;
  hipEvent_t staging_done[2] = {nullptr, nullptr};
  bool staging_pending[2] = {false, false};

  pkd::PlanScratch scratch;

  // pkd_plan_static: the two host halves the plan image is built in before it
  // is copied to the static array's staging region (allocated on the first
  // static plan, then reused)
  std::vector<int32_t> static_host;
  bool static_plan = false;  // the current plan lives in the static array
  int32_t plan_flags = 0;    // PKD_PLAN_* flags of the current plan


  // profiling
  bool profile = false;
  std::vector<hipEvent_t> prof_events;  // 3 per run: start, after decode, after merge
  size_t prof_used = 0;
};

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PKD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Sets the handle's device for the duration of a call.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) {
      err = hipSetDevice(dev);
      ok = err == hipSuccess;
    }
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

size_t ints_to_bytes(int64_t n) { return size_t(n) * sizeof(int32_t); }

// Merge-list entries the current plan's int workspace holds from the list's
// fixed offset on: a merge workgroup may request its first entry before it
// knows the list's length, and stays inside the workspace this way.
int32_t merge_cap(const pkd_handle* h) {
  const int64_t ints = int64_t(h->int_bytes / sizeof(int32_t));
  const int64_t cap = (ints - pkd::plan_off_merge(h->num_slots)) / 4;
  return int32_t(std::max<int64_t>(0, std::min<int64_t>(cap, INT32_MAX)));
}

constexpr int64_t kStagingAlignInts = 64;  // 256-byte aligned halves

int64_t staging_half_ints(int64_t max_batch, int64_t num_slots) {
  const int64_t I = pkd::max_items(max_batch, num_slots);
  const int64_t ints = pkd::plan_image_ints(num_slots, I, max_batch);
  return (ints + kStagingAlignInts - 1) / kStagingAlignInts * kStagingAlignInts;
}

pkd::PlanInput make_input(const int32_t* indptr, const int32_t* last, int32_t batch, int32_t Hq,
                          int32_t Hkv, int32_t D, int32_t P, int32_t S,
                          const pkd_plan_opts* opts) {
  pkd::PlanInput in;
  in.indptr = indptr;
  in.last = last;
  in.batch = batch;
  in.num_qo_heads = Hq;
  in.num_kv_heads = Hkv;
  in.head_dim = D;
  in.page_size = P;
  in.num_slots = S;
  if (opts) {
    in.fixed_chunk_pages = opts->fixed_chunk_pages;
    in.min_chunk_tokens = opts->min_chunk_tokens;
    in.alpha = opts->alpha;
    in.beta = opts->beta;
    in.flags = opts->flags;
  }
  return in;
}

int check_shapes(int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t q_dtype, int32_t kv_dtype,
                 int32_t layout) {
  if (q_dtype != PKD_DTYPE_BF16 || (kv_dtype != PKD_DTYPE_BF16 && kv_dtype != PKD_DTYPE_FP8_E4M3))
    return fail(PKD_ERR_UNSUPPORTED,
                "q must be bf16 and the KV cache bf16 or fp8 e4m3 (PKD_DTYPE_BF16 / _FP8_E4M3)");
  if (layout != PKD_LAYOUT_NHD) return fail(PKD_ERR_UNSUPPORTED, "only the NHD cache layout is built");
  if (D != pkd::kHeadDim) return fail(PKD_ERR_UNSUPPORTED, "only head_dim 128 is built");
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(PKD_ERR_INVALID_ARG, "num_qo_heads must be a positive multiple of num_kv_heads");
  if (kv_dtype == PKD_DTYPE_FP8_E4M3) {
    if (!pkd::fp8_variant_built(Hq / Hkv, P))
      return fail(PKD_ERR_UNSUPPORTED,
                  "an fp8 e4m3 cache is built for group sizes 1 to 8 and page_size 1, 2, 4, 8, 16, "
                  "32 or 64");
    return PKD_OK;
  }
  if (!pkd::decode_variant_built(Hq / Hkv, P) && !pkd::pv_variant_built(Hq / Hkv, P))
    return fail(PKD_ERR_UNSUPPORTED,
                "group size must be 1 to 8 and page_size 1, 2, 4, 8, 16, 32 or 64");
  return PKD_OK;
}

// plan_build without letting an exception (host memory for the work items
// of an enormous plan) cross the C ABI.
int guarded_plan_build(const pkd::PlanInput& in, pkd::PlanScratch& s, int32_t* image,
                       int64_t image_ints, pkd::PlanLayout* layout, std::string* err) {
  try {
    return pkd::plan_build(in, s, image, image_ints, layout, err);
  } catch (const std::exception& e) {
    *err = std::string("planning failed on the host: ") + e.what();
    return PKD_ERR_INVALID_ARG;
  }
}

// Three profiling events for one run of `h` (start, after the decode
// kernel, after the merge) when its profiling is on and `s` is not being
// captured; *ev stays null otherwise.
hipError_t profile_events(pkd_handle* h, hipStream_t s, hipEvent_t** ev) {
  *ev = nullptr;
  if (!h->profile) return hipSuccess;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return hipSuccess;
  if (h->prof_used + 3 > h->prof_events.size()) {
    for (int i = 0; i < 3; ++i) {
      hipEvent_t x;
      // device-scope release only: a system-scope fence per record would
      // stretch the gaps between the timed kernels
      hipError_t e = hipEventCreateWithFlags(&x, hipEventDisableSystemFence);
      if (e != hipSuccess) return e;
      h->prof_events.push_back(x);
    }
  }
  *ev = &h->prof_events[h->prof_used];
  h->prof_used += 3;
  return hipSuccess;
}

int check_shared_shapes(int32_t Hq, int32_t Hkv, int32_t P) {
  if (!pkd::prefix_variant_built(Hq / Hkv, P))
    return fail(PKD_ERR_UNSUPPORTED,
                "shared-prefix plans are built for group size 1, 2, 4 or 8 and page_size 16, 32 or 64");
  return PKD_OK;
}

}  // namespace

// Below this many KV tokens per persistent slot the default bf16 kernel is
// the one with both products on the matrix cores (see pkd_plan).
constexpr int64_t kPvMaxTokensPerSlot = 768;

extern "C" {

const char* pkd_last_error(void) { return g_last_error.c_str(); }

int pkd_create(pkd_handle** out, int32_t device, int32_t num_slots) {
  if (!out) return fail(PKD_ERR_INVALID_ARG, "out must be non-null");
  *out = nullptr;
  if (num_slots < 0) return fail(PKD_ERR_INVALID_ARG, "num_slots must be >= 0");
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device < 0 || device >= count) return fail(PKD_ERR_INVALID_ARG, "no such HIP device");
  DeviceGuard guard(device);
  if (!guard.ok) return hip_fail(guard.err, "hipSetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  pkd_handle* h = new pkd_handle();
  h->device = device;
  h->cu_count = prop.multiProcessorCount;
  h->waves_per_block = pkd::kMaxWavesPerBlock;
  h->num_slots = num_slots > 0 ? num_slots
                               : h->cu_count * pkd::decode_blocks_per_cu(h->waves_per_block);
  if (num_slots == 0 && h->num_slots > 2 * h->cu_count) h->num_slots = 2 * h->cu_count;
  h->merge_grid = 4 * h->cu_count;
  // the address of the library's device scratch on this device (taken once
  // per device; a failure is reported by pkd_plan_static, the only user)
  (void)pkd::static_scratch_init(device);
  for (int i = 0; i < 2; ++i) {
    e = hipEventCreateWithFlags(&h->staging_done[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      pkd_destroy(h);
      return hip_fail(e, "hipEventCreate");
    }
  }
  *out = h;
  return PKD_OK;
}

int pkd_destroy(pkd_handle* h) {
  if (!h) return PKD_OK;
  pkd::static_scratch_release(h->device, h);
  DeviceGuard guard(h->device);
  for (int i = 0; i < 2; ++i) {
    if (h->staging_done[i]) {
      (void)hipEventSynchronize(h->staging_done[i]);
      (void)hipEventDestroy(h->staging_done[i]);
    }
  }
  for (hipEvent_t ev : h->prof_events) (void)hipEventDestroy(ev);
  delete h;
  return PKD_OK;
}

int32_t pkd_num_slots(const pkd_handle* h) { return h ? h->num_slots : 0; }

int32_t pkd_planned_variant(const pkd_handle* h) { return h && h->planned ? h->variant : 0; }

int64_t pkd_plan_id(const pkd_handle* h) { return h && h->planned ? h->plan_counter : 0; }

int pkd_plan_shape(const pkd_handle* h, int32_t* shape) {
  if (!h || !shape) return fail(PKD_ERR_INVALID_ARG, "null argument");
  if (!h->planned) return fail(PKD_ERR_STALE_PLAN, "no plan on this handle");
  const int32_t v[8] = {h->batch, h->Hq, h->Hkv, h->D, h->P, h->q_dtype, h->kv_dtype,
                        h->layout.kind};
  std::memcpy(shape, v, sizeof(v));
  return PKD_OK;
}

size_t pkd_int_workspace_bytes(int32_t max_batch, int32_t max_nnz, int32_t num_slots) {
  if (max_batch < 1 || max_nnz < 1 || num_slots < 1) return 0;
  const int64_t I = pkd::max_items(max_batch, num_slots);
  return ints_to_bytes(pkd::plan_image_ints(num_slots, I, max_batch) + max_nnz);
}

size_t pkd_float_workspace_bytes(int32_t max_batch, int32_t num_slots, int32_t num_qo_heads,
                                 int32_t head_dim) {
  if (max_batch < 1 || num_slots < 1 || num_qo_heads < 1 || head_dim < 1) return 0;
  const int64_t I = pkd::max_items(max_batch, num_slots);
  return size_t(I) * size_t(num_qo_heads) * size_t(head_dim + 1) * sizeof(float);
}

size_t pkd_host_workspace_bytes(int32_t max_batch, int32_t num_slots) {
  if (max_batch < 1 || num_slots < 1) return 0;
  return 2 * ints_to_bytes(staging_half_ints(max_batch, num_slots));
}

int pkd_shared_workspace_bytes(int32_t max_groups, int32_t max_batch, int32_t max_nnz,
                               int32_t num_slots, int32_t num_qo_heads, int32_t num_kv_heads,
                               int32_t head_dim, size_t* int_bytes, size_t* float_bytes,
                               size_t* host_bytes) {
  if (max_groups < 1 || max_batch < max_groups || max_nnz < 1 || num_slots < 1 ||
      num_qo_heads < 1 || num_kv_heads < 1 || num_qo_heads % num_kv_heads != 0 || head_dim < 1)
    return fail(PKD_ERR_INVALID_ARG, "invalid sizes for pkd_shared_workspace_bytes");
  const int64_t I =
      pkd::max_items_shared(max_groups, max_batch, num_slots, num_qo_heads, num_kv_heads);
  int64_t image = pkd::plan_image_ints(num_slots, I, max_batch, max_groups);
  image = (image + kStagingAlignInts - 1) / kStagingAlignInts * kStagingAlignInts;
  const int64_t partials = pkd::max_partials_shared(max_batch, num_slots, num_kv_heads);
  if (int_bytes) *int_bytes = ints_to_bytes(image + max_nnz);
  if (float_bytes)
    *float_bytes = size_t(partials) * size_t(num_qo_heads) * size_t(head_dim + 1) * sizeof(float);
  if (host_bytes) *host_bytes = 2 * ints_to_bytes(image);
  return PKD_OK;
}

int pkd_plan_host(const int32_t* kv_indptr, const int32_t* kv_last_page_len, int32_t batch,
                  int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t page_size, int32_t num_slots, const pkd_plan_opts* opts, int32_t* out,
                  size_t out_bytes, int64_t* out_ints) {
  pkd::PlanInput in = make_input(kv_indptr, kv_last_page_len, batch, num_qo_heads, num_kv_heads,
                                 head_dim, page_size, num_slots, opts);
  pkd::PlanScratch scratch;
  pkd::PlanLayout layout;
  std::string err;
  const int rc = guarded_plan_build(in, scratch, out, int64_t(out_bytes / sizeof(int32_t)),
                                    &layout, &err);
  if (rc != PKD_OK) return fail(rc, err);
  if (out_ints) *out_ints = layout.off_indices;
  return PKD_OK;
}

int pkd_plan_shared_host(const int32_t* qo_indptr, const int32_t* kv_indptr,
                         const int32_t* kv_last_page_len, int32_t num_groups,
                         int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t page_size, int32_t num_slots, const pkd_plan_opts* opts,
                         int32_t* out, size_t out_bytes, int64_t* out_ints) {
  if (!qo_indptr) return fail(PKD_ERR_INVALID_ARG, "qo_indptr must be non-null");
  pkd::PlanInput in = make_input(kv_indptr, kv_last_page_len, num_groups, num_qo_heads,
                                 num_kv_heads, head_dim, page_size, num_slots, opts);
  in.qo_indptr = qo_indptr;
  pkd::PlanScratch scratch;
  pkd::PlanLayout layout;
  std::string err;
  const int rc = guarded_plan_build(in, scratch, out, int64_t(out_bytes / sizeof(int32_t)),
                                    &layout, &err);
  if (rc != PKD_OK) return fail(rc, err);
  if (out_ints) *out_ints = layout.off_indices;
  return PKD_OK;
}

// Both plan kinds: qo_indptr is null for a decode plan, the group table of
// requests for a shared-prefix plan (then `batch` counts groups).
static int plan_impl(pkd_handle* h, const int32_t* qo_indptr, const int32_t* kv_indptr,
                     const int32_t* kv_indices, const int32_t* kv_last_page_len, int32_t batch,
                     int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t page_size, int32_t q_dtype, int32_t kv_dtype, int32_t kv_layout,
                     void* int_workspace, size_t int_workspace_bytes, void* float_workspace,
                     size_t float_workspace_bytes, void* host_workspace,
                     size_t host_workspace_bytes, const pkd_plan_opts* opts,
                     pkd_stream_t stream, bool use_static = false) {
  if (!h) return fail(PKD_ERR_INVALID_ARG, "null handle");
  if (use_static) {
    // the library's device array in place of the int and float workspaces,
    // the handle's host memory in place of the pinned staging
    char* base = static_cast<char*>(pkd::static_scratch_ptr(h->device));
    if (!base) {
      DeviceGuard g(h->device);
      const hipError_t e = g.ok ? pkd::static_scratch_init(h->device) : g.err;
      base = static_cast<char*>(pkd::static_scratch_ptr(h->device));
      if (!base) return hip_fail(e == hipSuccess ? hipErrorInvalidValue : e,
                                 "address of the static scratch array");
    }
    int_workspace = base;
    int_workspace_bytes = PKD_STATIC_INT_BYTES;
    float_workspace = base + PKD_STATIC_INT_BYTES;
    float_workspace_bytes = PKD_STATIC_FLOAT_BYTES;
    if (h->static_host.empty())
      h->static_host.assign(2 * PKD_STATIC_STAGE_BYTES / sizeof(int32_t), 0);
    host_workspace = h->static_host.data();
    host_workspace_bytes = 2 * size_t(PKD_STATIC_STAGE_BYTES);
  }
  int rc = check_shapes(num_qo_heads, num_kv_heads, head_dim, page_size, q_dtype, kv_dtype,
                        kv_layout);
  if (rc != PKD_OK) return rc;
  if (qo_indptr && (rc = check_shared_shapes(num_qo_heads, num_kv_heads, page_size)) != PKD_OK)
    return rc;
  if (!kv_indices || !int_workspace || !float_workspace || !host_workspace)
    return fail(PKD_ERR_INVALID_ARG, "kv_indices and the three workspaces must be non-null");
  if ((reinterpret_cast<uintptr_t>(int_workspace) & 255) ||
      (reinterpret_cast<uintptr_t>(float_workspace) & 255) ||
      (!use_static && (reinterpret_cast<uintptr_t>(host_workspace) & 255)))
    return fail(PKD_ERR_INVALID_ARG, "workspaces must be 256-byte aligned");

  const int32_t variant = opts ? opts->variant : PKD_VARIANT_AUTO;
  if (variant != PKD_VARIANT_AUTO && variant != PKD_VARIANT_DOT2 && variant != PKD_VARIANT_MFMA &&
      variant != PKD_VARIANT_MFMA_PV)
    return fail(PKD_ERR_INVALID_ARG, "unknown decode kernel variant");
  if (variant == PKD_VARIANT_MFMA_PV &&
      (kv_dtype != PKD_DTYPE_BF16 || !pkd::pv_variant_built(num_qo_heads / num_kv_heads, page_size)))
    return fail(PKD_ERR_UNSUPPORTED,
                "the PKD_VARIANT_MFMA_PV kernel is built for a bf16 cache and group sizes 1 to 8");
  if (variant == PKD_VARIANT_DOT2 && kv_dtype == PKD_DTYPE_FP8_E4M3)
    return fail(PKD_ERR_UNSUPPORTED, "an fp8 e4m3 cache has only the matrix-core kernel");
  if ((variant == PKD_VARIANT_DOT2 || variant == PKD_VARIANT_MFMA) &&
      kv_dtype == PKD_DTYPE_BF16 && !pkd::decode_variant_built(num_qo_heads / num_kv_heads, page_size))
    return fail(PKD_ERR_UNSUPPORTED,
                "the PKD_VARIANT_DOT2 and PKD_VARIANT_MFMA kernels are built for group size 1, 2, 4 "
                "or 8");

  DeviceGuard guard(h->device);
  if (!guard.ok) return hip_fail(guard.err, "hipSetDevice");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_static) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
      return fail(PKD_ERR_INVALID_ARG, "pkd_plan_static runs outside graph capture (capture the runs)");
  }

  // Build into the staging half that is not the latest in-flight copy.
  const int half = h->staging_next;
  if (h->staging_pending[half]) {
    hipError_t e = hipEventSynchronize(h->staging_done[half]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    h->staging_pending[half] = false;
  }
  const int64_t half_ints = int64_t(host_workspace_bytes / sizeof(int32_t) / 2) /
                            kStagingAlignInts * kStagingAlignInts;
  int32_t* image = static_cast<int32_t*>(host_workspace) + half * half_ints;

  pkd::PlanInput in = make_input(kv_indptr, kv_last_page_len, batch, num_qo_heads, num_kv_heads,
                                 head_dim, page_size, h->num_slots, opts);
  in.qo_indptr = qo_indptr;
  in.plan_id = h->plan_counter + 1;
  pkd::PlanLayout layout;
  std::string err;
  rc = guarded_plan_build(in, h->scratch, image, half_ints, &layout, &err);
  if (rc == PKD_ERR_WORKSPACE_TOO_SMALL)
    return fail(rc, use_static ? "the plan image exceeds PKD_STATIC_STAGE_BYTES"
                               : "host workspace too small for this plan (size it with "
                                 "pkd_host_workspace_bytes)");
  if (rc != PKD_OK) return fail(rc, err);

  const size_t need_int = ints_to_bytes(layout.off_indices + layout.nnz);
  const size_t need_float =
      size_t(layout.n_partials) * size_t(num_qo_heads) * size_t(head_dim + 1) * sizeof(float);
  if (int_workspace_bytes < need_int)
    return fail(PKD_ERR_WORKSPACE_TOO_SMALL, "int workspace too small for this plan (needs " +
                                                 std::to_string(need_int) + " bytes)");
  if (float_workspace_bytes < need_float)
    return fail(PKD_ERR_WORKSPACE_TOO_SMALL, "float workspace too small for this plan (needs " +
                                                 std::to_string(need_float) + " bytes)");

  hipError_t e;
  if (h->err_cleared_for != int_workspace) {
    // fresh workspace: clear the device-only words (error flag) once
    e = hipMemsetAsync(int_workspace, 0, ints_to_bytes(PKD_HEADER_BASE), s);
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync");
    h->err_cleared_for = int_workspace;
  }
  if (use_static) {
    // the image goes from the handle's (pageable) host half to the staging
    // region at the end of the array; the upload kernel reads it there
  } else if (h->host_view_for != host_workspace) {
    // the GPU reads the staging area directly, so it must be pinned memory
    void* view = nullptr;
    e = hipHostGetDevicePointer(&view, host_workspace, 0);
    if (e != hipSuccess || !view) {
      (void)hipGetLastError();
      return fail(PKD_ERR_INVALID_ARG,
                  "host workspace must be pinned host memory (hipHostMalloc, torch pin_memory)");
    }
    h->host_view = static_cast<int32_t*>(view);
    h->host_view_for = host_workspace;
  }
  int32_t* dev = static_cast<int32_t*>(int_workspace);
  // the item rows of a decode plan (the first-item table and the items) get
  // their items' first two page ids on the device, in words 6 and 7; a
  // shared-prefix plan keeps row block and head there
  const bool decode_rows = layout.kind == PKD_PLAN_DECODE;
  const int64_t first_rows = decode_rows ? int64_t(h->num_slots) : 0;
  const int64_t item_rows = decode_rows ? int64_t(layout.num_items) : 0;
  const int32_t* src = nullptr;
  if (!use_static) {
    src = h->host_view + half * half_ints;
  } else {
    int32_t* stage = reinterpret_cast<int32_t*>(static_cast<char*>(int_workspace) +
                                                PKD_STATIC_INT_BYTES + PKD_STATIC_FLOAT_BYTES);
    e = hipMemcpyAsync(stage + PKD_HEADER_BASE, image + PKD_HEADER_BASE,
                       ints_to_bytes(layout.off_indices - PKD_HEADER_BASE),
                       hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "copy of the plan image to the static scratch");
    src = stage;
  }
  e = pkd::launch_plan_upload(src + PKD_HEADER_BASE,
                              dev + PKD_HEADER_BASE, layout.off_indices - PKD_HEADER_BASE,
                              kv_indices, dev + layout.off_indices, layout.nnz,
                              layout.off_first - PKD_HEADER_BASE, first_rows,
                              layout.off_items - PKD_HEADER_BASE, item_rows, s);
  if (e != hipSuccess) return hip_fail(e, "plan upload kernel");
  e = hipEventRecord(h->staging_done[half], s);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  h->staging_pending[half] = true;
  h->staging_next = half ^ 1;

  h->planned = true;
  h->plan_counter += 1;
  h->static_plan = use_static;
  h->plan_flags = in.flags;
  if (use_static) pkd::static_scratch_claim(h->device, h);
  h->batch = layout.num_requests;
  h->Hq = num_qo_heads;
  h->Hkv = num_kv_heads;
  h->D = head_dim;
  h->P = page_size;
  h->q_dtype = q_dtype;
  h->kv_dtype = kv_dtype;
  // The default kernel, by measurement in the benchmark (caches streamed from
  // HBM, alternating runs on one box): both products on the matrix cores for
  // group size 8 (1.3-1.4x), for pages below 16 tokens (1.0-1.7x over the
  // dot-product kernel) and where each slot has little work (skewed batch,
  // about 520 tokens per slot: 87.8 vs 92.1 us); with about 1,000 tokens per
  // slot and smaller groups the q.k-only matrix-core kernel streams faster
  // (Llama-3-8B-like layer: 156.1 vs 160.8 us).  Group sizes 3, 5, 6 and 7
  // are built for the P.V kernel only.  An FP8 cache has its own kernel.
  if (variant == PKD_VARIANT_AUTO) {
    const int g = num_qo_heads / num_kv_heads;
    const int64_t tokens_per_slot = layout.total_tokens / h->num_slots;
    const bool pv = kv_dtype == PKD_DTYPE_BF16 && pkd::pv_variant_built(g, page_size) &&
                    (g == 8 || page_size < 16 || tokens_per_slot < kPvMaxTokensPerSlot ||
                     !pkd::decode_variant_built(g, page_size));
    h->variant = pv ? PKD_VARIANT_MFMA_PV : PKD_VARIANT_MFMA;
  } else {
    h->variant = variant;
  }
  h->layout = layout;
  h->int_ws = int_workspace;
  h->int_bytes = int_workspace_bytes;
  h->float_ws = float_workspace;
  h->float_bytes = float_workspace_bytes;
  h->host_ws = host_workspace;
  h->host_bytes = host_workspace_bytes;
  return PKD_OK;
}

int pkd_plan(pkd_handle* h, const int32_t* kv_indptr, const int32_t* kv_indices,
             const int32_t* kv_last_page_len, int32_t batch, int32_t num_qo_heads,
             int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t q_dtype,
             int32_t kv_dtype, int32_t kv_layout, void* int_workspace,
             size_t int_workspace_bytes, void* float_workspace, size_t float_workspace_bytes,
             void* host_workspace, size_t host_workspace_bytes, const pkd_plan_opts* opts,
             pkd_stream_t stream) {
  return plan_impl(h, nullptr, kv_indptr, kv_indices, kv_last_page_len, batch, num_qo_heads,
                   num_kv_heads, head_dim, page_size, q_dtype, kv_dtype, kv_layout,
                   int_workspace, int_workspace_bytes, float_workspace, float_workspace_bytes,
                   host_workspace, host_workspace_bytes, opts, stream);
}

int pkd_plan_shared(pkd_handle* h, const int32_t* qo_indptr, const int32_t* kv_indptr,
                    const int32_t* kv_indices, const int32_t* kv_last_page_len,
                    int32_t num_groups, int32_t num_qo_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t page_size, int32_t q_dtype, int32_t kv_dtype,
                    int32_t kv_layout, void* int_workspace, size_t int_workspace_bytes,
                    void* float_workspace, size_t float_workspace_bytes, void* host_workspace,
                    size_t host_workspace_bytes, const pkd_plan_opts* opts,
                    pkd_stream_t stream) {
  if (!qo_indptr) return fail(PKD_ERR_INVALID_ARG, "qo_indptr must be non-null");
  return plan_impl(h, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, num_groups,
                   num_qo_heads, num_kv_heads, head_dim, page_size, q_dtype, kv_dtype, kv_layout,
                   int_workspace, int_workspace_bytes, float_workspace, float_workspace_bytes,
                   host_workspace, host_workspace_bytes, opts, stream);
}

int pkd_plan_static(pkd_handle* h, const int32_t* kv_indptr, const int32_t* kv_indices,
                    const int32_t* kv_last_page_len, int32_t batch, int32_t num_qo_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t q_dtype,
                    int32_t kv_dtype, int32_t kv_layout, const pkd_plan_opts* opts,
                    pkd_stream_t stream) {
  return plan_impl(h, nullptr, kv_indptr, kv_indices, kv_last_page_len, batch, num_qo_heads,
                   num_kv_heads, head_dim, page_size, q_dtype, kv_dtype, kv_layout, nullptr, 0,
                   nullptr, 0, nullptr, 0, opts, stream, true);
}

int pkd_run(pkd_handle* h, const void* q, int32_t batch, const void* kv_cache, int64_t num_pages,
            int32_t q_dtype, int32_t kv_dtype, void* o, float* lse, float sm_scale,
            pkd_stream_t stream) {
  return pkd_run_scaled(h, q, batch, kv_cache, num_pages, q_dtype, kv_dtype, o, lse, sm_scale,
                        1.f, 1.f, stream);
}

int pkd_run_scaled(pkd_handle* h, const void* q, int32_t batch, const void* kv_cache,
                   int64_t num_pages, int32_t q_dtype, int32_t kv_dtype, void* o, float* lse,
                   float sm_scale, float k_scale, float v_scale, pkd_stream_t stream) {
  if (!h) return fail(PKD_ERR_INVALID_ARG, "null handle");
  if (!h->planned) return fail(PKD_ERR_STALE_PLAN, "pkd_run before any pkd_plan on this handle");
  if (batch != h->batch)
    return fail(PKD_ERR_STALE_PLAN, "batch " + std::to_string(batch) + " differs from the planned batch " +
                                        std::to_string(h->batch) + " (call pkd_plan for this batch)");
  if (q_dtype != h->q_dtype || kv_dtype != h->kv_dtype)
    return fail(PKD_ERR_DTYPE_MISMATCH, "run dtypes differ from the dtypes the plan was made for");
  if (h->static_plan && pkd::static_scratch_owner(h->device) != h)
    return fail(PKD_ERR_STALE_PLAN,
                "another handle's pkd_plan_static has replaced this handle's plan in the static "
                "scratch array (plan again)");
  if (!q || !kv_cache || !o) return fail(PKD_ERR_INVALID_ARG, "q, kv_cache and o must be non-null");
  if (num_pages < 1) return fail(PKD_ERR_INVALID_ARG, "num_pages must be >= 1");
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(kv_cache) & 15) ||
      (reinterpret_cast<uintptr_t>(o) & 15))
    return fail(PKD_ERR_INVALID_ARG, "q, kv_cache and o must be 16-byte aligned");
  if (!(std::isfinite(sm_scale))) return fail(PKD_ERR_INVALID_ARG, "sm_scale must be finite");
  if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(PKD_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0");
  if (h->kv_dtype != PKD_DTYPE_FP8_E4M3 && (k_scale != 1.f || v_scale != 1.f))
    return fail(PKD_ERR_INVALID_ARG, "k_scale and v_scale apply to an fp8 e4m3 cache only");

  DeviceGuard guard(h->device);
  if (!guard.ok) return hip_fail(guard.err, "hipSetDevice");
  hipStream_t s = static_cast<hipStream_t>(stream);

  const float scale = sm_scale > 0.f ? sm_scale : 1.f / std::sqrt(float(h->D));
  pkd::DecodeParams dp;
  dp.q = static_cast<const uint16_t*>(q);
  dp.kv = static_cast<const uint16_t*>(kv_cache);
  dp.o = static_cast<uint16_t*>(o);
  dp.lse = lse;
  dp.ws = static_cast<const int32_t*>(h->int_ws);
  dp.fws = static_cast<float*>(h->float_ws);
  dp.err = static_cast<int32_t*>(h->int_ws);
  dp.num_pages = num_pages;
  dp.scale_log2 = scale * k_scale * 1.44269504088896341f;
  dp.out_scale = v_scale;
  dp.num_qo_heads = h->Hq;
  dp.num_kv_heads = h->Hkv;

  pkd::MergeParams mp;
  std::memset(&mp, 0, sizeof(mp));
  mp.o_in = h->float_ws;
  mp.lse_in = nullptr;  // located from the plan header on the device
  mp.o_stride_c = int64_t(h->Hq) * pkd::kHeadDim;
  mp.lse_stride_c = h->Hq;
  mp.ws = static_cast<const int32_t*>(h->int_ws);
  mp.H = h->Hq;
  mp.o_out = static_cast<uint16_t*>(o);
  mp.lse_out = lse;
  mp.num_slots = h->num_slots;
  mp.merge_cap = merge_cap(h);

  hipEvent_t* ev = nullptr;
  hipError_t pe = profile_events(h, s, &ev);
  if (pe != hipSuccess) return hip_fail(pe, "hipEventCreate");
  const bool prof = ev != nullptr;

  hipError_t e;
  if (prof && (e = hipEventRecord(ev[0], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (h->layout.kind == PKD_PLAN_SHARED)
    e = pkd::launch_prefix_mfma(dp, h->Hq / h->Hkv, h->P, h->num_slots,
                                h->kv_dtype == PKD_DTYPE_FP8_E4M3, s);
  else if (h->kv_dtype == PKD_DTYPE_FP8_E4M3)
    e = pkd::launch_decode_fp8(dp, h->Hq / h->Hkv, h->P, h->num_slots, s);
  else if (h->variant == PKD_VARIANT_MFMA_PV)
    e = pkd::launch_decode_pv(dp, h->Hq / h->Hkv, h->P, h->num_slots, s);
  else if (h->variant == PKD_VARIANT_DOT2)
    e = pkd::launch_decode(dp, h->Hq / h->Hkv, h->P, h->num_slots, s);
  else
    e = pkd::launch_decode_mfma(dp, h->Hq / h->Hkv, h->P, h->num_slots, s);
  if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  if (prof && (e = hipEventRecord(ev[1], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  e = pkd::launch_merge_partials(mp, h->merge_grid, s);
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  if (prof && (e = hipEventRecord(ev[2], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return PKD_OK;
}

int pkd_run_composable(pkd_handle* prefix, pkd_handle* suffix, const void* q, int32_t batch,
                       const void* kv_cache, int64_t num_pages, int32_t q_dtype, int32_t kv_dtype,
                       void* o, float* lse, float sm_scale, pkd_stream_t stream) {
  return pkd_run_composable_scaled(prefix, suffix, q, batch, kv_cache, num_pages, q_dtype,
                                   kv_dtype, o, lse, sm_scale, 1.f, 1.f, stream);
}

int pkd_run_composable_scaled(pkd_handle* prefix, pkd_handle* suffix, const void* q,
                              int32_t batch, const void* kv_cache, int64_t num_pages,
                              int32_t q_dtype, int32_t kv_dtype, void* o, float* lse,
                              float sm_scale, float k_scale, float v_scale, pkd_stream_t stream) {
  if (!prefix || !suffix || prefix == suffix)
    return fail(PKD_ERR_INVALID_ARG, "two distinct handles are needed (prefix plan, suffix plan)");
  if (!prefix->planned || !suffix->planned)
    return fail(PKD_ERR_STALE_PLAN, "pkd_run_composable before both plans");
  if (prefix->layout.kind != PKD_PLAN_SHARED || suffix->layout.kind != PKD_PLAN_DECODE)
    return fail(PKD_ERR_INVALID_ARG,
                "the first handle needs a shared-prefix plan, the second a decode plan");
  if (!(prefix->plan_flags & PKD_PLAN_ALL_PARTIALS) || !(suffix->plan_flags & PKD_PLAN_ALL_PARTIALS))
    return fail(PKD_ERR_INVALID_ARG, "both plans must be made with PKD_PLAN_ALL_PARTIALS");
  if (batch != prefix->batch || batch != suffix->batch)
    return fail(PKD_ERR_STALE_PLAN, "batch differs from the plans' batch (plan both for this batch)");
  if (prefix->Hq != suffix->Hq || prefix->Hkv != suffix->Hkv || prefix->D != suffix->D ||
      prefix->P != suffix->P)
    return fail(PKD_ERR_INVALID_ARG, "the two plans differ in heads, head_dim or page size");
  if (q_dtype != prefix->q_dtype || kv_dtype != prefix->kv_dtype || q_dtype != suffix->q_dtype ||
      kv_dtype != suffix->kv_dtype)
    return fail(PKD_ERR_DTYPE_MISMATCH, "run dtypes differ from the dtypes the plans were made for");
  if (prefix->device != suffix->device)
    return fail(PKD_ERR_INVALID_ARG, "the two handles are on different devices");
  for (pkd_handle* h : {prefix, suffix})
    if (h->static_plan && pkd::static_scratch_owner(h->device) != h)
      return fail(PKD_ERR_STALE_PLAN,
                  "another handle's pkd_plan_static has replaced a plan in the static scratch array");
  if (prefix->static_plan && suffix->static_plan)
    return fail(PKD_ERR_INVALID_ARG, "the two plans cannot both live in the static scratch array");
  if (!q || !kv_cache || !o) return fail(PKD_ERR_INVALID_ARG, "q, kv_cache and o must be non-null");
  if (num_pages < 1) return fail(PKD_ERR_INVALID_ARG, "num_pages must be >= 1");
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(kv_cache) & 15) ||
      (reinterpret_cast<uintptr_t>(o) & 15))
    return fail(PKD_ERR_INVALID_ARG, "q, kv_cache and o must be 16-byte aligned");
  if (!(std::isfinite(sm_scale))) return fail(PKD_ERR_INVALID_ARG, "sm_scale must be finite");
  if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(PKD_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0");
  if (prefix->kv_dtype != PKD_DTYPE_FP8_E4M3 && (k_scale != 1.f || v_scale != 1.f))
    return fail(PKD_ERR_INVALID_ARG, "k_scale and v_scale apply to an fp8 e4m3 cache only");
  const bool fp8 = prefix->kv_dtype == PKD_DTYPE_FP8_E4M3;

  DeviceGuard guard(prefix->device);
  if (!guard.ok) return hip_fail(guard.err, "hipSetDevice");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale = sm_scale > 0.f ? sm_scale : 1.f / std::sqrt(float(prefix->D));
  auto params = [&](pkd_handle* h) {
    pkd::DecodeParams dp;
    dp.q = static_cast<const uint16_t*>(q);
    dp.kv = static_cast<const uint16_t*>(kv_cache);
    dp.o = static_cast<uint16_t*>(o);  // not written: every item writes a partial state
    dp.lse = lse;
    dp.ws = static_cast<const int32_t*>(h->int_ws);
    dp.fws = static_cast<float*>(h->float_ws);
    dp.err = static_cast<int32_t*>(h->int_ws);
    dp.num_pages = num_pages;
    dp.scale_log2 = scale * k_scale * 1.44269504088896341f;
    dp.out_scale = v_scale;
    dp.num_qo_heads = h->Hq;
    dp.num_kv_heads = h->Hkv;
    return dp;
  };
  // When the two grids fit the chip side by side (one workgroup per compute
  // unit each) and the suffix plan runs the matrix-core P.V kernel, one
  // launch runs both: the prefix plan's workgroups and the suffix plan's on
  // disjoint compute units at the same time.  Otherwise the two kernels run
  // one after the other.  (Two streams forked and joined inside the call were
  // measured first: the waits between them cost more than the overlap gave.)
  // (over an E4M3 cache the suffix plan always runs the FP8 decode kernel,
  // whose code has a one-launch form too)
  const bool one_launch = prefix->num_slots + suffix->num_slots <= prefix->cu_count &&
                          (fp8 || suffix->variant == PKD_VARIANT_MFMA_PV);
  // profiling, both handles: start, after the attention kernel(s), after the merge
  hipEvent_t *ep = nullptr, *es = nullptr;
  hipError_t e = profile_events(prefix, s, &ep);
  if (e == hipSuccess) e = profile_events(suffix, s, &es);
  if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  for (hipEvent_t* ev : {ep, es})
    if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  const pkd::DecodeParams dpre = params(prefix), ds = params(suffix);
  const int g = suffix->Hq / suffix->Hkv;
  if (one_launch) {
    e = pkd::launch_composable(dpre, ds, g, prefix->P, prefix->num_slots, suffix->num_slots, fp8,
                               s);
    if (e != hipSuccess) return hip_fail(e, "composable kernel launch");
  } else {
    e = pkd::launch_prefix_mfma(dpre, prefix->Hq / prefix->Hkv, prefix->P, prefix->num_slots, fp8,
                                s);
    if (e != hipSuccess) return hip_fail(e, "shared-prefix kernel launch");
    if (suffix->kv_dtype == PKD_DTYPE_FP8_E4M3)
      e = pkd::launch_decode_fp8(ds, g, suffix->P, suffix->num_slots, s);
    else if (suffix->variant == PKD_VARIANT_MFMA_PV)
      e = pkd::launch_decode_pv(ds, g, suffix->P, suffix->num_slots, s);
    else if (suffix->variant == PKD_VARIANT_DOT2)
      e = pkd::launch_decode(ds, g, suffix->P, suffix->num_slots, s);
    else
      e = pkd::launch_decode_mfma(ds, g, suffix->P, suffix->num_slots, s);
    if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  }
  for (hipEvent_t* ev : {ep, es})
    if (ev && (e = hipEventRecord(ev[1], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  e = pkd::launch_merge_composable(static_cast<const int32_t*>(prefix->int_ws),
                                   static_cast<const float*>(prefix->float_ws),
                                   prefix->num_slots, merge_cap(prefix),
                                   static_cast<const int32_t*>(suffix->int_ws),
                                   static_cast<const float*>(suffix->float_ws),
                                   suffix->num_slots, merge_cap(suffix), prefix->Hq,
                                   static_cast<uint16_t*>(o), lse, prefix->merge_grid, s);
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  for (hipEvent_t* ev : {ep, es})
    if (ev && (e = hipEventRecord(ev[2], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return PKD_OK;
}

int pkd_read_device_error(pkd_handle* h, int32_t* flags, pkd_stream_t stream) {
  if (!h || !flags) return fail(PKD_ERR_INVALID_ARG, "null argument");
  *flags = 0;
  if (!h->int_ws) return PKD_OK;
  DeviceGuard guard(h->device);
  if (!guard.ok) return hip_fail(guard.err, "hipSetDevice");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t value = 0;
  hipError_t e = hipMemcpyAsync(&value, h->int_ws, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the device error word");
  if (value != 0) {
    static const int32_t zero = 0;
    e = hipMemcpyAsync(h->int_ws, &zero, sizeof(int32_t), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "clearing the device error word");
  }
  *flags = value;
  return PKD_OK;
}

int pkd_append_positions(const int32_t* append_indptr, const int32_t* kv_indptr,
                         const int32_t* kv_last_page_len, int32_t batch, int32_t page_size,
                         int32_t* batch_indices, int32_t* positions, pkd_stream_t stream) {
  if (batch < 0 || page_size < 1)
    return fail(PKD_ERR_INVALID_ARG, "batch must be >= 0 and page_size >= 1");
  if (batch == 0) return PKD_OK;
  if (!append_indptr || !kv_indptr || !kv_last_page_len || !batch_indices || !positions)
    return fail(PKD_ERR_INVALID_ARG, "pkd_append_positions: null array");
  hipError_t e = pkd::launch_append_positions(append_indptr, kv_indptr, kv_last_page_len, batch,
                                              page_size, batch_indices, positions,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKD_OK : hip_fail(e, "append positions kernel launch");
}

int pkd_append_paged_kv(const void* k_new, const void* v_new, const int32_t* batch_indices,
                        const int32_t* positions, int64_t nnz_append, const int32_t* kv_indptr,
                        const int32_t* kv_indices, int32_t batch, int32_t num_kv_heads,
                        int32_t head_dim, int32_t page_size, int32_t kv_dtype,
                        int32_t kv_layout, void* kv_cache, int64_t num_pages,
                        int32_t* device_error, pkd_stream_t stream) {
  return pkd_append_paged_kv_scaled(k_new, v_new, batch_indices, positions, nnz_append, kv_indptr,
                                    kv_indices, batch, num_kv_heads, head_dim, page_size, kv_dtype,
                                    kv_layout, kv_cache, num_pages, 1.f, 1.f, device_error,
                                    stream);
}

int pkd_append_paged_kv_scaled(const void* k_new, const void* v_new,
                               const int32_t* batch_indices, const int32_t* positions,
                               int64_t nnz_append, const int32_t* kv_indptr,
                               const int32_t* kv_indices, int32_t batch, int32_t num_kv_heads,
                               int32_t head_dim, int32_t page_size, int32_t kv_dtype,
                               int32_t kv_layout, void* kv_cache, int64_t num_pages,
                               float k_scale, float v_scale, int32_t* device_error,
                               pkd_stream_t stream) {
  if (kv_dtype != PKD_DTYPE_BF16 && kv_dtype != PKD_DTYPE_FP8_E4M3)
    return fail(PKD_ERR_UNSUPPORTED, "the cache must be bf16 or fp8 e4m3");
  if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(PKD_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0");
  if (kv_dtype == PKD_DTYPE_BF16 && (k_scale != 1.f || v_scale != 1.f))
    return fail(PKD_ERR_INVALID_ARG, "k_scale and v_scale apply to an fp8 e4m3 cache only");
  if (kv_layout != PKD_LAYOUT_NHD) return fail(PKD_ERR_UNSUPPORTED, "only the NHD layout is built");
  if (head_dim != pkd::kHeadDim) return fail(PKD_ERR_UNSUPPORTED, "only head_dim 128 is built");
  if (nnz_append < 0 || batch < 1 || num_kv_heads < 1 || page_size < 1 || num_pages < 1)
    return fail(PKD_ERR_INVALID_ARG, "invalid sizes for pkd_append_paged_kv");
  if (nnz_append == 0) return PKD_OK;
  if (!k_new || !v_new || !batch_indices || !positions || !kv_indptr || !kv_indices || !kv_cache)
    return fail(PKD_ERR_INVALID_ARG, "pkd_append_paged_kv: null array");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
       reinterpret_cast<uintptr_t>(kv_cache)) & 15)
    return fail(PKD_ERR_INVALID_ARG, "k_new, v_new and kv_cache must be 16-byte aligned");
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  if (kv_dtype == PKD_DTYPE_FP8_E4M3)
    e = pkd::launch_append_kv_fp8(k_new, v_new, batch_indices, positions, nnz_append, kv_indptr,
                                  kv_indices, batch, num_kv_heads, page_size, kv_cache, num_pages,
                                  float(1.0 / double(k_scale)), float(1.0 / double(v_scale)),
                                  device_error, 8 * cus, static_cast<hipStream_t>(stream));
  else
    e = pkd::launch_append_kv(k_new, v_new, batch_indices, positions, nnz_append, kv_indptr,
                              kv_indices, batch, num_kv_heads, page_size, kv_cache, num_pages,
                              device_error, 8 * cus, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKD_OK : hip_fail(e, "append kernel launch");
}

int pkd_merge_state(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                    int32_t n, int32_t H, int32_t D, void* o_out, float* lse_out,
                    pkd_stream_t stream) {
  if (D != pkd::kHeadDim) return fail(PKD_ERR_UNSUPPORTED, "only head_dim 128 is built");
  if (n < 0 || H < 1) return fail(PKD_ERR_INVALID_ARG, "n must be >= 0 and H >= 1");
  if (n == 0) return PKD_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out)
    return fail(PKD_ERR_INVALID_ARG, "null pointer");
  hipError_t e = pkd::launch_merge_two_bf16(
      static_cast<const uint16_t*>(o_a), lse_a, static_cast<const uint16_t*>(o_b), lse_b,
      int64_t(n) * H, static_cast<uint16_t*>(o_out), lse_out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge_state launch");
  return PKD_OK;
}

int pkd_merge_states(const void* o, const float* lse, int32_t n, int32_t k, int32_t H, int32_t D,
                     void* o_out, float* lse_out, pkd_stream_t stream) {
  if (D != pkd::kHeadDim) return fail(PKD_ERR_UNSUPPORTED, "only head_dim 128 is built");
  if (n < 0 || k < 1 || H < 1) return fail(PKD_ERR_INVALID_ARG, "n >= 0, k >= 1 and H >= 1 required");
  if (n == 0) return PKD_OK;
  if (!o || !lse || !o_out) return fail(PKD_ERR_INVALID_ARG, "null pointer");
  pkd::MergeParams mp;
  std::memset(&mp, 0, sizeof(mp));
  mp.o_in = o;
  mp.lse_in = lse;
  mp.o_stride_c = int64_t(H) * pkd::kHeadDim;
  mp.lse_stride_c = H;
  mp.rows = n;
  mp.k = k;
  mp.H = H;
  mp.o_out = static_cast<uint16_t*>(o_out);
  mp.lse_out = lse_out;
  hipError_t e = pkd::launch_merge_states_bf16(mp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge_states launch");
  return PKD_OK;
}

int32_t pkd_read_sink_words(int32_t grid) {
  return grid < 1 ? 0 : grid * pkd::read_ceiling_threads();
}

int pkd_read_stream(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid,
                    pkd_stream_t stream) {
  if (!buf || !sink) return fail(PKD_ERR_INVALID_ARG, "null pointer");
  if (bytes <= 0 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
    return fail(PKD_ERR_INVALID_ARG, "bytes must be a positive multiple of 16, buf 16-byte aligned");
  if (grid < 1 || grid > (1 << 20)) return fail(PKD_ERR_INVALID_ARG, "grid must be in [1, 2^20]");
  hipError_t e = pkd::launch_read_stream(buf, bytes / 16, sink, grid,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKD_OK : hip_fail(e, "read_stream launch");
}

int pkd_read_pages(const void* base, int64_t num_pages, int64_t page_bytes,
                   const int32_t* page_ids, int64_t n_ids, uint32_t* sink, int32_t grid,
                   pkd_stream_t stream) {
  if (!base || !page_ids || !sink) return fail(PKD_ERR_INVALID_ARG, "null pointer");
  if (num_pages < 1 || n_ids < 1) return fail(PKD_ERR_INVALID_ARG, "num_pages and n_ids must be >= 1");
  if (page_bytes < 16 || (page_bytes & (page_bytes - 1)) || reinterpret_cast<uintptr_t>(base) % 16)
    return fail(PKD_ERR_INVALID_ARG,
                "page_bytes must be a power of two of at least 16, base 16-byte aligned");
  if (grid < 1 || grid > (1 << 20)) return fail(PKD_ERR_INVALID_ARG, "grid must be in [1, 2^20]");
  hipError_t e = pkd::launch_read_pages(base, page_ids, n_ids, num_pages, page_bytes, sink, grid,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKD_OK : hip_fail(e, "read_pages launch");
}

int pkd_profile_enable(pkd_handle* h, int32_t enable) {
  if (!h) return fail(PKD_ERR_INVALID_ARG, "null handle");
  h->profile = enable != 0;
  return PKD_OK;
}

int pkd_profile_read(pkd_handle* h, double* decode_ms, double* merge_ms, int64_t* runs) {
  if (!h || !decode_ms || !merge_ms || !runs) return fail(PKD_ERR_INVALID_ARG, "null argument");
  DeviceGuard guard(h->device);
  double dsum = 0, msum = 0;
  int64_t n = 0;
  for (size_t i = 0; i + 3 <= h->prof_used; i += 3) {
    hipError_t e = hipEventSynchronize(h->prof_events[i + 2]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float a = 0, b = 0;
    e = hipEventElapsedTime(&a, h->prof_events[i], h->prof_events[i + 1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&b, h->prof_events[i + 1], h->prof_events[i + 2]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    dsum += a;
    msum += b;
    ++n;
  }
  h->prof_used = 0;
  *decode_ms = dsum;
  *merge_ms = msum;
  *runs = n;
  return PKD_OK;
}

}  // extern "C"
