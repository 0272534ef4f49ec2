// The composable format's two attention kernels in one launch, for gfx950.
//
// The pinghaoyang FlashInfer page, section "Composable Format：共享前缀与独有
// 后缀分开算", computes a prefix that several requests share and each
// request's own suffix apart and merges the two states.  Here both run in
// one grid: workgroups [0, prefix_slots) run the shared-prefix kernel's code
// (prefix_mfma.h) on the prefix plan, workgroups [prefix_slots, prefix_slots
// + suffix_slots) the decode kernel with both products on the matrix cores
// (decode_pv.h; over an FP8 E4M3 cache, the FP8 decode kernel, decode_fp8.h)
// on the suffix plan.  Sized so that the whole grid is resident
// at once (one workgroup per compute unit), the two halves stream their K
// and V side by side on disjoint compute units, with no ordering between
// them to pay for; the merge that follows on the same stream waits for both.
// Both plans write every chunk's state as a partial state.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_fp8.h"
#include "decode_pv.h"
#include "kernels.h"
#include "prefix_mfma.h"

namespace pkd {
namespace {

// LDS of one workgroup: the prefix code's tiles or the decode code's
// per-wave areas, never both.
union ComposableShared {
  prefix::PShared prefix;
  struct {
    pv::VShared waves[kMaxWavesPerBlock];
    int progress[kMaxWavesPerBlock];
  } suffix;
};

// (The parameters are passed one by one: read from a structure passed by
// value, the compiler could not keep the slot's bounds in scalar registers.)
template <int G, int P>
__global__ __launch_bounds__(prefix::kThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
void composable_kernel(const uint16_t* __restrict__ q_ptr, const uint16_t* __restrict__ kv_ptr,
                       uint16_t* __restrict__ o_ptr, float* __restrict__ lse_ptr,
                       int64_t num_pages, float scale_log2, int num_qo_heads, int num_kv_heads,
                       const int32_t* __restrict__ ws_pre, float* __restrict__ fws_pre,
                       int32_t* __restrict__ err_pre, const int32_t* __restrict__ ws_suf,
                       float* __restrict__ fws_suf, int32_t* __restrict__ err_suf,
                       int prefix_slots, int suffix_slots) {
  static_assert(prefix::kThreads == 64 * kMaxWavesPerBlock, "one workgroup size for both");
  __shared__ ComposableShared sh;
  const int b = blockIdx.x;
  if (b < prefix_slots) {
    prefix::prefix_body<G, P, false>(q_ptr, kv_ptr, o_ptr, lse_ptr, ws_pre, fws_pre, err_pre,
                                     num_pages, scale_log2, 1.f, num_qo_heads, num_kv_heads, b,
                                     prefix_slots, sh.prefix);
  } else {
    pv::decode_pv_body<G, P>(q_ptr, kv_ptr, o_ptr, lse_ptr, ws_suf, fws_suf, err_suf, num_pages,
                             scale_log2, num_qo_heads, num_kv_heads, b - prefix_slots,
                             suffix_slots, sh.suffix.waves, sh.suffix.progress);
  }
}

// The same over an FP8 E4M3 cache: the shared-prefix code in its E4M3 mode
// and the FP8 decode kernel's code, both with the scales folded in as in
// their own kernels (scale_log2 carries k_scale, out_scale is v_scale).
union ComposableFp8Shared {
  prefix::PShared prefix;
  struct {
    fp8::FShared waves[kMaxWavesPerBlock];
    int progress[kMaxWavesPerBlock];
  } suffix;
};

template <int G, int P>
__global__ __launch_bounds__(prefix::kThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
void composable_fp8_kernel(const uint16_t* __restrict__ q_ptr, const uint8_t* __restrict__ kv_ptr,
                           uint16_t* __restrict__ o_ptr, float* __restrict__ lse_ptr,
                           int64_t num_pages, float scale_log2, float out_scale,
                           int num_qo_heads, int num_kv_heads,
                           const int32_t* __restrict__ ws_pre, float* __restrict__ fws_pre,
                           int32_t* __restrict__ err_pre, const int32_t* __restrict__ ws_suf,
                           float* __restrict__ fws_suf, int32_t* __restrict__ err_suf,
                           int prefix_slots, int suffix_slots) {
  __shared__ ComposableFp8Shared sh;
  const int b = blockIdx.x;
  if (b < prefix_slots) {
    prefix::prefix_body<G, P, true>(q_ptr, reinterpret_cast<const uint16_t*>(kv_ptr), o_ptr,
                                    lse_ptr, ws_pre, fws_pre, err_pre, num_pages, scale_log2,
                                    out_scale, num_qo_heads, num_kv_heads, b, prefix_slots,
                                    sh.prefix);
  } else {
    fp8::decode_fp8_body<G, P>(q_ptr, kv_ptr, o_ptr, lse_ptr, ws_suf, fws_suf, err_suf,
                               num_pages, scale_log2, out_scale, num_qo_heads, num_kv_heads,
                               b - prefix_slots, suffix_slots, sh.suffix.waves,
                               sh.suffix.progress);
  }
}

template <int G, int P>
hipError_t launch_c(const DecodeParams& pre, const DecodeParams& suf, int prefix_slots,
                    int suffix_slots, bool fp8, hipStream_t stream) {
  if (fp8)
    hipLaunchKernelGGL((composable_fp8_kernel<G, P>), dim3(prefix_slots + suffix_slots),
                       dim3(prefix::kThreads), 0, stream, pre.q,
                       reinterpret_cast<const uint8_t*>(pre.kv), pre.o, pre.lse, pre.num_pages,
                       pre.scale_log2, pre.out_scale, pre.num_qo_heads, pre.num_kv_heads, pre.ws,
                       pre.fws, pre.err, suf.ws, suf.fws, suf.err, prefix_slots, suffix_slots);
  else
    hipLaunchKernelGGL((composable_kernel<G, P>), dim3(prefix_slots + suffix_slots),
                       dim3(prefix::kThreads), 0, stream, pre.q, pre.kv, pre.o, pre.lse,
                       pre.num_pages, pre.scale_log2, pre.num_qo_heads, pre.num_kv_heads, pre.ws,
                       pre.fws, pre.err, suf.ws, suf.fws, suf.err, prefix_slots, suffix_slots);
  return hipGetLastError();
}

template <int G>
hipError_t launch_cg(const DecodeParams& pre, const DecodeParams& suf, int page_size,
                     int prefix_slots, int suffix_slots, bool fp8, hipStream_t stream) {
  switch (page_size) {
    case 16: return launch_c<G, 16>(pre, suf, prefix_slots, suffix_slots, fp8, stream);
    case 32: return launch_c<G, 32>(pre, suf, prefix_slots, suffix_slots, fp8, stream);
    case 64: return launch_c<G, 64>(pre, suf, prefix_slots, suffix_slots, fp8, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_composable(const DecodeParams& pre, const DecodeParams& suf, int g,
                             int page_size, int prefix_slots, int suffix_slots, bool fp8,
                             hipStream_t stream) {
  if (prefix_slots < 1 || suffix_slots < 1) return hipErrorInvalidValue;
  switch (g) {
    case 1: return launch_cg<1>(pre, suf, page_size, prefix_slots, suffix_slots, fp8, stream);
    case 2: return launch_cg<2>(pre, suf, page_size, prefix_slots, suffix_slots, fp8, stream);
    case 4: return launch_cg<4>(pre, suf, page_size, prefix_slots, suffix_slots, fp8, stream);
    case 8: return launch_cg<8>(pre, suf, page_size, prefix_slots, suffix_slots, fp8, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkd
