// Shared-prefix (composable) attention kernel for gfx950: the kernel and its
// launchers.  The device code, and how a 64-token tile is computed for the
// 128 query rows of a row block, are in prefix_mfma.h.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"
#include "prefix_mfma.h"

namespace pkd {
namespace {

template <int G, int P, bool kFp8>
__global__ __launch_bounds__(prefix::kThreads) void prefix_mfma_kernel(
    const uint16_t* __restrict__ q_ptr, const uint16_t* __restrict__ kv_ptr,
    uint16_t* __restrict__ o_ptr, float* __restrict__ lse_ptr, const int32_t* __restrict__ ws,
    float* __restrict__ fws, int32_t* __restrict__ err, int64_t num_pages, float scale_log2,
    float out_scale, int num_qo_heads, int num_kv_heads) {
  __shared__ prefix::PShared sh;
  prefix::prefix_body<G, P, kFp8>(q_ptr, kv_ptr, o_ptr, lse_ptr, ws, fws, err, num_pages,
                                  scale_log2, out_scale, num_qo_heads, num_kv_heads, blockIdx.x,
                                  gridDim.x, sh);
}

template <int G, int P, bool kFp8>
hipError_t launch_p(const DecodeParams& p, int num_slots, hipStream_t stream) {
  hipLaunchKernelGGL((prefix_mfma_kernel<G, P, kFp8>), dim3(num_slots), dim3(prefix::kThreads), 0,
                     stream, p.q, p.kv, p.o, p.lse, p.ws, p.fws, p.err, p.num_pages, p.scale_log2,
                     kFp8 ? p.out_scale : 1.f, p.num_qo_heads, p.num_kv_heads);
  return hipGetLastError();
}

template <int G, bool kFp8>
hipError_t launch_pg(const DecodeParams& p, int page_size, int num_slots, hipStream_t stream) {
  switch (page_size) {
    case 16: return launch_p<G, 16, kFp8>(p, num_slots, stream);
    case 32: return launch_p<G, 32, kFp8>(p, num_slots, stream);
    case 64: return launch_p<G, 64, kFp8>(p, num_slots, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int G>
hipError_t launch_pgf(const DecodeParams& p, int page_size, int num_slots, bool fp8,
                      hipStream_t stream) {
  return fp8 ? launch_pg<G, true>(p, page_size, num_slots, stream)
             : launch_pg<G, false>(p, page_size, num_slots, stream);
}

}  // namespace

bool prefix_variant_built(int g, int page_size) {
  return (g == 1 || g == 2 || g == 4 || g == 8) &&
         (page_size == 16 || page_size == 32 || page_size == 64);
}

hipError_t launch_prefix_mfma(const DecodeParams& p, int g, int page_size, int num_slots,
                              bool fp8, hipStream_t stream) {
  switch (g) {
    case 1: return launch_pgf<1>(p, page_size, num_slots, fp8, stream);
    case 2: return launch_pgf<2>(p, page_size, num_slots, fp8, stream);
    case 4: return launch_pgf<4>(p, page_size, num_slots, fp8, stream);
    case 8: return launch_pgf<8>(p, page_size, num_slots, fp8, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkd
