// Paged GQA decode over an FP8 (E4M3) KV cache for gfx950: the kernel and
// its launchers.  The device code, and how a 32-token step is computed, are
// in decode_fp8.h.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_fp8.h"
#include "kernels.h"

namespace pkd {
namespace {

template <int G, int P>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 8)))
void decode_fp8_kernel(const uint16_t* __restrict__ q_ptr, const uint8_t* __restrict__ kv_ptr,
                       uint16_t* __restrict__ o_ptr, float* __restrict__ lse_ptr,
                       const int32_t* __restrict__ ws, float* __restrict__ fws,
                       int32_t* __restrict__ err, int64_t num_pages, float scale_log2,
                       float out_scale, int num_qo_heads, int num_kv_heads) {
  __shared__ fp8::FShared shared[kMaxWavesPerBlock];
  __shared__ int progress[kMaxWavesPerBlock];
  fp8::decode_fp8_body<G, P>(q_ptr, kv_ptr, o_ptr, lse_ptr, ws, fws, err, num_pages, scale_log2,
                             out_scale, num_qo_heads, num_kv_heads, blockIdx.x, gridDim.x, shared,
                             progress);
}

template <int G, int P>
hipError_t launch_f(const DecodeParams& p, int num_slots, hipStream_t stream) {
  const int waves = p.num_kv_heads < kMaxWavesPerBlock ? p.num_kv_heads : kMaxWavesPerBlock;
  hipLaunchKernelGGL((decode_fp8_kernel<G, P>), dim3(num_slots), dim3(64 * waves), 0, stream,
                     p.q, reinterpret_cast<const uint8_t*>(p.kv), p.o, p.lse, p.ws, p.fws, p.err,
                     p.num_pages, p.scale_log2, p.out_scale, p.num_qo_heads, p.num_kv_heads);
  return hipGetLastError();
}

template <int G>
hipError_t launch_fg(const DecodeParams& p, int page_size, int num_slots, hipStream_t stream) {
  switch (page_size) {
    case 1: return launch_f<G, 1>(p, num_slots, stream);
    case 2: return launch_f<G, 2>(p, num_slots, stream);
    case 4: return launch_f<G, 4>(p, num_slots, stream);
    case 8: return launch_f<G, 8>(p, num_slots, stream);
    case 16: return launch_f<G, 16>(p, num_slots, stream);
    case 32: return launch_f<G, 32>(p, num_slots, stream);
    case 64: return launch_f<G, 64>(p, num_slots, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool fp8_variant_built(int g, int page_size) {
  return g >= 1 && g <= 8 &&
         (page_size == 1 || page_size == 2 || page_size == 4 || page_size == 8 ||
          page_size == 16 || page_size == 32 || page_size == 64);
}

hipError_t launch_decode_fp8(const DecodeParams& p, int g, int page_size, int num_slots,
                             hipStream_t stream) {
  switch (g) {
    case 1: return launch_fg<1>(p, page_size, num_slots, stream);
    case 2: return launch_fg<2>(p, page_size, num_slots, stream);
    case 3: return launch_fg<3>(p, page_size, num_slots, stream);
    case 4: return launch_fg<4>(p, page_size, num_slots, stream);
    case 5: return launch_fg<5>(p, page_size, num_slots, stream);
    case 6: return launch_fg<6>(p, page_size, num_slots, stream);
    case 7: return launch_fg<7>(p, page_size, num_slots, stream);
    case 8: return launch_fg<8>(p, page_size, num_slots, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkd
