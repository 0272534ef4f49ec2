// Read-ceiling kernels for gfx950: how fast this GPU reads HBM when a kernel
// does nothing but read, for the two patterns the decode path depends on.
//
// Decode streams every cached key and value once per step, so its roofline
// is HBM bandwidth (aicassindra "Why serving attention is a different
// problem").  The published peak is one bound; these kernels measure what a
// plain streaming read and a plain page gather actually reach on the part, as
// context for the decode kernels' achieved rate.
//
// * stream: a contiguous buffer read once with 16-byte nontemporal loads,
//   each workgroup a contiguous range, eight loads per lane in flight.
// * page gather: whole pages (a power of two of bytes) read in the order of
//   a page-id list, each workgroup a contiguous run of the list read as one
//   stream of 16-byte pieces, eight loads per lane in flight: the access
//   pattern of a paged K/V cache read page by page.  Ids outside the buffer
//   are skipped.
//
// Each lane folds what it read into one 32-bit XOR and writes it to `sink`,
// so no load can be dropped; the XOR over the whole sink is the XOR of every
// 32-bit word read, which a test checks on the host.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"

namespace pkd {
namespace {

constexpr int kCeilThreads = 512;
constexpr int kPerLane = 8;                           // loads in flight per lane
constexpr int kStep = kCeilThreads * kPerLane;        // 16-byte pieces per workgroup step

__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Workgroup b reads pieces [b per, (b + 1) per) of the buffer, kStep pieces
// per step, 8 loads in flight per lane (64 KiB per workgroup).
__global__ __launch_bounds__(kCeilThreads) void read_stream_kernel(const uint4* __restrict__ p,
                                                                   int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t per = ((n16 + gridDim.x - 1) / gridDim.x + kStep - 1) / kStep * kStep;
  const int64_t begin = int64_t(blockIdx.x) * per;
  const int64_t end = min(n16, begin + per);
  uint32_t acc = 0;
  for (int64_t base = begin; base < end; base += kStep) {
    uint4 v[kPerLane];
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
      const int64_t i = base + k * kCeilThreads + threadIdx.x;
      v[k] = i < end ? load_stream16(p + i) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) acc ^= fold(v[k]);
  }
  sink[int64_t(blockIdx.x) * kCeilThreads + threadIdx.x] = acc;
}

// Workgroup b reads the pages of ids [b per, (b + 1) per), whole and in
// order, as one stream of 16-byte pieces (pages of 2^shift pieces), kStep
// pieces per step with 8 loads in flight per lane; the page ids of the next
// step are requested before the current step's data is waited for.
__global__ __launch_bounds__(kCeilThreads) void read_pages_kernel(
    const char* __restrict__ base, const int32_t* __restrict__ ids, int64_t n_ids,
    int64_t num_pages, int shift, uint32_t* __restrict__ sink) {
  const int64_t page_bytes = int64_t(16) << shift;
  const int64_t per = (n_ids + gridDim.x - 1) / gridDim.x;
  const int64_t kbeg = int64_t(blockIdx.x) * per;
  const int64_t kend = min(n_ids, kbeg + per);
  const int64_t np = kend > kbeg ? (kend - kbeg) << shift : 0;
  const int64_t mask = (int64_t(1) << shift) - 1;
  uint32_t acc = 0;
  int32_t id_next[kPerLane];
  auto read_ids = [&](int64_t step_base, int32_t (&dst)[kPerLane]) {
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
      const int64_t j = step_base + k * kCeilThreads + threadIdx.x;
      dst[k] = j < np ? ids[kbeg + (j >> shift)] : -1;
    }
  };
  read_ids(0, id_next);
  for (int64_t sb = 0; sb < np; sb += kStep) {
    int32_t id[kPerLane];
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) id[k] = id_next[k];
    uint4 v[kPerLane];
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
      const int64_t j = sb + k * kCeilThreads + threadIdx.x;
      // ids outside the buffer (and pieces past the range) are skipped
      v[k] = id[k] >= 0 && id[k] < num_pages
                 ? load_stream16(base + int64_t(id[k]) * page_bytes + (j & mask) * 16)
                 : make_uint4(0u, 0u, 0u, 0u);
    }
    read_ids(sb + kStep, id_next);
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) acc ^= fold(v[k]);
  }
  sink[int64_t(blockIdx.x) * kCeilThreads + threadIdx.x] = acc;
}

}  // namespace

int read_ceiling_threads() { return kCeilThreads; }

hipError_t launch_read_stream(const void* buf, int64_t n16, uint32_t* sink, int grid,
                              hipStream_t stream) {
  hipLaunchKernelGGL(read_stream_kernel, dim3(grid), dim3(kCeilThreads), 0, stream,
                     static_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError();
}

hipError_t launch_read_pages(const void* base, const int32_t* ids, int64_t n_ids,
                             int64_t num_pages, int64_t page_bytes, uint32_t* sink, int grid,
                             hipStream_t stream) {
  int shift = 0;
  while ((int64_t(16) << shift) < page_bytes) ++shift;
  if ((int64_t(16) << shift) != page_bytes) return hipErrorInvalidValue;
  hipLaunchKernelGGL(read_pages_kernel, dim3(grid), dim3(kCeilThreads), 0, stream,
                     static_cast<const char*>(base), ids, n_ids, num_pages, shift, sink);
  return hipGetLastError();
}

}  // namespace pkd
