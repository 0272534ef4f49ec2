// Plan upload for gfx950: one kernel on the caller's stream moves the plan
// image from pinned host memory (read by the GPU over the bus) and the
// kv_indices snapshot into the int workspace.  Keeping the upload on the
// compute queue, rather than handing it to a copy engine, leaves no
// cross-engine wait between the plan and the first decode launch behind it.
// On the way it writes into each item row of a decode plan the ids of the
// item's first two pages, which only the device holds; the decode kernels
// then start an item's loads as soon as its row has arrived.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace pkd {
namespace {

constexpr int kUploadThreads = 256;

__global__ __launch_bounds__(kUploadThreads) void plan_upload_kernel(
    const int4* __restrict__ image, int4* __restrict__ dst, int64_t image_vec4,
    const int32_t* __restrict__ indices, int32_t* __restrict__ dst_indices, int64_t nnz,
    int64_t first_vec4, int64_t first_rows, int64_t items_vec4, int64_t item_rows) {
  const int64_t stride = int64_t(gridDim.x) * kUploadThreads;
  const int64_t tid = int64_t(blockIdx.x) * kUploadThreads + threadIdx.x;
  for (int64_t i = tid; i < image_vec4; i += stride) {
    int4 v = image[i];
    // words 6 and 7 of an item row (in the first-item table or the items),
    // written by the thread that copies the row's second half; both tables
    // start at a multiple of 8 ints
    const int64_t r1 = i - first_vec4;
    const int64_t r2 = i - items_vec4;
    if (((r1 >= 0 && r1 < 2 * first_rows) || (r2 >= 0 && r2 < 2 * item_rows)) && (i & 1)) {
      const int4 head = image[i - 1];  // request, page_begin, num_pages, last_len
      if (head.z > 0) {
        v.z = indices[head.y];
        v.w = indices[head.y + (head.z > 1 ? 1 : 0)];
      }
    }
    dst[i] = v;
  }
  for (int64_t i = tid; i < nnz; i += stride) dst_indices[i] = indices[i];
}

}  // namespace

hipError_t launch_plan_upload(const int32_t* image, int32_t* dst, int64_t image_ints,
                              const int32_t* indices, int32_t* dst_indices, int64_t nnz,
                              int64_t first_off, int64_t first_rows, int64_t items_off,
                              int64_t item_rows, hipStream_t stream) {
  if ((reinterpret_cast<uintptr_t>(image) | reinterpret_cast<uintptr_t>(dst)) & 15 ||
      image_ints % 4 != 0 || first_off % 8 != 0 || first_off < 0 ||
      first_off + 8 * first_rows > image_ints || items_off % 8 != 0 || items_off < 0 ||
      items_off + 8 * item_rows > image_ints)
    return hipErrorInvalidValue;
  const int64_t work = image_ints / 4 > nnz ? image_ints / 4 : nnz;
  int64_t grid = (work + kUploadThreads - 1) / kUploadThreads;
  if (grid > 1024) grid = 1024;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(plan_upload_kernel, dim3(unsigned(grid)), dim3(kUploadThreads), 0, stream,
                     reinterpret_cast<const int4*>(image), reinterpret_cast<int4*>(dst),
                     image_ints / 4, indices, dst_indices, nnz, first_off / 4, first_rows,
                     items_off / 4, item_rows);
  return hipGetLastError();
}

}  // namespace pkd
