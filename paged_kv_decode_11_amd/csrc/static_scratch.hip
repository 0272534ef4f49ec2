// The library's own device scratch, for pkd_plan_static: callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid hipMalloc) plan into this array instead of
// caller-owned workspaces.
//
// `scratch` is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, from the code object's load until
// the process ends.  In host code the array's name only stands in for the
// symbol; its device address on each GPU comes from hipGetSymbolAddress,
// taken once per device with that device current (from pkd_create) and kept
// here.  Host code passes that address, never the name, to kernels and
// copies.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kernels.h"
#include "pkd.h"

namespace pkd {

static __device__ __align__(256) char scratch[PKD_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};
hipError_t g_err[kMaxDevices] = {};
bool g_done[kMaxDevices] = {};
const void* g_owner[kMaxDevices] = {};  // handle whose plan the array holds

}  // namespace

hipError_t static_scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_done[device]) return g_err[device];
  int current = -1;
  hipError_t e = hipGetDevice(&current);
  if (e == hipSuccess && current != device) e = hipErrorInvalidDevice;  // caller sets the device
  void* ptr = nullptr;
  if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e == hipSuccess && (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255)))
    e = hipErrorInvalidValue;
  g_ptr[device] = e == hipSuccess ? ptr : nullptr;
  g_err[device] = e;
  g_done[device] = true;
  return e;
}

void* static_scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  return g_done[device] ? g_ptr[device] : nullptr;
}

void static_scratch_claim(int device, const void* owner) {
  if (device < 0 || device >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_mutex);
  g_owner[device] = owner;
}

void static_scratch_release(int device, const void* owner) {
  if (device < 0 || device >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_owner[device] == owner) g_owner[device] = nullptr;
}

const void* static_scratch_owner(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  return g_owner[device];
}

}  // namespace pkd
