// Device helpers shared by the decode kernels: lane exchanges within a
// wave64, bf16 unpacking and packing, constants.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkd {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.44269504088896341f;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// DPP controls used below: swap neighbours (quad_perm [1,0,3,2]), swap pairs
// (quad_perm [2,3,0,1]), mirror within 8 lanes, mirror within 16 lanes.
// Applied in that order they pair every lane of a 16-lane row with each of
// the other 15 exactly once, so a row reduction takes 4 steps and leaves
// identical bits in all 16 lanes.
constexpr int kDppSwap1 = 0xB1;
constexpr int kDppSwap2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<kDppSwap1>(v);
  v += dpp<kDppSwap2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<kDppSwap1>(v));
  v = fmaxf(v, dpp<kDppSwap2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}

// Exchange with the lane 32 (permlane32) or 16 (permlane16) positions away:
// each swap instruction returns both registers, so with v in both, lane L
// ends up holding v[L] in one and v[L ^ 32] (or v[L ^ 16]) in the other.  The
// pair is read through a 64-bit cast: element access on the builtin's vector
// result loses the second element with this compiler.
__device__ __forceinline__ void xswap32(float v, float& a, float& b) {
  const auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                                  __builtin_bit_cast(uint32_t, v), false, false);
  const uint64_t u = __builtin_bit_cast(uint64_t, s);
  a = __uint_as_float(uint32_t(u));
  b = __uint_as_float(uint32_t(u >> 32));
}

__device__ __forceinline__ void xswap16(float v, float& a, float& b) {
  const auto s = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                                  __builtin_bit_cast(uint32_t, v), false, false);
  const uint64_t u = __builtin_bit_cast(uint64_t, s);
  a = __uint_as_float(uint32_t(u));
  b = __uint_as_float(uint32_t(u >> 32));
}

// Combine the 4 rows of 16 lanes: every lane gets the max (sum) of its
// column over the rows.
__device__ __forceinline__ float rows_max(float v) {
  float a, b;
  xswap32(v, a, b);
  xswap16(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float rows_sum(float v) {
  float a, b;
  xswap32(v, a, b);
  xswap16(a + b, a, b);
  return a + b;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 E4M3 codes (two dwords, code i in byte i % 4 of dword i / 4) to 8 bf16,
// element i in the low (even i) or high half of dword i / 2.  Every E4M3
// value is exact in bf16.
__device__ __forceinline__ uint4 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  return make_uint4(
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true)));
}

// Round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Streaming loads of the KV cache carry the nontemporal hint: every byte is
// read once per layer, and keeping it out of the caches' way measurably
// raises the read rate of paged gathers on gfx950.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const void* ptr) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ptr));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t load_stream4(const void* ptr) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ptr));
}

// Cache-policy operand of the raw buffer load builtins selecting "nt".
constexpr int kBufferNontemporal = 2;

// Workgroup barrier for hand-offs through LDS: orders LDS accesses around
// the barrier without waiting for the wave's outstanding global loads, as a
// full __syncthreads() would (which would drain any prefetch in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Keeping the waves of a workgroup together.  Waves w and w + 4 of an
// 8-wave workgroup share a SIMD, and when both can issue, the older one does,
// so w + 4 falls behind and the heads of one page get read far apart in time.
// Called once per few tiles by every wave: a workgroup barrier with LDS-only
// fences (the wave's prefetch stays in flight), taken only when `lockstep`
// (every wave then meets the same number of calls), and issue priority for
// the wave of its pair that has done fewer tiles.  `progress` is a
// workgroup-shared array of one counter per wave (LDS); `done` counts this
// wave's tiles so far.
template <int kWaves>
__device__ __forceinline__ void keep_pace(int* progress, int wave, int nwaves, bool lockstep,
                                          int done) {
  if (lockstep) lds_barrier();
  if (nwaves == kWaves) {
    __hip_atomic_store(&progress[wave], done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (done < __hip_atomic_load(&progress[wave ^ (kWaves / 2)], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP))
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
  }
}

// A page id outside [0, num_pages) is replaced by page 0 and remembered.
__device__ __forceinline__ int64_t safe_page(int32_t id, int64_t num_pages, int& bad) {
  const bool ok = id >= 0 && id < num_pages;
  bad |= ok ? 0 : 1;
  return ok ? id : 0;
}

// Raises the page-id flag (`code`) when any lane of the wave replaced an id.
// With pages below 16 tokens each lane reads the ids of its own rows, and
// lane 0's rows need not touch every page of a tile.
__device__ __forceinline__ void report_bad_pages(int bad, int lane, int32_t* err, int32_t code) {
  if (__builtin_amdgcn_ballot_w64(bad != 0) != 0 && lane == 0) err[0] = code;
}

}  // namespace pkd
