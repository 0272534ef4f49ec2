// Merge of attention states for gfx950.
//
// The combine is the one on the pinghaoyang FlashInfer page, section
// "在线 Softmax 为什么允许任意切块" (why online softmax allows any split), and
// in aicassindra "Load balancing with split-KV": with M = max_c lse_c and
// w_c = exp(lse_c - M), the merged state is o = sum_c w_c o_c / sum_c w_c and
// lse = M + log sum_c w_c.  States are merged in a fixed order with no
// atomics, so results are reproducible (pinghaoyang, Stream-K paragraph).
//
// Work units are taken in a grid-stride loop so the grid is fixed.  A
// (row, query head) task of few states is done by 32 lanes in one round trip
// (merge_small); a task of more states by a workgroup whose 8 groups of 32
// lanes fold every 8th state (merge_task, also the uniform bf16 merge); in a
// plan with a task above 64 states, each task of more than a few is cut
// across head_dim over several workgroups (merge_wide).
// Every path folds its states in a fixed order, by the rule above, into a
// running (max, weight sum, weighted o).  Empty states (lse = -inf) get
// weight 0; a task with only empty states yields o = 0, lse = -inf.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"
#include "pkd.h"
#include "plan_layout.h"

namespace pkd {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kMergeThreads = 256;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

// Where a task's states are and where its result goes.
struct Task {
  int64_t first;    // index of state 0 (times the strides below)
  int k;            // number of states
  int64_t out_row;  // output row (request)
};

// States of a task are dealt to 8 groups of 32 lanes (state c to group
// c % 8).  A group loads up to kRound of its states -- lse and o together --
// in one go, folds them into a running (max, sum of weights, weighted o),
// and repeats; the 8 group states are then combined in group order.  A task
// with up to 8 * kRound states thus costs one dependent round trip to memory.
constexpr int kRound = 8;

template <typename OT>
__device__ void merge_task(const MergeParams& p, const Task& t, int h, float* grp_m, float* grp_s,
                           float4* grp_acc) {
  const int tid = threadIdx.x;
  const int grp = tid >> 5;
  const int gl = tid & 31;
  const OT* o_in = static_cast<const OT*>(p.o_in);

  float m = kNegInf, s = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = grp; c0 < t.k; c0 += 8 * kRound) {
    float L[kRound];
    float4 v[kRound];
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      const int c = c0 + 8 * r;
      L[r] = kNegInf;
      v[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < t.k) {
        const int64_t st = t.first + c;
        L[r] = p.lse_in[st * p.lse_stride_c + h];
        v[r] = load4(o_in + st * p.o_stride_c + int64_t(h) * kHeadDim + gl * 4);
      }
    }
    float mr = m;
#pragma unroll
    for (int r = 0; r < kRound; ++r) mr = fmaxf(mr, L[r]);
    if (mr == kNegInf) continue;  // only empty states so far
    const float keep = __builtin_amdgcn_exp2f((m - mr) * kLog2e);  // 0 when m = -inf
    s *= keep;
    acc.x *= keep;
    acc.y *= keep;
    acc.z *= keep;
    acc.w *= keep;
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      const float w = __builtin_amdgcn_exp2f((L[r] - mr) * kLog2e);  // 0 for empty states
      s += w;
      acc.x = fmaf(w, v[r].x, acc.x);
      acc.y = fmaf(w, v[r].y, acc.y);
      acc.z = fmaf(w, v[r].z, acc.z);
      acc.w = fmaf(w, v[r].w, acc.w);
    }
    m = mr;
  }
  if (gl == 0) {
    grp_m[grp] = m;
    grp_s[grp] = s;
  }
  grp_acc[grp * 32 + gl] = acc;
  __syncthreads();

  if (grp == 0) {
    float M = kNegInf;
#pragma unroll
    for (int g = 0; g < 8; ++g) M = fmaxf(M, grp_m[g]);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float lse = kNegInf;
    if (M != kNegInf) {
      float S = 0.f;
      float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const float w = __builtin_amdgcn_exp2f((grp_m[g] - M) * kLog2e);
        const float4 a = grp_acc[g * 32 + gl];
        S = fmaf(w, grp_s[g], S);
        A.x = fmaf(w, a.x, A.x);
        A.y = fmaf(w, a.y, A.y);
        A.z = fmaf(w, a.z, A.z);
        A.w = fmaf(w, a.w, A.w);
      }
      const float inv = 1.f / S;
      o = make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
      lse = M + __log2f(S) * kLn2;
    }
    uint2 w;
    w.x = pack_bf16x2(o.x, o.y);
    w.y = pack_bf16x2(o.z, o.w);
    *reinterpret_cast<uint2*>(p.o_out + (t.out_row * p.H + h) * kHeadDim + gl * 4) = w;
    if (p.lse_out && gl == 0) p.lse_out[t.out_row * p.H + h] = lse;
  }
  __syncthreads();
}

// A task of at most kSmallK fp32 states done by one group of 32 lanes: all
// its states loaded at once, then folded in order.
constexpr int kSmallK = 16;

__device__ void merge_small(const MergeParams& p, const Task& t, int h, int gl) {
  const float* o_in = static_cast<const float*>(p.o_in);
  float L[kSmallK];
  float4 v[kSmallK];
#pragma unroll
  for (int c = 0; c < kSmallK; ++c) {
    L[c] = kNegInf;
    v[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < t.k) {
      const int64_t st = t.first + c;
      L[c] = p.lse_in[st * p.lse_stride_c + h];
      v[c] = load4(o_in + st * p.o_stride_c + int64_t(h) * kHeadDim + gl * 4);
    }
  }
  float M = kNegInf;
#pragma unroll
  for (int c = 0; c < kSmallK; ++c) M = fmaxf(M, L[c]);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float lse = kNegInf;
  if (M != kNegInf) {
    float S = 0.f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int c = 0; c < kSmallK; ++c) {
      const float w = __builtin_amdgcn_exp2f((L[c] - M) * kLog2e);  // 0 past k
      S += w;
      A.x = fmaf(w, v[c].x, A.x);
      A.y = fmaf(w, v[c].y, A.y);
      A.z = fmaf(w, v[c].z, A.z);
      A.w = fmaf(w, v[c].w, A.w);
    }
    const float inv = 1.f / S;
    o = make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
    lse = M + __log2f(S) * kLn2;
  }
  uint2 w;
  w.x = pack_bf16x2(o.x, o.y);
  w.y = pack_bf16x2(o.z, o.w);
  *reinterpret_cast<uint2*>(p.o_out + (t.out_row * p.H + h) * kHeadDim + gl * 4) = w;
  if (p.lse_out && gl == 0) p.lse_out[t.out_row * p.H + h] = lse;
}

// A task of many fp32 states, cut across head_dim into kSlices work units of
// 16 dims, so that one long task (a request split over every slot) spreads
// over as many workgroups.  Lane l of a unit covers dims 4 (l & 3) .. + 3 of
// the slice and the states c = (l >> 2) + 64 i: up to kWideRound of them per
// round trip to memory, all 256 states of a round requested at once.  Each
// lane folds its states in order into a running (max, weight sum, weighted
// o); the 16 lanes of a wave that share dims then combine pairwise (lanes
// 4 and 8, 16, 32 apart, a fixed tree) and the 4 waves in wave order.
constexpr int kSlices = 8;
constexpr int kWideRound = 4;

struct Running {
  float m, s;
  float4 a;
};

// x := the merge of states x and y (an empty state has m = -inf, s = 0).
__device__ __forceinline__ void fold(Running& x, const Running& y) {
  const float M = fmaxf(x.m, y.m);
  if (M == kNegInf) return;
  const float wx = __builtin_amdgcn_exp2f((x.m - M) * kLog2e);  // 0 when x.m = -inf
  const float wy = __builtin_amdgcn_exp2f((y.m - M) * kLog2e);
  x.m = M;
  x.s = wx * x.s + wy * y.s;
  x.a = make_float4(wx * x.a.x + wy * y.a.x, wx * x.a.y + wy * y.a.y, wx * x.a.z + wy * y.a.z,
                    wx * x.a.w + wy * y.a.w);
}

__device__ __forceinline__ Running shfl_xor(const Running& x, int d) {
  Running y;
  y.m = __shfl_xor(x.m, d);
  y.s = __shfl_xor(x.s, d);
  y.a = make_float4(__shfl_xor(x.a.x, d), __shfl_xor(x.a.y, d), __shfl_xor(x.a.z, d),
                    __shfl_xor(x.a.w, d));
  return y;
}

__device__ void merge_wide(const MergeParams& p, const Task& t, int h, int slice,
                           Running* wave_state) {
  const int tid = threadIdx.x;
  const int piece = tid & 3;
  const int dim = 16 * slice + 4 * piece;
  const float* o_in = static_cast<const float*>(p.o_in);
  Running x = {kNegInf, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
  for (int c0 = tid >> 2; c0 < t.k; c0 += 64 * kWideRound) {
    float L[kWideRound];
    float4 v[kWideRound];
#pragma unroll
    for (int r = 0; r < kWideRound; ++r) {
      const int c = c0 + 64 * r;
      L[r] = kNegInf;
      v[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < t.k) {
        const int64_t st = t.first + c;
        L[r] = p.lse_in[st * p.lse_stride_c + h];
        v[r] = load4(o_in + st * p.o_stride_c + int64_t(h) * kHeadDim + dim);
      }
    }
    float mr = x.m;
#pragma unroll
    for (int r = 0; r < kWideRound; ++r) mr = fmaxf(mr, L[r]);
    if (mr == kNegInf) continue;  // only empty states so far
    const float keep = __builtin_amdgcn_exp2f((x.m - mr) * kLog2e);  // 0 when x.m = -inf
    x.s *= keep;
    x.a = make_float4(x.a.x * keep, x.a.y * keep, x.a.z * keep, x.a.w * keep);
#pragma unroll
    for (int r = 0; r < kWideRound; ++r) {
      const float w = __builtin_amdgcn_exp2f((L[r] - mr) * kLog2e);  // 0 for empty states
      x.s += w;
      x.a.x = fmaf(w, v[r].x, x.a.x);
      x.a.y = fmaf(w, v[r].y, x.a.y);
      x.a.z = fmaf(w, v[r].z, x.a.z);
      x.a.w = fmaf(w, v[r].w, x.a.w);
    }
    x.m = mr;
  }
#pragma unroll
  for (int d = 4; d < 64; d <<= 1) fold(x, shfl_xor(x, d));
  const int wave = tid >> 6;
  if ((tid & 63) < 4) wave_state[4 * wave + piece] = x;
  __syncthreads();
  if (tid < 4) {
    Running z = wave_state[piece];
#pragma unroll
    for (int w = 1; w < kMergeThreads / 64; ++w) fold(z, wave_state[4 * w + piece]);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float lse = kNegInf;
    if (z.m != kNegInf) {
      const float inv = 1.f / z.s;
      o = make_float4(z.a.x * inv, z.a.y * inv, z.a.z * inv, z.a.w * inv);
      lse = z.m + __log2f(z.s) * kLn2;
    }
    uint2 w;
    w.x = pack_bf16x2(o.x, o.y);
    w.y = pack_bf16x2(o.z, o.w);
    *reinterpret_cast<uint2*>(p.o_out + (t.out_row * p.H + h) * kHeadDim + dim) = w;
    if (p.lse_out && slice == 0 && piece == 0) p.lse_out[t.out_row * p.H + h] = lse;
  }
  __syncthreads();
}

// Split requests of the current plan: fp32 partials in the float workspace.
// Tasks (split request e, q head h) = e H + h form blocks of 8.  A block where
// no task has more than kSmallK states is one work unit: each group of 32
// lanes does one of its tasks in a single round trip to memory.  The tasks of
// the other blocks are work units of their own, done with all 256 lanes
// (merge_task, one round trip up to 64 states), or, when some task of the
// plan has more than 64 states, cut into kSlices work units each
// (merge_wide), so a few long tasks still spread over many workgroups.
__device__ __forceinline__ Task task_of_entry(const int4 m) {
  Task t;
  t.out_row = m.x;
  t.first = m.y;
  t.k = m.z;
  return t;
}

__device__ __forceinline__ int4 merge_entry(const int32_t* merges, int e) {
  return *reinterpret_cast<const int4*>(merges + 4 * int64_t(e));
}

__global__ __launch_bounds__(kMergeThreads) void merge_partials_kernel(MergeParams p) {
  __shared__ Running wave_state[4 * (kMergeThreads / 64)];
  __shared__ float grp_m[8];
  __shared__ float grp_s[8];
  __shared__ float4 grp_acc[8 * 32];
  const int32_t* hdr = p.ws + PKD_HEADER_BASE;
  const int32_t* merges = p.ws + plan_off_merge(p.num_slots);
  const int H = p.H;
  const int grp = threadIdx.x >> 5;
  const int gl = threadIdx.x & 31;
  // The merge list sits at an offset fixed by the slot count, so the entry
  // of this workgroup's first work unit on either pass is requested together
  // with the header (clamped into the workspace; an entry past the list is
  // never used) and both are waited for at once.
  const int b = blockIdx.x;
  const int last_entry = max(p.merge_cap - 1, 0);
  const int4 pre_small = merge_entry(merges, min((8 * b + grp) / H, last_entry));
  // The large-task pass takes a task per unit or cuts each task into
  // kSlices units (which, the header tells); the entry of unit b either way.
  // (Vector loads, so that they are issued with the others, not after the
  // header's scalar loads have been waited for.)
  int e_one = min(b / H, last_entry);
  int e_wide = min(b / kSlices / H, last_entry);
  asm volatile("" : "+v"(e_one), "+v"(e_wide));
  const int4 pre_one = merge_entry(merges, e_one);
  const int4 pre_wide = merge_entry(merges, e_wide);
  const int n_split = hdr[PKD_H_SPLIT];
  const int n_partials = hdr[PKD_H_PARTIALS];
  const int kmin = hdr[PKD_H_MIN_CHUNKS];
  const int kmax = hdr[PKD_H_MAX_CHUNKS];
  asm volatile("" ::"v"(pre_small.x), "v"(pre_small.y), "v"(pre_small.z), "v"(pre_one.x),
               "v"(pre_one.y), "v"(pre_one.z), "v"(pre_wide.x), "v"(pre_wide.y), "v"(pre_wide.z),
               "s"(n_split), "s"(n_partials), "s"(kmin), "s"(kmax));
  MergeParams q = p;
  q.lse_in = static_cast<const float*>(p.o_in) + int64_t(n_partials) * H * kHeadDim;
  const int tasks = n_split * H;
  const int blocks = (tasks + 7) / 8;
  auto small_block = [&](int blk) {
    int most = 0;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int task = 8 * blk + g;
      if (task < tasks) most = max(most, merges[4 * (task / H) + 2]);
    }
    return most <= kSmallK;
  };
  // the plan's fewest and most states per entry tell which passes have work
  const bool some_small = kmin <= kSmallK;
  const bool some_large = kmax > kSmallK;
  if (some_small) {
    for (int blk = b; blk < blocks; blk += gridDim.x) {
      if (some_large && !small_block(blk)) continue;
      const int task = 8 * blk + grp;
      if (task < tasks) {
        const int4 m = blk == b ? pre_small : merge_entry(merges, task / H);
        merge_small(q, task_of_entry(m), task % H, gl);
      }
    }
  }
  if (some_large) {
    // up to 8 * kRound states a task is one round trip for one workgroup;
    // past that (a plan with a request cut into more chunks) every large
    // task is cut across head_dim
    const int slices = kmax > 8 * kRound ? kSlices : 1;
    const int units = tasks * slices;
    for (int u = b; u < units; u += gridDim.x) {
      const int task = u / slices;
      if (some_small && small_block(task / 8)) continue;
      const int4 m = u != b ? merge_entry(merges, task / H) : slices == 1 ? pre_one : pre_wide;
      if (slices == 1)
        merge_task<float>(q, task_of_entry(m), task % H, grp_m, grp_s, grp_acc);
      else
        merge_wide(q, task_of_entry(m), task % H, u % kSlices, wave_state);
    }
  }
}

// The composable format's merge: for each request r and query head h, the
// partial states of r in plan A (a shared-prefix plan: the chunks of r's
// group) followed by those of r in plan B (a decode plan: the chunks of r's
// own pages), both plans made with every request's states as partials, so
// entry r of each plan's merge list is request r.  The states are dealt to
// the 8 lane groups as in merge_task, state c of the joint sequence being
// A's c-th for c < k_A and B's (c - k_A)-th after, and combined by the same
// rule in the same fixed order.
struct Segment {
  const float* o;    // partial o of the plan, [n_partials, H, 128]
  const float* lse;  // partial lse, [n_partials, H]
  int64_t first;
  int k;
};

__device__ void merge_segments(const Segment& a, const Segment& b, int H, int h, int64_t out_row,
                               uint16_t* o_out, float* lse_out, float* grp_m, float* grp_s,
                               float4* grp_acc) {
  const int tid = threadIdx.x;
  const int grp = tid >> 5;
  const int gl = tid & 31;
  const int k = a.k + b.k;
  float m = kNegInf, s = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = grp; c0 < k; c0 += 8 * kRound) {
    float L[kRound];
    float4 v[kRound];
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      const int c = c0 + 8 * r;
      L[r] = kNegInf;
      v[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < k) {
        const bool in_a = c < a.k;
        const Segment& g = in_a ? a : b;
        const int64_t st = g.first + (in_a ? c : c - a.k);
        L[r] = g.lse[st * H + h];
        v[r] = load4(g.o + (st * H + h) * kHeadDim + gl * 4);
      }
    }
    float mr = m;
#pragma unroll
    for (int r = 0; r < kRound; ++r) mr = fmaxf(mr, L[r]);
    if (mr == kNegInf) continue;
    const float keep = __builtin_amdgcn_exp2f((m - mr) * kLog2e);
    s *= keep;
    acc.x *= keep;
    acc.y *= keep;
    acc.z *= keep;
    acc.w *= keep;
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      const float w = __builtin_amdgcn_exp2f((L[r] - mr) * kLog2e);
      s += w;
      acc.x = fmaf(w, v[r].x, acc.x);
      acc.y = fmaf(w, v[r].y, acc.y);
      acc.z = fmaf(w, v[r].z, acc.z);
      acc.w = fmaf(w, v[r].w, acc.w);
    }
    m = mr;
  }
  if (gl == 0) {
    grp_m[grp] = m;
    grp_s[grp] = s;
  }
  grp_acc[grp * 32 + gl] = acc;
  __syncthreads();
  if (grp == 0) {
    float M = kNegInf;
#pragma unroll
    for (int g = 0; g < 8; ++g) M = fmaxf(M, grp_m[g]);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float lse = kNegInf;
    if (M != kNegInf) {
      float S = 0.f;
      float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const float w = __builtin_amdgcn_exp2f((grp_m[g] - M) * kLog2e);
        const float4 x = grp_acc[g * 32 + gl];
        S = fmaf(w, grp_s[g], S);
        A.x = fmaf(w, x.x, A.x);
        A.y = fmaf(w, x.y, A.y);
        A.z = fmaf(w, x.z, A.z);
        A.w = fmaf(w, x.w, A.w);
      }
      const float inv = 1.f / S;
      o = make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
      lse = M + __log2f(S) * kLn2;
    }
    uint2 w;
    w.x = pack_bf16x2(o.x, o.y);
    w.y = pack_bf16x2(o.z, o.w);
    *reinterpret_cast<uint2*>(o_out + (out_row * H + h) * kHeadDim + gl * 4) = w;
    if (lse_out && gl == 0) lse_out[out_row * H + h] = lse;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kMergeThreads) void merge_composable_kernel(
    const int32_t* __restrict__ ws_a, const float* __restrict__ fws_a, int slots_a, int cap_a,
    const int32_t* __restrict__ ws_b, const float* __restrict__ fws_b, int slots_b, int cap_b,
    int H, uint16_t* __restrict__ o_out, float* __restrict__ lse_out) {
  __shared__ float grp_m[8];
  __shared__ float grp_s[8];
  __shared__ float4 grp_acc[8 * 32];
  const int32_t* ha = ws_a + PKD_HEADER_BASE;
  const int32_t* hb = ws_b + PKD_HEADER_BASE;
  const int32_t* ma = ws_a + plan_off_merge(slots_a);
  const int32_t* mb = ws_b + plan_off_merge(slots_b);
  // this workgroup's first entry of both lists, requested with the headers
  // (clamped into each workspace; unused when past the lists)
  const int e0 = int(blockIdx.x) / H;
  const int4 pre_a = merge_entry(ma, min(e0, max(cap_a - 1, 0)));
  const int4 pre_b = merge_entry(mb, min(e0, max(cap_b - 1, 0)));
  const int split_a = ha[PKD_H_SPLIT], split_b = hb[PKD_H_SPLIT];
  const int parts_a = ha[PKD_H_PARTIALS], parts_b = hb[PKD_H_PARTIALS];
  asm volatile("" ::"s"(pre_a.x), "s"(pre_a.y), "s"(pre_a.z), "s"(pre_b.y), "s"(pre_b.z),
               "s"(split_a), "s"(split_b), "s"(parts_a), "s"(parts_b));
  // both lists name every request in order (checked on the host)
  const int n = min(split_a, split_b);
  const float* lse_a = fws_a + int64_t(parts_a) * H * kHeadDim;
  const float* lse_b = fws_b + int64_t(parts_b) * H * kHeadDim;
  const int64_t tasks = int64_t(n) * H;
  for (int64_t task = blockIdx.x; task < tasks; task += gridDim.x) {
    const int e = int(task / H);
    const int h = int(task - int64_t(e) * H);
    const bool first = task == blockIdx.x;
    const int4 xa = first ? pre_a : merge_entry(ma, e);
    const int4 xb = first ? pre_b : merge_entry(mb, e);
    const Segment a = {fws_a, lse_a, xa.y, xa.z};
    const Segment b = {fws_b, lse_b, xb.y, xb.z};
    merge_segments(a, b, H, h, xa.x, o_out, lse_out, grp_m, grp_s, grp_acc);
  }
}

// k bf16 states per row, rows laid out uniformly.
__global__ __launch_bounds__(kMergeThreads) void merge_states_kernel(MergeParams p) {
  __shared__ float grp_m[8];
  __shared__ float grp_s[8];
  __shared__ float4 grp_acc[8 * 32];
  const int64_t tasks = int64_t(p.rows) * p.H;
  for (int64_t task = blockIdx.x; task < tasks; task += gridDim.x) {
    const int64_t row = task / p.H;
    const int h = int(task - row * p.H);
    Task t;
    t.out_row = row;
    t.first = row * p.k;
    t.k = p.k;
    merge_task<uint16_t>(p, t, h, grp_m, grp_s, grp_acc);
  }
}

// Two bf16 states per row; 32 lanes per row, 4 elements per lane.
__global__ __launch_bounds__(256) void merge_two_kernel(const uint16_t* o_a, const float* lse_a,
                                                        const uint16_t* o_b, const float* lse_b,
                                                        int64_t rows, uint16_t* o_out,
                                                        float* lse_out) {
  const int64_t row = int64_t(blockIdx.x) * 8 + (threadIdx.x >> 5);
  const int gl = threadIdx.x & 31;
  if (row >= rows) return;
  const float la = lse_a[row];
  const float lb = lse_b[row];
  const float4 a = load4(o_a + row * kHeadDim + gl * 4);
  const float4 b = load4(o_b + row * kHeadDim + gl * 4);
  const float M = fmaxf(la, lb);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float lse = kNegInf;
  if (M != kNegInf) {
    const float wa = __builtin_amdgcn_exp2f((la - M) * kLog2e);
    const float wb = __builtin_amdgcn_exp2f((lb - M) * kLog2e);
    const float inv = 1.f / (wa + wb);
    o = make_float4((wa * a.x + wb * b.x) * inv, (wa * a.y + wb * b.y) * inv,
                    (wa * a.z + wb * b.z) * inv, (wa * a.w + wb * b.w) * inv);
    lse = M + __log2f(wa + wb) * kLn2;
  }
  uint2 w;
  w.x = pack_bf16x2(o.x, o.y);
  w.y = pack_bf16x2(o.z, o.w);
  *reinterpret_cast<uint2*>(o_out + row * kHeadDim + gl * 4) = w;
  if (gl == 0) lse_out[row] = lse;
}

}  // namespace

hipError_t launch_merge_partials(const MergeParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(merge_partials_kernel, dim3(grid), dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_merge_composable(const int32_t* ws_a, const float* fws_a, int slots_a, int cap_a,
                                   const int32_t* ws_b, const float* fws_b, int slots_b, int cap_b,
                                   int H, uint16_t* o_out, float* lse_out, int grid,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(merge_composable_kernel, dim3(grid), dim3(kMergeThreads), 0, stream, ws_a,
                     fws_a, slots_a, cap_a, ws_b, fws_b, slots_b, cap_b, H, o_out, lse_out);
  return hipGetLastError();
}

hipError_t launch_merge_states_bf16(const MergeParams& p, hipStream_t stream) {
  const int64_t tasks = int64_t(p.rows) * p.H;
  const int grid = int(tasks < 65536 ? tasks : 65536);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_states_kernel, dim3(grid), dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_merge_two_bf16(const uint16_t* o_a, const float* lse_a, const uint16_t* o_b,
                                 const float* lse_b, int64_t rows, uint16_t* o_out,
                                 float* lse_out, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t grid = (rows + 7) / 8;
  hipLaunchKernelGGL(merge_two_kernel, dim3(unsigned(grid)), dim3(256), 0, stream, o_a, lse_a,
                     o_b, lse_b, rows, o_out, lse_out);
  return hipGetLastError();
}

}  // namespace pkd
