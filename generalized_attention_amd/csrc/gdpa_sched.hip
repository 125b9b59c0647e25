// Jagged work decomposition: one workgroup builds the longest-first list of
// (group, head, sequence) work items from the device offsets.
//
// The Kunlun review (section 2.3) names tile scheduling over jagged, large-batch inputs as one of
// the GDPA kernel's levers. Here a work item is one whole (sequence, head) pair; the
// main kernels take items in list order, one workgroup per item, and the hardware dispatcher
// hands the next item to whichever compute unit frees up first, so a longest-first order gives
// the classic LPT balance without a persistent kernel or atomics in the main kernels.
#include "gdpa_check.hpp"
#include "gdpa_device.hpp"
#include "gdpa_launch.hpp"

namespace gdpa {

// Two classes of items share one descending key space: the items of short-key groups (which the
// backward runs in a kernel of its own, over the tail of the list) take keys [0, kNumBuckets), every
// other group's items keys [kNumBuckets, 2 kNumBuckets), so the second class comes first and each
// class is longest-first within itself.
constexpr int kClassKeys = 2 * kNumBuckets;

// Launched with exactly kNumBuckets threads (two adjacent keys per thread in the scan).
__global__ void __launch_bounds__(kNumBuckets) build_schedule_kernel(LaunchDesc d) {
  static_assert(kNumBuckets % 64 == 0 && kNumBuckets / 64 <= 64, "bucket scan layout");
  __shared__ int32_t hist[kClassKeys];
  __shared__ int32_t cursor[kClassKeys];
  __shared__ int32_t wave_total[kNumBuckets / 64];
  const int tid = threadIdx.x;
  if (tid == 0) {
    d.err[0] = 0;           // a new call: clear the device error word
    d.err[1] = d.plan_sig;  // the list's signature, for planned calls
  }
  for (int i = tid; i < kClassKeys; i += blockDim.x) hist[i] = 0;
  __syncthreads();

  // pass 1: bucket key of every sequence (the thread's first sequence stays in registers, later
  // ones go through the scratch array) and the bucket histogram in work items
  int key0 = 0, g0 = 0, b0 = 0;
  for (int s = tid; s < d.n_seqs_total; s += blockDim.x) {
    int g = 0;
    while (g + 1 < d.n_groups && s >= d.grp[g + 1].seq_base) ++g;
    const GroupDesc& gd = d.grp[g];
    const int b = s - gd.seq_base;
    const int64_t L = gd.q_off[b + 1] - gd.q_off[b];
    int64_t N = gd.kv_off[b + 1] - gd.kv_off[b];
    if (gd.wl >= 0 && gd.wr >= 0) N = N < (int64_t)(gd.wl + gd.wr + 1) ? N : (int64_t)(gd.wl + gd.wr + 1);
    const int64_t work = (L + 32) * (N + 32) * gd.head_dim;  // +32: fixed per-tile costs
    int64_t key = work >> d.work_shift;
    if (key > kNumBuckets - 1) key = kNumBuckets - 1;
    if (key < 0) key = 0;  // (offsets that decrease: the main kernels refuse such an item)
    if (!gd.short_keys) key += kNumBuckets;
    if (s == tid) {
      key0 = (int)key;
      g0 = g;
      b0 = b;
    } else {
      d.scratch[s] = (int32_t)key;
    }
    atomicAdd(&hist[key], gd.num_heads);
  }
  __syncthreads();
  // exclusive prefix sum in descending key order (longest work first): thread t owns keys
  // kClassKeys-1-2t and the one below it. Each wave scans its 64 key pairs with lane shuffles; the
  // wave totals are then added in wave order.
  {
    const int k = kClassKeys - 1 - 2 * tid;
    const int lane = tid & 63, wave = tid >> 6;
    const int32_t v = hist[k] + hist[k - 1];
    int32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t up = __shfl_up(incl, off, 64);
      if (lane >= off) incl += up;
    }
    if (lane == 63) wave_total[wave] = incl;
    __syncthreads();
    int32_t base = 0;
    for (int w = 0; w < wave; ++w) base += wave_total[w];
    cursor[k] = base + incl - v;
    cursor[k - 1] = base + incl - v + hist[k];
  }
  __syncthreads();
  // pass 2: each sequence takes num_heads consecutive slots of its bucket (the order inside a
  // bucket is free: items of one bucket have about the same work)
  for (int s = tid; s < d.n_seqs_total; s += blockDim.x) {
    int g, b;
    int32_t key;
    if (s == tid) {
      g = g0;
      b = b0;
      key = key0;
    } else {
      g = 0;
      while (g + 1 < d.n_groups && s >= d.grp[g + 1].seq_base) ++g;
      b = s - d.grp[g].seq_base;
      key = d.scratch[s];
    }
    const GroupDesc& gd = d.grp[g];
    const int32_t pos = atomicAdd(&cursor[key], gd.num_heads);
    for (int h = 0; h < gd.num_heads; ++h) d.items[pos + h] = pack_item(g, h, b);
  }
}

hipError_t launch_schedule(const LaunchDesc& d, hipStream_t stream) {
  hipLaunchKernelGGL(build_schedule_kernel, dim3(1), dim3(kNumBuckets), 0, stream, d);
  return hipGetLastError();
}

// Debug validation: one workgroup checks every sequence of every group by the offsets rules and
// stores the OR of the error bits into the device error word (0 when all hold).
__global__ void __launch_bounds__(1024) validate_offsets_kernel(LaunchDesc d) {
  __shared__ int32_t bits;
  if (threadIdx.x == 0) bits = 0;
  __syncthreads();
  int32_t e = 0;
  for (int g = 0; g < d.n_groups; ++g) {
    const GroupDesc& gd = d.grp[g];
    OffsetsRules r;
    r.num_seqs = gd.num_seqs;
    r.self_attention = gd.self_attn;
    r.total_q = gd.total_q;
    r.total_kv = gd.total_kv;
    r.max_q = gd.max_q;
    r.max_kv = gd.max_kv;
    for (int b = threadIdx.x; b < gd.num_seqs; b += blockDim.x) e |= seq_offsets_error(r, gd.q_off, gd.kv_off, b);
  }
  if (e) atomicOr(&bits, e);
  __syncthreads();
  if (threadIdx.x == 0) *d.err = bits;
}

hipError_t launch_validate(const LaunchDesc& d, hipStream_t stream) {
  hipLaunchKernelGGL(validate_offsets_kernel, dim3(1), dim3(1024), 0, stream, d);
  return hipGetLastError();
}

// Clears the device error word (calls whose kernels do not start with the work-list builder).
__global__ void clear_error_kernel(int32_t* err) { *err = 0; }

hipError_t launch_clear_error(int32_t* err, hipStream_t stream) {
  hipLaunchKernelGGL(clear_error_kernel, dim3(1), dim3(1), 0, stream, err);
  return hipGetLastError();
}

}  // namespace gdpa
