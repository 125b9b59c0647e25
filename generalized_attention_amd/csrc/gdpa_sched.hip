// Jagged work decomposition: one workgroup builds the longest-first list of
// (group, head, sequence) work items from the device offsets.
//
// The pages name tile scheduling over jagged, large-batch inputs as one of the GDPA kernel's
// levers (Kunlun review, section 2.3). Here a work item is one whole (sequence, head) pair; the
// main kernels take items in list order, one workgroup per item, and the hardware dispatcher
// hands the next item to whichever compute unit frees up first, so a longest-first order gives
// the classic LPT balance without a persistent kernel or atomics in the main kernels.
#include "gdpa_device.hpp"
#include "gdpa_launch.hpp"

namespace gdpa {

// Launched with exactly kNumBuckets threads (one per bucket in the scan).
__global__ void __launch_bounds__(kNumBuckets) build_schedule_kernel(LaunchDesc d) {
  __shared__ int32_t hist[kNumBuckets];
  __shared__ int32_t cursor[kNumBuckets];
  const int tid = threadIdx.x;
  for (int i = tid; i < kNumBuckets; i += blockDim.x) hist[i] = 0;
  __syncthreads();

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
    d.scratch[s] = (int32_t)key;
    atomicAdd(&hist[key], gd.num_heads);
  }
  __syncthreads();
  // exclusive prefix sum in descending bucket order (longest work first): thread t owns bucket
  // kNumBuckets-1-t; Hillis-Steele scan over the 1024 buckets in LDS.
  {
    const int k = kNumBuckets - 1 - tid;
    int32_t v = hist[k];
    cursor[tid] = v;
    __syncthreads();
    for (int off = 1; off < kNumBuckets; off <<= 1) {
      const int32_t add = tid >= off ? cursor[tid - off] : 0;
      __syncthreads();
      cursor[tid] += add;
      __syncthreads();
    }
    const int32_t excl = cursor[tid] - v;
    __syncthreads();
    hist[k] = excl;  // hist now holds the start position of each bucket
    __syncthreads();
    cursor[k] = excl;
  }
  __syncthreads();
  for (int s = tid; s < d.n_seqs_total; s += blockDim.x) {
    int g = 0;
    while (g + 1 < d.n_groups && s >= d.grp[g + 1].seq_base) ++g;
    const GroupDesc& gd = d.grp[g];
    const int b = s - gd.seq_base;
    const int32_t key = d.scratch[s];
    const int32_t pos = atomicAdd(&cursor[key], gd.num_heads);
    for (int h = 0; h < gd.num_heads; ++h) d.items[pos + h] = pack_item(g, h, b);
  }
}

hipError_t launch_schedule(const LaunchDesc& d, hipStream_t stream) {
  hipLaunchKernelGGL(build_schedule_kernel, dim3(1), dim3(kNumBuckets), 0, stream, d);
  return hipGetLastError();
}

}  // namespace gdpa
