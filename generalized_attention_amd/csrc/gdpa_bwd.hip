// Launchers of the bf16 backward kernels (the kernels themselves are in gdpa_bwd.hpp): the
// dispatch over kernel families, the short-key kernel and the shared-query dQ sum. Compiled with
// MFMA results in the VGPR form (no register-class copies between the accumulators and the
// element-wise code).
#include "gdpa_bwd.hpp"

namespace gdpa {

// Kernel families, each instantiated in a unit of its own so that the library builds in parallel:
// element-wise forms (gdpa_bwd_pw.hip) and the softmax form at d <= 64 (gdpa_bwd_sm.hip), both
// with MFMA results in the VGPR form; the softmax form at d = 128 or over several head dims
// (gdpa_bwd_agpr.hip) and launches holding every activation (gdpa_bwd_mix_*.hip) without it.
hipError_t launch_bwd_pointwise(const LaunchDesc& d, int dim_set, int act_set, hipStream_t stream);
hipError_t launch_bwd_softmax(const LaunchDesc& d, int dim_set, BwdSoftmaxForm form, hipStream_t stream);
hipError_t launch_bwd_softmax_agpr(const LaunchDesc& d, int dim_set, hipStream_t stream);
hipError_t launch_bwd_mixed_d32(const LaunchDesc& d, hipStream_t stream);
hipError_t launch_bwd_mixed_d64(const LaunchDesc& d, hipStream_t stream);
hipError_t launch_bwd_mixed_d128(const LaunchDesc& d, hipStream_t stream);
hipError_t launch_bwd_mixed_all(const LaunchDesc& d, hipStream_t stream);

// One instantiation per head-dim set and activation present: a launch with one element-wise
// activation runs a kernel without the softmax paths (and their registers); several head dims
// share the kernel that holds all three.
// softmax_form: the softmax-only launches at d <= 64 run 8 waves when the launch has no window or
// every window streams through the ring.
hipError_t launch_bwd_bf16(const LaunchDesc& d, int dim_set, int act_set, bool small, BwdSoftmaxForm softmax_form,
                           hipStream_t stream) {
  if (d.n_items == 0) return hipSuccess;
  constexpr int kGelu_ = 1 << GDPA_ACT_GELU, kSilu_ = 1 << GDPA_ACT_SILU;
  if (small) {
    // every sequence has at most 32 keys (element-wise forms, no window): one wave per item
    const dim3 sgrid((d.n_items + 3) / 4);
#define GDPA_SMALL(DS, AS) \
  hipLaunchKernelGGL((bwd_small_kernel<DS, AS>), sgrid, dim3(4 * kWave), (bwd_small_lds_bytes<DS>()), stream, d)
#define GDPA_SMALL_ACTS(DS)                                                      \
  if (act_set == kGelu_) GDPA_SMALL(DS, kGelu_);                                  \
  else if (act_set == kSilu_) GDPA_SMALL(DS, kSilu_);                             \
  else GDPA_SMALL(DS, kGelu_ | kSilu_);
    switch (dim_set) {
      case kDim32: GDPA_SMALL_ACTS(kDim32); break;
      case kDim64: GDPA_SMALL_ACTS(kDim64); break;
      case kDim128: GDPA_SMALL_ACTS(kDim128); break;
      default: GDPA_SMALL_ACTS(kDim32 | kDim64 | kDim128); break;
    }
#undef GDPA_SMALL_ACTS
#undef GDPA_SMALL
    return hipGetLastError();
  }
  constexpr int kSoftmax = 1 << GDPA_ACT_SOFTMAX;
  if (act_set == kGelu_ || act_set == kSilu_) return launch_bwd_pointwise(d, dim_set, act_set, stream);
  if (act_set == kSoftmax && (dim_set == kDim32 || dim_set == kDim64))
    return launch_bwd_softmax(d, dim_set, softmax_form, stream);
  if (act_set == kSoftmax) return launch_bwd_softmax_agpr(d, dim_set, stream);
  switch (dim_set) {
    case kDim32: return launch_bwd_mixed_d32(d, stream);
    case kDim64: return launch_bwd_mixed_d64(d, stream);
    case kDim128: return launch_bwd_mixed_d128(d, stream);
    default: return launch_bwd_mixed_all(d, stream);
  }
}

// ---- shared query matrix: dQ = scale * sum over sequences of their fp32 partial rows ----------
//
// Sequence b's partial rows sit at rows [b * S, b * S + L_b) of the workspace (S = shared_q); rows
// past L_b were never written and are skipped. Two deterministic stages: each thread of the first
// sums kSeqsPerSlot sequences of one 4-float column into the first sequence's slot (in place), the
// second sums those slots in sequence order and writes dq in bf16.
constexpr int kSeqsPerSlot = 8;

// (both stages return at once where the main kernels refused the launch: failed validation, or a
// planned call whose work list was built for other problems)
__device__ inline bool reduce_refused(const int32_t* err, int32_t check_err, int32_t plan_sig, int32_t check_plan) {
  return (check_err && err[0] != 0) || (check_plan && err[1] != plan_sig);
}

__global__ void __launch_bounds__(256) reduce_shared_dq_stage1(GroupDesc gd, const int32_t* err, int32_t check_err,
                                                               int32_t plan_sig, int32_t check_plan) {
  if (reduce_refused(err, check_err, plan_sig, check_plan)) return;
  const int S = gd.shared_q, rowf4 = gd.num_heads * gd.head_dim / 4;
  const int64_t cols = (int64_t)S * rowf4;
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= cols) return;
  const int s = (int)(col / rowf4);
  f32x4* part = reinterpret_cast<f32x4*>(gd.dq32);
  for (int b0 = blockIdx.y * kSeqsPerSlot; b0 < gd.num_seqs; b0 += gridDim.y * kSeqsPerSlot) {
    f32x4 v[kSeqsPerSlot];
#pragma unroll
    for (int i = 0; i < kSeqsPerSlot; ++i) {
      const int b = b0 + i;
      v[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (b < gd.num_seqs && s < gd.q_off[b + 1] - gd.q_off[b]) v[i] = part[(int64_t)b * cols + col];
    }
    f32x4 acc = v[0];
#pragma unroll
    for (int i = 1; i < kSeqsPerSlot; ++i) acc += v[i];
    part[(int64_t)b0 * cols + col] = acc;
  }
}

__global__ void __launch_bounds__(256) reduce_shared_dq_stage2(GroupDesc gd, const int32_t* err, int32_t check_err,
                                                               int32_t plan_sig, int32_t check_plan) {
  if (reduce_refused(err, check_err, plan_sig, check_plan)) return;
  const int S = gd.shared_q, rowf4 = gd.num_heads * gd.head_dim / 4;
  const int64_t cols = (int64_t)S * rowf4;
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= cols) return;
  const f32x4* part = reinterpret_cast<const f32x4*>(gd.dq32);
  f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // the same sequence order as one slot at a time, with four slots' loads in flight together
  int b0 = 0;
  for (; b0 + 4 * kSeqsPerSlot <= gd.num_seqs; b0 += 4 * kSeqsPerSlot) {
    f32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = part[(int64_t)(b0 + i * kSeqsPerSlot) * cols + col];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += v[i];
  }
  for (; b0 < gd.num_seqs; b0 += kSeqsPerSlot) acc += part[(int64_t)b0 * cols + col];
  out_store4(out_ptr(gd.dq, gd.out_f32, (size_t)col * 4), acc * gd.scale);
}

hipError_t launch_reduce_shared_dq(const LaunchDesc& d, const GroupDesc& gd, hipStream_t stream) {
  const int64_t cols = (int64_t)gd.shared_q * gd.num_heads * gd.head_dim / 4;
  if (cols == 0) return hipSuccess;
  const unsigned nx = (unsigned)((cols + 255) / 256);
  if (gd.num_seqs > 0) {
    const int slots = (gd.num_seqs + kSeqsPerSlot - 1) / kSeqsPerSlot;
    const unsigned ny = (unsigned)(slots < 65535 ? slots : 65535);
    hipLaunchKernelGGL(reduce_shared_dq_stage1, dim3(nx, ny), dim3(256), 0, stream, gd, d.err, d.check_err,
                       d.plan_sig, d.check_plan);
  }
  hipLaunchKernelGGL(reduce_shared_dq_stage2, dim3(nx), dim3(256), 0, stream, gd, d.err, d.check_err, d.plan_sig,
                     d.check_plan);
  return hipGetLastError();
}

}  // namespace gdpa
