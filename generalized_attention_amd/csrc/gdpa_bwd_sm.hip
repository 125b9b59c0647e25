// Backward launches of the softmax form at one head dim <= 64 (compiled with MFMA results in the
// VGPR form): 8 waves per workgroup when the launch has no window (kBwdWideSoftmax) or every
// window streams through the ring (kBwdRingSoftmax), else 4 waves with every sweep.
#include "gdpa_bwd.hpp"

namespace gdpa {

hipError_t launch_bwd_softmax(const LaunchDesc& d, int dim_set, BwdSoftmaxForm form, hipStream_t stream) {
  const dim3 grid(d.n_items);
  constexpr int kSoftmax = 1 << GDPA_ACT_SOFTMAX;
  constexpr int kWide = kSoftmax | kBwdWideSoftmax, kRing = kSoftmax | kBwdRingSoftmax;
#define GDPA_LAUNCH(DS, AS) \
  hipLaunchKernelGGL((bwd_bf16_kernel<DS, AS>), grid, dim3((bwd_waves<DS, AS>() * kWave)), (bwd_lds_bytes<DS, AS>()), stream, d)
  if (dim_set == kDim32) {
    if (form == kSoftmaxNoWindow) GDPA_LAUNCH(kDim32, kWide);
    else if (form == kSoftmaxRingWindow) GDPA_LAUNCH(kDim32, kRing);
    else GDPA_LAUNCH(kDim32, kSoftmax);
  } else {
    if (form == kSoftmaxNoWindow) GDPA_LAUNCH(kDim64, kWide);
    else if (form == kSoftmaxRingWindow) GDPA_LAUNCH(kDim64, kRing);
    else GDPA_LAUNCH(kDim64, kSoftmax);
  }
#undef GDPA_LAUNCH
  return hipGetLastError();
}

}  // namespace gdpa
