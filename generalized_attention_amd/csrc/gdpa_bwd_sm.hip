// Backward launches of the softmax form at one head dim <= 64 (compiled with MFMA results in the
// VGPR form). wide_softmax: no window, 8 waves per workgroup.
#include "gdpa_bwd.hpp"

namespace gdpa {

hipError_t launch_bwd_softmax(const LaunchDesc& d, int dim_set, bool wide_softmax, hipStream_t stream) {
  const dim3 grid(d.n_items);
  constexpr int kSoftmax = 1 << GDPA_ACT_SOFTMAX;
#define GDPA_LAUNCH(DS, AS) \
  hipLaunchKernelGGL((bwd_bf16_kernel<DS, AS>), grid, dim3((bwd_waves<DS, AS>() * kWave)), (bwd_lds_bytes<DS, AS>()), stream, d)
  if (dim_set == kDim32) {
    if (wide_softmax) {
      GDPA_LAUNCH(kDim32, (kSoftmax | kBwdWideSoftmax));
    } else {
      GDPA_LAUNCH(kDim32, kSoftmax);
    }
  } else {
    if (wide_softmax) {
      GDPA_LAUNCH(kDim64, (kSoftmax | kBwdWideSoftmax));
    } else {
      GDPA_LAUNCH(kDim64, kSoftmax);
    }
  }
#undef GDPA_LAUNCH
  return hipGetLastError();
}

}  // namespace gdpa
