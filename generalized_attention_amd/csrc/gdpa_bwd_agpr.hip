// Backward kernels compiled with the default (accumulation-register) form of the MFMA results:
// the launches that carry the softmax form at d = 128 or every activation at once, whose register
// demand the VGPR-form build of gdpa_bwd.hip does not handle.
#include "gdpa_bwd.hpp"

namespace gdpa {

hipError_t launch_bwd_bf16_agpr(const LaunchDesc& d, int dim_set, int act_set, hipStream_t stream) {
  if (d.n_items == 0) return hipSuccess;
  const dim3 grid(d.n_items);
  constexpr int kAll = (1 << GDPA_ACT_GELU) | (1 << GDPA_ACT_SILU) | (1 << GDPA_ACT_SOFTMAX);
  constexpr int kDimAll = kDim32 | kDim64 | kDim128;
#define GDPA_LAUNCH(DS, AS) \
  hipLaunchKernelGGL((bwd_bf16_kernel<DS, AS>), grid, dim3((bwd_waves<DS, AS>() * kWave)), (bwd_lds_bytes<DS, AS>()), stream, d)
  if (act_set == 1 << GDPA_ACT_SOFTMAX) {
    if (dim_set == kDim128) GDPA_LAUNCH(kDim128, 1 << GDPA_ACT_SOFTMAX);
    else GDPA_LAUNCH(kDimAll, 1 << GDPA_ACT_SOFTMAX);
  } else {
    switch (dim_set) {
      case kDim32: GDPA_LAUNCH(kDim32, kAll); break;
      case kDim64: GDPA_LAUNCH(kDim64, kAll); break;
      case kDim128: GDPA_LAUNCH(kDim128, kAll); break;
      default: GDPA_LAUNCH(kDimAll, kAll); break;
    }
  }
#undef GDPA_LAUNCH
  return hipGetLastError();
}

}  // namespace gdpa
