// Backward launches of the softmax form at d = 128 or over several head dims, compiled with the
// default (accumulation-register) form of the MFMA results: the VGPR-form build does not handle
// their register demand.
#include "gdpa_bwd.hpp"

namespace gdpa {

hipError_t launch_bwd_softmax_agpr(const LaunchDesc& d, int dim_set, hipStream_t stream) {
  const dim3 grid(d.n_items);
  constexpr int kDimAll = kDim32 | kDim64 | kDim128;
  constexpr int kSoftmax = 1 << GDPA_ACT_SOFTMAX;
#define GDPA_LAUNCH(DS, AS) \
  hipLaunchKernelGGL((bwd_bf16_kernel<DS, AS>), grid, dim3((bwd_waves<DS, AS>() * kWave)), (bwd_lds_bytes<DS, AS>()), stream, d)
  if (dim_set == kDim128) GDPA_LAUNCH(kDim128, kSoftmax);
  else GDPA_LAUNCH(kDimAll, kSoftmax);
#undef GDPA_LAUNCH
  return hipGetLastError();
}

}  // namespace gdpa
