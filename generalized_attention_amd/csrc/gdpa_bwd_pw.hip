// Backward launches with one element-wise activation (compiled with MFMA results in the VGPR
// form).
#include "gdpa_bwd.hpp"

namespace gdpa {

hipError_t launch_bwd_pointwise(const LaunchDesc& d, int dim_set, int act_set, hipStream_t stream) {
  const dim3 grid(d.n_items);
  constexpr int kDimAll = kDim32 | kDim64 | kDim128;
  constexpr int kGelu = 1 << GDPA_ACT_GELU, kSilu = 1 << GDPA_ACT_SILU;
#define GDPA_LAUNCH(DS, AS) \
  hipLaunchKernelGGL((bwd_bf16_kernel<DS, AS>), grid, dim3((bwd_waves<DS, AS>() * kWave)), (bwd_lds_bytes<DS, AS>()), stream, d)
#define GDPA_LAUNCH_DIMS(AS)                            \
  switch (dim_set) {                                    \
    case kDim32: GDPA_LAUNCH(kDim32, AS); break;        \
    case kDim64: GDPA_LAUNCH(kDim64, AS); break;        \
    case kDim128: GDPA_LAUNCH(kDim128, AS); break;      \
    default: GDPA_LAUNCH(kDimAll, AS); break;           \
  }
  if (act_set == kGelu) {
    GDPA_LAUNCH_DIMS(kGelu);
  } else {
    GDPA_LAUNCH_DIMS(kSilu);
  }
#undef GDPA_LAUNCH_DIMS
#undef GDPA_LAUNCH
  return hipGetLastError();
}

}  // namespace gdpa
