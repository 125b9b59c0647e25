// Launchers of the bf16 backward kernels (the kernels themselves are in gdpa_bwd.hpp).
//
// This translation unit is compiled with MFMA results in the VGPR form, which keeps the score
// accumulators next to the element-wise code (no register-class copies in the inner loop). The
// d = 128 softmax-only kernel is built in its own unit without that option.
#include "gdpa_bwd.hpp"

namespace gdpa {

hipError_t launch_bwd_bf16_d128_softmax(const LaunchDesc& d, hipStream_t stream);

hipError_t launch_bwd_bf16(const LaunchDesc& d, int dim_set, int act_set, hipStream_t stream) {
  if (d.n_items == 0) return hipSuccess;
  const dim3 grid(d.n_items);
  constexpr int kAll = (1 << GDPA_ACT_GELU) | (1 << GDPA_ACT_SILU) | (1 << GDPA_ACT_SOFTMAX);
#define GDPA_LAUNCH(DS, AS) \
  hipLaunchKernelGGL((bwd_bf16_kernel<DS, AS>), grid, dim3(kBwdWaves * kWave), bwd_lds_bytes<DS>(), stream, d)
#define GDPA_LAUNCH_ACTS(DS)                                                   \
  switch (act_set) {                                                           \
    case 1 << GDPA_ACT_GELU: GDPA_LAUNCH(DS, 1 << GDPA_ACT_GELU); break;       \
    case 1 << GDPA_ACT_SILU: GDPA_LAUNCH(DS, 1 << GDPA_ACT_SILU); break;       \
    case 1 << GDPA_ACT_SOFTMAX: GDPA_LAUNCH(DS, 1 << GDPA_ACT_SOFTMAX); break; \
    default: GDPA_LAUNCH(DS, kAll); break;                                     \
  }
  switch (dim_set) {
    case kDim32: GDPA_LAUNCH_ACTS(kDim32); break;
    case kDim64: GDPA_LAUNCH_ACTS(kDim64); break;
    case kDim128:
      switch (act_set) {
        case 1 << GDPA_ACT_GELU: GDPA_LAUNCH(kDim128, 1 << GDPA_ACT_GELU); break;
        case 1 << GDPA_ACT_SILU: GDPA_LAUNCH(kDim128, 1 << GDPA_ACT_SILU); break;
        case 1 << GDPA_ACT_SOFTMAX: return launch_bwd_bf16_d128_softmax(d, stream);
        default: GDPA_LAUNCH(kDim128, kAll); break;
      }
      break;
    case kDim32 | kDim128: GDPA_LAUNCH(kDim32 | kDim128, kAll); break;
    default: GDPA_LAUNCH(kDim32 | kDim64 | kDim128, kAll); break;
  }
#undef GDPA_LAUNCH_ACTS
#undef GDPA_LAUNCH
  return hipGetLastError();
}

}  // namespace gdpa
