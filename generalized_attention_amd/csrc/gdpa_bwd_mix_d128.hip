// Backward launches that hold several activations (per-head activations, or groups with
// different ones) at head dims 128, compiled with the default (accumulation-register) form of
// the MFMA results. (One unit per head-dim set, so that they compile in parallel.)
#include "gdpa_bwd.hpp"

namespace gdpa {

hipError_t launch_bwd_mixed_d128(const LaunchDesc& d, hipStream_t stream) {
  constexpr int kAll = (1 << GDPA_ACT_GELU) | (1 << GDPA_ACT_SILU) | (1 << GDPA_ACT_SOFTMAX);
  constexpr int DS = kDim128;
  hipLaunchKernelGGL((bwd_bf16_kernel<DS, kAll>), dim3(d.n_items), dim3((bwd_waves<DS, kAll>() * kWave)),
                     (bwd_lds_bytes<DS, kAll>()), stream, d);
  return hipGetLastError();
}

}  // namespace gdpa
