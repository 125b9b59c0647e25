// The d = 128 softmax-only backward kernel, compiled without the VGPR-form MFMA option used for
// the other backward kernels.
#include "gdpa_bwd.hpp"

namespace gdpa {

hipError_t launch_bwd_bf16_d128_softmax(const LaunchDesc& d, hipStream_t stream) {
  if (d.n_items == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_bf16_kernel<kDim128, 1 << GDPA_ACT_SOFTMAX>), dim3(d.n_items), dim3(kBwdWaves * kWave),
                     bwd_lds_bytes<kDim128>(), stream, d);
  return hipGetLastError();
}

}  // namespace gdpa
