// Launchers of the bf16 forward kernels (the kernels are in gdpa_fwd.hpp). The launch mode that
// builds every path (kFwdAny) is instantiated in gdpa_fwd_any.hip, so the two units compile in
// parallel.
#include "gdpa_fwd.hpp"

namespace gdpa {

hipError_t launch_fwd_bf16_any(const LaunchDesc& d, int dim_set, int act_set, hipStream_t stream);

hipError_t launch_fwd_bf16(const LaunchDesc& d, int dim_set, int act_set, int key_mode, hipStream_t stream) {
  if (d.n_items == 0) return hipSuccess;
  if (key_mode == kFwdResident) return launch_fwd_bf16_t<kFwdResident>(d, dim_set, act_set, stream);
  if (key_mode == kFwdLong8) return launch_fwd_bf16_t<kFwdLong8>(d, dim_set, act_set, stream);
  return launch_fwd_bf16_any(d, dim_set, act_set, stream);
}

}  // namespace gdpa
