// The bf16 forward launch that builds every key path (resident keys, ring window, key chunks).
#include "gdpa_fwd.hpp"

namespace gdpa {

hipError_t launch_fwd_bf16_any(const LaunchDesc& d, int dim_set, int act_set, hipStream_t stream) {
  return launch_fwd_bf16_t<kFwdAny>(d, dim_set, act_set, stream);
}

}  // namespace gdpa
