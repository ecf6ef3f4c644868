// Instances of the token-recurrent kernel family for one mode (see
// recurrent_kernel.h, and recurrent_wy.h for fp32 states at d >= 64); one
// translation unit per mode so they compile in parallel.
#include "recurrent_wy.h"

namespace gdn {

hipError_t launch_rec_woa(const RecurrentLaunch &p, hipStream_t stream) {
  return launch_woa(p, stream);
}

}  // namespace gdn
