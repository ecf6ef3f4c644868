// Instances of the token-recurrent kernel family for one mode (see
// recurrent_kernel.h); one translation unit per mode so they compile in parallel.
#include "recurrent_kernel.h"

namespace gdn {

hipError_t launch_rec_tokens(const RecurrentLaunch &p, hipStream_t stream) {
  return launch_rec_mode<17, kModeTokens>(p, stream);
}

}  // namespace gdn
