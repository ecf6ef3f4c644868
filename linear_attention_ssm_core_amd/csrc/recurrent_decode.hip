// Instances of the token-recurrent kernel family for one mode (see
// recurrent_kernel.h); one translation unit per mode so they compile in parallel.
// This one also holds the dispatch over the modes.
#include "recurrent_kernel.h"

namespace gdn {

hipError_t launch_rec_decode(const RecurrentLaunch &p, hipStream_t stream) {
  return launch_rec_mode<1, kModeDecode>(p, stream);
}

hipError_t launch_recurrent(const RecurrentLaunch &p, hipStream_t stream) {
  switch (p.mode) {
    case kModeDecode: return launch_rec_decode(p, stream);
    case kModeTokens: return launch_rec_tokens(p, stream);
    case kModeVerify: return launch_rec_verify(p, stream);
    case kModeWoa: return launch_rec_woa(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
