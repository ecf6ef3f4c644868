// Chunked WY/UT-form prefill (placeholder until the MFMA kernels land).
#include "common.h"
#include "internal.h"

namespace gdn {

size_t prefill_core_workspace(const Geometry &, int, int64_t) { return 0; }

hipError_t launch_prefill(const PrefillLaunch &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gdn
