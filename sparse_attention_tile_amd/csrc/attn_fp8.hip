// fp8 (OCP e4m3fn) GNA attention: not built yet; the launcher reports the
// dtype as unsupported so callers get NA_ERR_UNSUPPORTED.
#include <hip/hip_runtime.h>

#include "attn_common.hpp"

namespace na {

bool attn_fp8_supported(int, int, int) { return false; }

hipError_t launch_attn_fp8(const AttnArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace na
