// MFMA tiled attention kernel (placeholder until the tiled path lands).
#include "olk_internal.h"

namespace olk {

bool tiled_supports(const Params &, int) { return false; }

hipError_t launch_tiled(const Params &, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace olk
