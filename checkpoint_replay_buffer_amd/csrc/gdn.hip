// gdn.hip -- Gated DeltaNet ReplaySSM decode kernels for gfx950 (no shapes compiled yet).
#include "dev_common.h"
#include "internal.h"

namespace rssm {

bool gdn_supported(int, int) { return false; }
hipError_t gdn_decode(const GdnStepArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t gdn_fold(const GdnFoldArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t gdn_rmw(const GdnRmwArgs &, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace rssm
