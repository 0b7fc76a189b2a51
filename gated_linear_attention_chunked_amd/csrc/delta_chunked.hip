// delta_chunked.hip -- chunkwise-parallel delta-rule scan on gfx950 matrix
// cores.  Not built yet for any variant: the recurrent schedule serves.
#include "lam_internal.h"

namespace lam {

bool delta_chunked_supported(const DeltaArgs &) { return false; }

hipError_t launch_delta_chunked(const DeltaArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace lam
