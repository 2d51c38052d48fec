// kvq_decode_mfma.hip -- matrix-core decode kernel (gfx950).  Not built yet:
// the library reports the MFMA variant as unsupported for every group size.
#include "kvq_internal.hpp"

namespace kvq {

bool mfma_supports(int) { return false; }

hipError_t launch_decode_mfma(const DecodeArgs &, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kvq
