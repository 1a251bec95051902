// pa_mfma.hip -- matrix-core decode kernel (placeholder until implemented).
#include "pa_launch.h"

namespace pa {

bool mfma_supported(int, int) { return false; }

hipError_t launch_mfma(const DecodeParams&, int, int, bool, hipStream_t) {
    return hipErrorInvalidValue;
}

}  // namespace pa
