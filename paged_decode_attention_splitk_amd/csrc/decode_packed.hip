// GQA-packed decode kernel (placeholder until the MFMA kernel lands).
#include <hip/hip_runtime.h>

#include "pda_kernels.h"

namespace pda {

hipError_t launch_packed(const PackedParams&, uint32_t, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace pda
