// SSD (Mamba-2) chunked forward for gfx950 -- kernel under construction.
#include <hip/hip_runtime.h>

#include "ssm_internal.h"

namespace ssm {

hipError_t launch_ssd(const SSDArgs& a, hipStream_t stream) {
    (void)a;
    (void)stream;
    return hipErrorNotSupported;
}

}  // namespace ssm
