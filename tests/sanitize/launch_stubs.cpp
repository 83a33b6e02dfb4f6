// Kernel-launch stand-ins for the host-only sanitizer build of the C-ABI
// layer.  The fuzz driver makes every call fail validation, so none of these
// may be reached: each one reports the call and aborts the driver.
#include <stdio.h>
#include <stdlib.h>

#include "ssm_internal.h"

namespace {
[[noreturn]] void reached(const char* what) {
    fprintf(stderr, "validation let a call through to %s\n", what);
    abort();
}
}  // namespace

namespace ssm {
hipError_t launch_s6(const S6Args&, hipStream_t) { reached("launch_s6"); }
hipError_t noalloc_scratch(void**) { reached("noalloc_scratch"); }
hipError_t launch_ssd(const SSDArgs&, hipStream_t) { reached("launch_ssd"); }
hipError_t launch_s6_step(const StepArgs&, hipStream_t) { reached("launch_s6_step"); }
hipError_t launch_s6_bwd(const S6BwdArgs&, hipStream_t) { reached("launch_s6_bwd"); }
hipError_t launch_s6_bwd_ckpt(const S6BwdArgs&, hipStream_t) { reached("launch_s6_bwd_ckpt"); }
hipError_t launch_conv1d(const ConvArgs&, hipStream_t) { reached("launch_conv1d"); }
}  // namespace ssm
