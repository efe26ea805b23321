// cbs_noalloc.hip -- the device-resident scratch of the entry point that
// allocates nothing (conv_bn_silu_run_unfused_noalloc): the two
// intermediates of the unfused sequence live in a static device array of
// fixed size, one copy per GPU, held until the process ends.
#include <hip/hip_runtime.h>

#include "cbs_launch.h"

namespace cbs {
namespace {

// t1 in the first half, t2 in the second.  Every element a call reads is
// written earlier in the same call, so nothing needs clearing between calls.
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

}  // namespace

// The device address of `scratch` on the current device.  In host code the
// array's name is only a host-side stand-in; kernels must be given this
// address.  Called once per device, when a handle is created on it.
hipError_t noalloc_scratch_address(void **out) { return hipGetSymbolAddress(out, HIP_SYMBOL(scratch)); }

}  // namespace cbs
