// The policy-loss kernels' dtype dispatch, and the library's own scratch
// (the workspace of the entry point that allocates nothing).  The kernels
// themselves are in loss_kernels_impl.h, instantiated per input dtype by
// loss_kernels_{f32,f16,bf16}.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "loss_kernels.h"

namespace rlpl {

const void* pick_kernel(int dtype, int mode, bool has_kl, bool write_grad, int shape) {
    switch (dtype) {
    case kF32: return pick_typed<float>(mode, has_kl, write_grad, shape);
    case kF16: return pick_typed<_Float16>(mode, has_kl, write_grad, shape);
    case kBF16: return pick_typed<__bf16>(mode, has_kl, write_grad, shape);
    }
    return nullptr;
}

// ----------------------------------------------------------------------------- the library's own scratch

// The workspace of the entry point that allocates nothing: the header and the
// entry arrays of a Workspace (what the per-token kernels address), one copy
// per device, held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address comes from
// scratch_address(), per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

int scratch_address(void** out) {
    return hipGetSymbolAddress(out, HIP_SYMBOL(scratch)) == hipSuccess ? 0 : -1;
}

// Zero-fills n 16-byte words (the scratch's first use on a device).
__global__ void __launch_bounds__(kThreads) clear_kernel(uint4* p, uint32_t n) {
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}
const void* clear_kernel_ptr() { return reinterpret_cast<const void*>(&clear_kernel); }

}  // namespace rlpl
