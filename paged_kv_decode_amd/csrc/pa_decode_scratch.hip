// pa_decode_scratch.hip -- the fixed device scratch of pa_decode_run_noalloc.
//
// One file-scope device array per GPU, loaded with the library's code object
// and held until the process ends.  Host code never passes the array's name
// to a kernel or a copy: in host code that name stands for a host-side
// handle, not a device address.  The device address is looked up once per
// device with hipGetSymbolAddress, with that device current (at
// pa_decode_create, the library's set-up call), and that address is what the
// kernels receive as their workspace.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>

#include "scratch.h"

namespace pa {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_address(int device, void** ptr)
{
    if (!ptr || device < 0 || device >= kMaxDevices)
        return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_addr[device]) {
        int prev = -1;
        hipError_t e = hipGetDevice(&prev);
        if (e == hipSuccess) e = hipSetDevice(device);
        void* p = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (prev >= 0) (void)hipSetDevice(prev);
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        scratch_addr[device] = p;
    }
    *ptr = scratch_addr[device];
    return hipSuccess;
}

}  // namespace pa
