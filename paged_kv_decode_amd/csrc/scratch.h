// scratch.h -- the fixed device scratch of pa_decode_run_noalloc.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace pa {

// Bytes of the per-device scratch array (partition states of one call).
constexpr size_t kScratchBytes = size_t(64) << 20;

// Device address of `device`'s scratch array, looked up on the first call
// for that device (with the device made current, then restored) and kept.
hipError_t scratch_address(int device, void** ptr);

}  // namespace pa
