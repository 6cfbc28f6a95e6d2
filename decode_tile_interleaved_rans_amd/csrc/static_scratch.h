// The device's static scratch array of the no-allocation forward (static_scratch.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace ep {

// One array per device, alive until the process ends, shared by every no-allocation call on it.
constexpr size_t kStaticScratchBytes = 64u << 20;

// Device address of the current device's array (resolved once per device).
hipError_t static_scratch(void** ptr);

}  // namespace ep
