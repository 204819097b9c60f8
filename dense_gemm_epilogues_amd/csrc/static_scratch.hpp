// Scratch of the allocation-free entry point (static_scratch.hip): a static device array of
// 64 MiB per device.
#pragma once
#include <hip/hip_runtime.h>

#include <stddef.h>

namespace ep {

constexpr size_t kStaticScratchBytes = size_t(64) << 20;
// device address and size of the scratch on `dev` (the current device), looked up once per device
hipError_t static_scratch(int dev, void** ptr, size_t* bytes);

}  // namespace ep
