// noalloc.h - the fixed scratch buffer of the allocation-free decode step.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace hsa {

// Bytes of the fixed scratch buffer: one copy per GPU, allocated when the library's
// device code is loaded on that GPU and kept until the process ends.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;

// Device address of `device`'s copy of the buffer (`device` must be current). Looked
// up once per device; later calls return the same address.
hipError_t noalloc_scratch(int device, void** ptr);

}  // namespace hsa
