// Scratch of the entry point that allocates nothing (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace dora {

// Size of the per-device scratch array: the magnitude-gradient partials of
// dora_compose_bwd at up to 24 MiB (every workload module here fits; the
// 27648-column, 10240-token one needs 17.7 MB).
constexpr size_t kNoAllocScratchBytes = size_t(24) << 20;

// Device address of the scratch array on the device of `stream`, looked up
// once per device (hipGetSymbolAddress with that device current).
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

}  // namespace dora
