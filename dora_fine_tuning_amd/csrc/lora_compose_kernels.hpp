// Host-side launch interface of the fused lora-projection compose (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dora {

struct LoraFwdArgs {
  int dtype;
  int64_t T, out, r;
  float s;
  int add_base;
  const void *base, *h, *B;
  const float *mag, *norm;
  void* y;
  hipStream_t stream;
};

// Largest grid (workgroups in one dimension) the launch uses.
int64_t lora_fwd_max_grid(int64_t T, int64_t out, bool vec);

// vec: out % 8 == 0, r % 8 == 0, r <= 2^20 and every pointer 16-byte aligned.
hipError_t launch_lora_fwd(const LoraFwdArgs& a, bool vec);

}  // namespace dora
