// Host-side launch interface of the compose kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dora {

// Tokens per block of the backward; one fp32 partial of the magnitude gradient
// per (token block, column) lives in the workspace.
constexpr int kBwdRows = 64;

struct ComposeArgs {
  int dtype;
  int64_t T, out;
  float s;
  int add_base;
  const float* mag;
  const float* norm;
  // forward
  const void* base;
  const void* lora;
  void* y;
  // backward
  const void* dy;
  void* d_lora;
  void* d_base;
  float* d_mag;
  float* partial;
  hipStream_t stream;
};

hipError_t launch_compose_fwd(const ComposeArgs& a, bool vec);
hipError_t launch_compose_bwd(const ComposeArgs& a, bool vec);

// Largest grid (workgroups in one dimension) the launches of these sizes use;
// the caller rejects sizes whose grid would exceed the launch limit.
int64_t compose_max_grid(int64_t T, int64_t out, bool vec);

}  // namespace dora
