// Host-side launch interface of the compose kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dora {

// Tokens per block of the backward; one fp32 partial of the magnitude gradient
// per (token block, column) lives in the workspace.  64 rows, or 16 when 64-row
// blocks would give fewer than 512 workgroups (a small module would leave CUs
// idle).  A function of (T, out) only, so the workspace query and the launch
// agree whatever path the pointers select.
constexpr int kBwdRowsWide = 64, kBwdRowsNarrow = 16;
int compose_bwd_rows(int64_t T, int64_t out);
size_t compose_bwd_workspace(int64_t T, int64_t out);

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
