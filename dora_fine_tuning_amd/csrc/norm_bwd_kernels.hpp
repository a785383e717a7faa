// Host-side plan and launch interface of the weight-norm backward (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lora_compose_kernels.hpp"
#include "norm_kernels.hpp"

namespace dora {

// Workspace layout of one norm-backward call: the norm plan's Gram region, c
// [out] fp32, Yhi | Ylo [out x 2r], Zhi | Zlo [r x 2r], and one region reused
// in turn by the W stream's partials, the slices of B^T Y, and the slices of
// d_A^T.  A pure function of (out, in, r, dtype).
struct NormBwdPlan {
  int64_t out = 0, in = 0, r = 0;
  bool vec = true;  // 16-byte MFMA path; else the general path (c, G, M in the workspace)
  NormPlan np;
  RowContractPlan rM, rW;  // B^T Y; [W0 ; A]^T [Y ; Z]
  size_t off_np = 0, off_c = 0, off_sigma = 0, off_y = 0, off_z = 0, off_big = 0, bytes = 0;
  int64_t max_grid = 0, max_slice_bytes = 0;
};

NormBwdPlan make_norm_bwd_plan(int64_t out, int64_t in, int64_t r, int dtype, bool vec);

// Workspace bytes covering both paths (the path depends on pointer alignment,
// known only at the call).
size_t norm_bwd_workspace_bytes(int64_t out, int64_t in, int64_t r, int dtype);

struct NormBwdArgs {
  int dtype;
  const void *W0, *A, *B;
  const float *norm, *d_norm;
  float s;
  void *d_A, *d_B;
  void* ws;
  hipStream_t stream;
};

// The 16-byte path (p.vec) needs in % 8 == 0, r % 8 == 0, in < 2^21, r <= 2^20
// and 16-byte aligned matrix and workspace pointers.
hipError_t launch_norm_bwd(const NormBwdPlan& p, const NormBwdArgs& a);

}  // namespace dora
