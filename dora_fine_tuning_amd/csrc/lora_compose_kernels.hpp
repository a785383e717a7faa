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

struct LoraBwdArgs {
  int dtype;
  int64_t T, out, r;
  float s;
  int add_base;
  const void *dy, *base, *h, *B;
  const float *mag, *norm;
  void* d_base;  // may be null
  void* d_B;
  float* d_mag;
  void* ws;
  hipStream_t stream;
};

// Workspace of the 16-byte path (the E slices and the column partials).
size_t lora_bwd_workspace_bytes(int64_t T, int64_t out, int64_t r);
int64_t lora_bwd_max_grid(int64_t T, int64_t out, int64_t r, bool vec);
// Largest byte range one token slice's buffer resource spans (must stay below 2^31).
int64_t lora_bwd_max_slice_bytes(int64_t T, int64_t out, int64_t r);

// vec: out % 8 == 0, r % 8 == 0, 1 <= r <= 2^20, T >= 1, every pointer 16-byte aligned.
hipError_t launch_lora_bwd(const LoraBwdArgs& a, bool vec);

// Plain contraction over the row (token) axis of two row-major matrices of the
// storage dtype, X [T x nx] and Y [T x ny] with row pitch ldy: E = X^T Y,
// computed in nSplit row slices whose fp32 partials are written to
// e_part[nSplit][nx][ny] (the caller adds them).  With dual, Y's rows hold a
// second block of ny columns at column ny (ldy >= 2 ny) that adds into the same
// E: E = X^T (Y[:, :ny] + Y[:, ny:2ny]).  With T2 > 0 the contraction axis
// continues over the rows of X2 [T2 x nx] and Y2 [T2 x ny] (pitch ldy), spread
// evenly over the same slices.  Needs nx, ny, ldy multiples of 8, 16-byte
// aligned X, Y, X2, Y2 and e_part, and slice_bytes < 2^31.
struct RowContractPlan {
  int nSplit = 0;            // row slices
  size_t bytes = 0;          // of e_part
  int64_t grid = 0;          // workgroups of the launch
  int64_t slice_bytes = 0;   // largest byte range one slice's buffer resource spans
};
RowContractPlan row_contract_plan(int64_t T, int64_t nx, int64_t ny, int64_t T2, int64_t ldy);
hipError_t launch_row_contract(const void* X, const void* Y, int64_t T, int64_t nx, int64_t ny, int64_t ldy, bool dual,
                               int dtype, float* e_part, hipStream_t stream, const void* X2 = nullptr,
                               const void* Y2 = nullptr, int64_t T2 = 0);

}  // namespace dora
