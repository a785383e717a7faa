// Host-side plan and launch interface of the factored-norm kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dora {

// Work decomposition and workspace layout of one factored-norm call.  A pure
// function of (out, in, r, dtype, path), so the workspace query and the launch
// agree.  vec selects the 16-byte path (direct global->LDS loads).
struct NormPlan {
  int64_t out = 0, in = 0, r = 0;
  int dtype = 0;
  bool vec = false;
  int tn = 0;  // 16-byte path: rank tile width 128*tn
  // fused W stream: row blocks x rank tiles x K splits over the augmented K axis
  int64_t nRB = 0;
  int nTiles = 0;
  int64_t S1 = 0, S2 = 0, S = 0;  // K stages: W0.A^T part, each B.G' part, total
  int nSplit = 0;
  // Gram: upper-triangular tiles per side (64 rows on the 16-byte path, 32
  // otherwise) x K splits
  int nTg = 0, splitG = 0;
  // one K split and no fp32 partial region: the Gram kernel writes G'hi/G'lo
  // directly (chosen when the partials would not fit the scratch bound)
  bool gram_direct = false;
  // small adapter (r <= kStripMaxRank, enough row strips): one launch of the
  // strip kernel, each workgroup taking 32 rows over the whole input axis and
  // forming the Gram matrix itself; no workspace is used
  bool strip = false;
  // workspace byte offsets
  size_t off_gpart = 0, off_ghi = 0, off_glo = 0, off_base = 0, off_cross = 0, off_count = 0, bytes = 0;
};

// store_acc: the plan of the norm backward's W stream, which stores every K
// split's accumulators (fewer splits).
NormPlan make_norm_plan(int64_t out, int64_t in, int64_t r, int dtype, bool vec, bool store_acc = false);

// The strip kernel (16-byte path): ranks up to 32, at least kStripMinBlocks
// strips of 32 rows, panels within 32-bit buffer offsets.
constexpr int64_t kStripMaxRank = 32;
constexpr int64_t kStripMinBlocks = 128;
inline int64_t cdiv_strip(int64_t out) { return (out + 31) / 32; }
bool norm_strip_fits(int64_t out, int64_t in, int64_t r);

// Largest grid (workgroups in one dimension) the launches of this plan use.
int64_t norm_max_grid(const NormPlan& p);

// Workspace bytes covering both paths (the path depends on pointer alignment,
// known only at the call).
size_t norm_workspace_bytes(int64_t out, int64_t in, int64_t r, int dtype);

// The factored memory bound 4*(out*r + r*r) + 64*out bytes (region
// alignment included).
size_t norm_scratch_bound(int64_t out, int64_t r);

struct NormArgs {
  const void* W0;
  const void* A;
  const void* B;
  float s;
  float* norm_out;
  void* ws;
  hipStream_t stream;
  const float* base_sq = nullptr;  // cached ||W0_i||^2 [out]; the W stream then skips the base term
};

hipError_t launch_norm(const NormPlan& p, const NormArgs& a);
hipError_t launch_norm_strip(const NormPlan& p, const NormArgs& a);

// sq[i] = ||W0_i||^2 in fp32 (vec: in % 8 == 0 and W0 16-byte aligned); grid cdiv(out, 4).
hipError_t launch_row_sqnorm(const void* W0, int64_t out, int64_t in, int dtype, bool vec, float* sq,
                             hipStream_t stream);

// Norm backward, the d_B half (16-byte path plans only):
//   d_B_i = s * c_i * (U_i + s * B_i G),  U = W0 A^T, G = A A^T,
// by the W stream over [W0 | B | B] . [A | G'hi | G'lo]^T with G' = s G, whose
// split-K accumulators go to acc_part (norm_bwd_acc_bytes(p) bytes) and are
// then added and scaled.  ws: the plan's workspace (its Gram regions are used).
size_t norm_bwd_acc_bytes(const NormPlan& p);
hipError_t launch_norm_bwd_db(const NormPlan& p, const void* W0, const void* A, const void* B, float s,
                              const float* c, void* dB, void* ws, float* acc_part, hipStream_t stream);

}  // namespace dora
