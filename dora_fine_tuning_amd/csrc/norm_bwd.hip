// Backward of the factored weight norm, for a caller that does not detach n
// (the press summary of arXiv:2603.22276 describes the norm as base, cross and
// Gram parts of ||W0 + s B A||; it is silent on whether n is differentiated, so
// this is the alternative to the detached reading).  With c_i = dn_i / n_i and
// L = sum_i dn_i n_i, by the chain rule through the same three parts:
//
//   d_B_i = s c_i (U_i + s B_i G),                 U = W0 A^T, G = A A^T
//   d_A   = s (c*B)^T W0 + s^2 (B^T diag(c) B) A
//
// and the out x in matrix B A is never formed.  Steps, in launch order:
//   nbwd_colmax,       (fp16 only) per rank j, max_i |s c_i B_ij| and from it
//   nbwd_colscale      the operand scale sigma_j, a power of two;
//   nbwd_prep          c_i (0 where n_i = 0) and Y_ij = sigma_j s c_i B_ij
//                      [out x r] as the storage-dtype pair Yhi | Ylo [out x 2r];
//   d_B                the norm's W stream with G' = s G, its accumulators
//                      U + s B G stored and then scaled by s c_i (norm.hip);
//   M                  the token-axis contraction kernel (lora_bwd.hip) over
//                      the rows of B, its two Y panels Yhi and Ylo adding into
//                      one accumulator: B^T (Yhi + Ylo) = s B^T diag(c) B, in
//                      row slices;
//   nbwd_finalize_m    Z = s (that r x r matrix), transposed, rescaled to
//                      carry sigma_j on its column j, as Zhi | Zlo;
//   d_A                the same contraction kernel, in one launch, over the
//                      rows of W0 with Yhi + Ylo and then over the rows of A
//                      with Zhi + Zlo (each row slice takes its share of both;
//                      each stage's W0 rows meet both halves, so W0 is read
//                      once): the contraction axis [out rows of W0 ; r rows of
//                      A] gives d_A^T in row slices;
//   nbwd_finalize_a    sum of the slices, row j over sigma_j, transposed
//                      through LDS into d_A [r x in].
// The hi/lo pairs carry about 16 (bf16) or 22 (fp16) significant bits of the
// computed operands Y and Z into the bf16/fp16 MFMAs; W0, A and B enter exactly.
// Sizes or pointers the 16-byte path cannot take go to a general path of plain
// fp32 loops (one thread per output element).
#include <algorithm>

#include "dora_common.hpp"
#include "lora_compose_kernels.hpp"
#include "norm_bwd_kernels.hpp"
#include "norm_kernels.hpp"

namespace dora {

namespace {

__host__ __device__ inline int64_t ndiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// fp16 only (its exponent range is narrow): column j of the operand Y = s c B
// is stored times a power of two sigma_j that brings max_i |Y_ij| into
// [1/2, 1), so a small upstream gradient, an early-training B or a single small
// column of B does not push the hi/lo pair into fp16's subnormal range.  Every
// operand column that feeds rank j of d_A carries sigma_j: column j of Y, and
// column j of Z (its finalize rescales s M' by sigma_j / sigma_l, exactly, since
// M' = B^T Y carries sigma_l on its column l).  The d_A finalize divides row j
// by sigma_j (exactly).  One scale for all of Y left a column of B that is small
// on every row (rank 87 of a 2 x 320, r = 216 module) with subnormal Z entries
// and ~2^-10 relative error in its row of d_A.  bf16 has fp32's exponent range
// and takes sigma = 1 (no scale kernels run).
constexpr int kColMaxParts = 64;

// Per-column maxima of |s c_i B_ij| over a share of the rows: workgroup p takes
// rows [out p / nparts, out (p + 1) / nparts) and leaves max_i in part[p][j],
// as the bits of a non-negative float (whose order is that of the values).
// With rc = r / 8 chunks of 8 columns per row, thread t keeps the running
// maxima of chunk t % rc (t + 256 k for rc > 256) over every (256 / rc)-th row
// of the share, then merges them into the workgroup's own row of part with
// atomicMax, which gives the same result in any order; the workgroup zeroes
// that row first (no other workgroup touches it).
template <int DT>
__global__ __launch_bounds__(256) void nbwd_colmax(const void* Bv, const float* norm, const float* d_norm, int64_t out,
                                                   int64_t r, float s, int nparts, unsigned* part) {
  const Chunk* B = static_cast<const Chunk*>(Bv);
  const int p = static_cast<int>(blockIdx.x), t = static_cast<int>(threadIdx.x);
  const int64_t i0 = out * p / nparts, i1 = out * (p + 1) / nparts;
  const int64_t rc = r / 8;
  unsigned* row = part + static_cast<int64_t>(p) * r;
  for (int64_t j = t; j < r; j += 256) row[j] = 0u;
  __syncthreads();
  const int lanes = rc < 256 ? static_cast<int>(256 / rc) : 1;  // rows handled side by side
  const int lane = rc < 256 ? static_cast<int>(t / rc) : 0;
  if (lane >= lanes) return;
  for (int64_t jc = rc < 256 ? t % rc : t; jc < rc; jc += 256) {
    float m[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t i = i0 + lane; i < i1; i += lanes) {
      const float ni = norm[i];
      const float ci = ni != 0.0f ? d_norm[i] / ni : 0.0f;
      float f[8];
      chunk_to_f32<DT>(B[i * rc + jc], f);
#pragma unroll
      for (int q = 0; q < 8; ++q) m[q] = fmaxf(m[q], fabsf((s * ci) * f[q]));
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) atomicMax(row + jc * 8 + q, __float_as_uint(m[q]));
    if (rc < 256) break;
  }
}

// sigma = 2^-e for max = f 2^e, f in [1/2, 1), e clamped to [-60, 60]; 1 for a
// zero or non-finite max
__device__ inline float operand_scale(float mx) {
  if (!(mx > 0.0f) || !isfinite(mx)) return 1.0f;
  int e;
  frexpf(mx, &e);
  return ldexpf(1.0f, -std::min(60, std::max(-60, e)));  // 2^-60 .. 2^60: sigma_j / sigma_l stays finite in fp32
}

// sigma_j = operand_scale(max over the nparts row shares of part[p][j])
__global__ __launch_bounds__(256) void nbwd_colscale(const unsigned* part, int nparts, int64_t r, float* sigma) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= r) return;
  unsigned m = 0u;
  for (int p = 0; p < nparts; ++p) m = std::max(m, part[static_cast<int64_t>(p) * r + j]);
  sigma[j] = operand_scale(__uint_as_float(m));
}

// c_i = dn_i / n_i (0 where n_i == 0); Y_ij = sigma_j s c_i B_ij split into
// hi = round(Y), lo = round(Y - hi), stored at [i][j] and [i][r + j].  One
// 16-byte chunk (8 elements of one row, r % 8 == 0) per thread and step.
// sigma == nullptr: sigma_j = 1.
template <int DT>
__global__ __launch_bounds__(256) void nbwd_prep(const void* Bv, const float* norm, const float* d_norm, int64_t out,
                                                 int64_t r, float s, const float* sigma, float* c, void* Yv) {
  using T = typename Dt<DT>::T;
  const Chunk* B = static_cast<const Chunk*>(Bv);
  T* Y = static_cast<T*>(Yv);
  const int64_t n = out * r / 8;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t i = (e * 8) / r, j = e * 8 - i * r;
    const float ni = norm[i];
    const float ci = ni != 0.0f ? d_norm[i] / ni : 0.0f;
    if (j == 0) c[i] = ci;
    float sg[8];
    if (sigma) {
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(sigma + j), s1 = *reinterpret_cast<const f32x4*>(sigma + j + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sg[q] = s0[q];
        sg[q + 4] = s1[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) sg[q] = 1.0f;
    }
    float f[8], hi[8], lo[8];
    chunk_to_f32<DT>(B[e], f);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float y = ((s * ci) * f[q]) * sg[q];  // sigma_j is a power of two: exact
      hi[q] = Dt<DT>::to_f(Dt<DT>::from_f(y));
      lo[q] = y - hi[q];
    }
    *reinterpret_cast<Chunk*>(Y + i * 2 * r + j) = f32_to_chunk<DT>(hi);
    *reinterpret_cast<Chunk*>(Y + i * 2 * r + r + j) = f32_to_chunk<DT>(lo);
  }
}

// Slices the finalize of d_A loads all at once before adding them.
constexpr int kFinA = 8;

// Z[l][j] = s * M'[j][l], M'[j][l] = sum over slices of E[j][l]
// (E = B^T (Yhi + Ylo), [nSplit][r][r]), split into hi/lo at [l][j], [l][r + j].
// An 8 x 32 tile of (j, l) per workgroup, one element per thread: reads
// coalesced along l, a transpose through LDS, then 16-byte runs along j per
// row of Z.  The slices go in groups of 8, all 16 loads of a group in flight
// before the group is added in slice order; lanes past r read a valid
// address and drop the result, so the loads stay unconditional.
template <int DT>
__global__ __launch_bounds__(256) void nbwd_finalize_m(const float* E, int nSplit, int64_t r, float s,
                                                       const float* sigma, void* Zv) {
  using T = typename Dt<DT>::T;
  __shared__ float tile[8][33];
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 8, l0 = static_cast<int64_t>(blockIdx.y) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t slice = r * r;
  {
    const int64_t j = j0 + ty, l = l0 + tx;
    const float* Ej = E + (j < r && l < r ? j * r + l : 0);
    float m = 0.0f;
    int p = 0;
    for (; p + 8 <= nSplit; p += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = Ej[(p + u) * slice];
#pragma unroll
      for (int u = 0; u < 8; ++u) m += v[u];
    }
    for (; p < nSplit; ++p) m += Ej[p * slice];
    // M' carries sigma_l on its column l; Z's column j is to carry sigma_j
    // (powers of two: both rescalings are exact)
    if (sigma && j < r && l < r) m = (m / sigma[l]) * sigma[j];
    tile[ty][tx] = s * m;
  }
  __syncthreads();
  T* Z = static_cast<T*>(Zv);
  const int jj = threadIdx.x & 7, ll = threadIdx.x >> 3;
  const int64_t l = l0 + ll, j = j0 + jj;
  if (l < r && j < r) {
    const float z = tile[jj][ll];
    const T hi = Dt<DT>::from_f(z);
    Z[l * 2 * r + j] = hi;
    Z[l * 2 * r + r + j] = Dt<DT>::from_f(z - Dt<DT>::to_f(hi));
  }
}

// d_A[j][k] = (sum over the slices of E[k][j]) / sigma_j (E [nParts][in][r],
// the slices added in order; sigma_j a power of two), rounded once.
// A 32 x 32 tile of (k, j) per workgroup: coalesced reads along j, a transpose
// through LDS, coalesced writes along k.
template <int DT>
__global__ __launch_bounds__(256) void nbwd_finalize_a(const float* E, int nParts, int64_t in, int64_t r,
                                                       const float* sigma, void* dAv) {
  // sigma == nullptr: sigma_j = 1
  using T = typename Dt<DT>::T;
  __shared__ float tile[32][33];
  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * 32, j0 = static_cast<int64_t>(blockIdx.y) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t slice = in * r;
  if (nParts <= kFinA) {
    // every slice of the thread's four elements in flight before the first
    // addition (clamped indices keep the loads unconditional); the sums keep
    // slice order
    float e[4][kFinA];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t k = std::min<int64_t>(k0 + ty + 8 * q, in - 1), j = std::min<int64_t>(j0 + tx, r - 1);
      const float* Ep = E + k * r + j;
#pragma unroll
      for (int p = 0; p < kFinA; ++p) e[q][p] = Ep[static_cast<int64_t>(p < nParts ? p : nParts - 1) * slice];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kk = ty + 8 * q;
      const int64_t k = k0 + kk, j = j0 + tx;
      float v = 0.0f;
#pragma unroll
      for (int p = 0; p < kFinA; ++p)
        if (p < nParts) v += e[q][p];
      tile[kk][tx] = (k < in && j < r) ? (sigma ? v / sigma[j] : v) : 0.0f;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kk = ty + 8 * q;
      const int64_t k = k0 + kk, j = j0 + tx;
      float v = 0.0f;
      if (k < in && j < r) {
        const float* Ep = E + k * r + j;
        for (int p = 0; p < nParts; ++p) v += Ep[p * slice];
        if (sigma) v /= sigma[j];
      }
      tile[kk][tx] = v;
    }
  }
  __syncthreads();
  T* dA = static_cast<T*>(dAv);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int jj = ty + 8 * q;
    const int64_t j = j0 + jj, k = k0 + tx;
    if (j < r && k < in) dA[j * in + k] = Dt<DT>::from_f(tile[tx][jj]);
  }
}

template <int DT>
__global__ __launch_bounds__(256) void nbwd_zero(void* pv, int64_t n) {
  using T = typename Dt<DT>::T;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * 256)
    static_cast<T*>(pv)[e] = Dt<DT>::from_f(0.0f);
}

inline dim3 stride_grid(int64_t n) { return dim3(static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(ndiv(n, 256), 4096)))); }

template <int DT>
hipError_t zero_t(void* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL((nbwd_zero<DT>), stride_grid(n), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// General path (in or r not a multiple of 8, or unaligned pointers): one
// thread per output element, every sum in order in fp32, no MFMA.

// c_i = dn_i / n_i (0 where n_i == 0)
__global__ __launch_bounds__(256) void nbwd_gen_c(const float* norm, const float* d_norm, int64_t out, float* c) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= out) return;
  const float ni = norm[i];
  c[i] = ni != 0.0f ? d_norm[i] / ni : 0.0f;
}

// G[j][l] = sum_k A_jk A_lk and M[j][l] = sum_i c_i B_ij B_il, both [r x r] fp32
template <int DT>
__global__ __launch_bounds__(256) void nbwd_gen_gm(const void* Av, const void* Bv, const float* c, int64_t out,
                                                   int64_t in, int64_t r, float* G, float* M) {
  using T = typename Dt<DT>::T;
  const T* A = static_cast<const T*>(Av);
  const T* B = static_cast<const T*>(Bv);
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= r * r) return;
  const int64_t j = e / r, l = e - j * r;
  float g = 0.0f, m = 0.0f;
  for (int64_t k = 0; k < in; ++k) g = __builtin_fmaf(Dt<DT>::to_f(A[j * in + k]), Dt<DT>::to_f(A[l * in + k]), g);
  for (int64_t i = 0; i < out; ++i)
    m = __builtin_fmaf(c[i] * Dt<DT>::to_f(B[i * r + j]), Dt<DT>::to_f(B[i * r + l]), m);
  G[e] = g;
  M[e] = m;
}

// d_B[i][j] = s c_i (sum_k W0_ik A_jk + s sum_l B_il G_lj)
template <int DT>
__global__ __launch_bounds__(256) void nbwd_gen_db(const void* Wv, const void* Av, const void* Bv, const float* c,
                                                   const float* G, int64_t out, int64_t in, int64_t r, float s,
                                                   void* dBv) {
  using T = typename Dt<DT>::T;
  const T *W = static_cast<const T*>(Wv), *A = static_cast<const T*>(Av), *B = static_cast<const T*>(Bv);
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= out * r) return;
  const int64_t i = e / r, j = e - i * r;
  float u = 0.0f, q = 0.0f;
  for (int64_t k = 0; k < in; ++k) u = __builtin_fmaf(Dt<DT>::to_f(W[i * in + k]), Dt<DT>::to_f(A[j * in + k]), u);
  for (int64_t l = 0; l < r; ++l) q = __builtin_fmaf(Dt<DT>::to_f(B[i * r + l]), G[l * r + j], q);
  static_cast<T*>(dBv)[e] = Dt<DT>::from_f((s * c[i]) * __builtin_fmaf(s, q, u));
}

// d_A[j][k] = s (sum_i c_i B_ij W0_ik + s sum_l M_jl A_lk)
template <int DT>
__global__ __launch_bounds__(256) void nbwd_gen_da(const void* Wv, const void* Av, const void* Bv, const float* c,
                                                   const float* M, int64_t out, int64_t in, int64_t r, float s,
                                                   void* dAv) {
  using T = typename Dt<DT>::T;
  const T *W = static_cast<const T*>(Wv), *A = static_cast<const T*>(Av), *B = static_cast<const T*>(Bv);
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= r * in) return;
  const int64_t j = e / in, k = e - j * in;  // k fastest: the reads of W0 rows are coalesced
  float a1 = 0.0f, a2 = 0.0f;
  for (int64_t i = 0; i < out; ++i)
    a1 = __builtin_fmaf(c[i] * Dt<DT>::to_f(B[i * r + j]), Dt<DT>::to_f(W[i * in + k]), a1);
  for (int64_t l = 0; l < r; ++l) a2 = __builtin_fmaf(M[j * r + l], Dt<DT>::to_f(A[l * in + k]), a2);
  static_cast<T*>(dAv)[e] = Dt<DT>::from_f(s * __builtin_fmaf(s, a2, a1));
}

template <int DT>
hipError_t launch_norm_bwd_gen_t(const NormBwdPlan& p, const NormBwdArgs& a) {
  const int64_t out = p.out, in = p.in, r = p.r;
  char* ws = static_cast<char*>(a.ws);
  float* c = reinterpret_cast<float*>(ws + p.off_c);
  float* G = reinterpret_cast<float*>(ws + p.off_y);
  float* M = reinterpret_cast<float*>(ws + p.off_z);
  hipLaunchKernelGGL(nbwd_gen_c, dim3(static_cast<unsigned>(ndiv(out, 256))), dim3(256), 0, a.stream, a.norm,
                     a.d_norm, out, c);
  hipLaunchKernelGGL((nbwd_gen_gm<DT>), dim3(static_cast<unsigned>(ndiv(r * r, 256))), dim3(256), 0, a.stream, a.A,
                     a.B, c, out, in, r, G, M);
  hipLaunchKernelGGL((nbwd_gen_db<DT>), dim3(static_cast<unsigned>(ndiv(out * r, 256))), dim3(256), 0, a.stream,
                     a.W0, a.A, a.B, c, G, out, in, r, a.s, a.d_B);
  hipLaunchKernelGGL((nbwd_gen_da<DT>), dim3(static_cast<unsigned>(ndiv(r * in, 256))), dim3(256), 0, a.stream,
                     a.W0, a.A, a.B, c, M, out, in, r, a.s, a.d_A);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_norm_bwd_t(const NormBwdPlan& p, const NormBwdArgs& a) {
  const int64_t out = p.out, in = p.in, r = p.r;
  if (r == 0) return hipSuccess;
  if (out == 0) return zero_t<DT>(a.d_A, r * in, a.stream);
  if (in == 0) return zero_t<DT>(a.d_B, out * r, a.stream);
  if (!p.vec) return launch_norm_bwd_gen_t<DT>(p, a);
  char* ws = static_cast<char*>(a.ws);
  float* c = reinterpret_cast<float*>(ws + p.off_c);
  void* Y = ws + p.off_y;
  void* Z = ws + p.off_z;
  float* big = reinterpret_cast<float*>(ws + p.off_big);
  // fp16: the per-rank operand scales sigma [r] (after kColMaxParts x r partial maxima)
  float* sigma = nullptr;
  if (DT == 1) {
    unsigned* part = reinterpret_cast<unsigned*>(ws + p.off_sigma);
    sigma = reinterpret_cast<float*>(part + static_cast<int64_t>(kColMaxParts) * r);
    const int nparts = static_cast<int>(std::min<int64_t>(kColMaxParts, ndiv(out, 64)));
    hipLaunchKernelGGL((nbwd_colmax<DT>), dim3(static_cast<unsigned>(nparts)), dim3(256), 0, a.stream, a.B, a.norm,
                       a.d_norm, out, r, a.s, nparts, part);
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
    hipLaunchKernelGGL(nbwd_colscale, dim3(static_cast<unsigned>(ndiv(r, 256))), dim3(256), 0, a.stream, part, nparts,
                       r, sigma);
    e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  hipLaunchKernelGGL((nbwd_prep<DT>), stride_grid(out * r / 8), dim3(256), 0, a.stream, a.B, a.norm, a.d_norm, out, r,
                     a.s, sigma, c, Y);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // d_B (the W stream's partials live in the big region until its finalize)
  e = launch_norm_bwd_db(p.np, a.W0, a.A, a.B, a.s, c, a.d_B, ws + p.off_np, big, a.stream);
  if (e != hipSuccess) return e;
  // M = B^T (Yhi + Ylo) -> Z
  e = launch_row_contract(a.B, Y, out, r, r, 2 * r, true, p.np.dtype, big, a.stream);
  if (e != hipSuccess) return e;
  const dim3 mgrid(static_cast<unsigned>(ndiv(r, 8)), static_cast<unsigned>(ndiv(r, 32)));
  hipLaunchKernelGGL((nbwd_finalize_m<DT>), mgrid, dim3(256), 0, a.stream, big, p.rM.nSplit, r, a.s, sigma, Z);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // d_A^T slices: the rows of W0 with Y, then (spread over the same slices) the rows of A with Z
  e = launch_row_contract(a.W0, Y, out, in, r, 2 * r, true, p.np.dtype, big, a.stream, a.A, Z, r);
  if (e != hipSuccess) return e;
  const dim3 fgrid(static_cast<unsigned>(ndiv(in, 32)), static_cast<unsigned>(ndiv(r, 32)));
  hipLaunchKernelGGL((nbwd_finalize_a<DT>), fgrid, dim3(256), 0, a.stream, big, p.rW.nSplit, in, r, sigma, a.d_A);
  return hipGetLastError();
}

}  // namespace

NormBwdPlan make_norm_bwd_plan(int64_t out, int64_t in, int64_t r, int dtype, bool vec) {
  NormBwdPlan p;
  p.out = out;
  p.in = in;
  p.r = r;
  p.vec = vec;
  if (out <= 0 || in <= 0 || r <= 0) return p;
  if (!vec) {
    // c [out], G and M [r x r] fp32 (in the Y and Z slots)
    p.off_c = 0;
    p.off_y = al256(static_cast<size_t>(out) * 4);
    p.off_z = p.off_y + al256(static_cast<size_t>(r) * r * 4);
    p.bytes = p.off_z + al256(static_cast<size_t>(r) * r * 4);
    p.max_grid = std::max({ndiv(out, 256), ndiv(r * r, 256), ndiv(out * r, 256), ndiv(r * in, 256)});
    return p;
  }
  p.np = make_norm_plan(out, in, r, dtype, true, true);
  p.rM = row_contract_plan(out, r, r, 0, 2 * r);
  p.rW = row_contract_plan(out, in, r, r, 2 * r);
  size_t off = 0;
  p.off_np = off;
  off += al256(p.np.bytes);
  p.off_c = off;
  off += al256(static_cast<size_t>(out) * 4);
  p.off_sigma = off;  // fp16: the operand scales' partial maxima [kColMaxParts x r] and the scales [r]
  off += al256(static_cast<size_t>(kColMaxParts + 1) * r * 4);
  p.off_y = off;
  off += al256(static_cast<size_t>(out) * 2 * r * 2);
  p.off_z = off;
  off += al256(static_cast<size_t>(r) * 2 * r * 2);
  p.off_big = off;
  off += al256(std::max({norm_bwd_acc_bytes(p.np), p.rM.bytes, p.rW.bytes}));
  p.bytes = off;
  p.max_grid = std::max({norm_max_grid(p.np), p.rM.grid, p.rW.grid, ndiv(in, 32), ndiv(out * r, 256)});
  p.max_slice_bytes = std::max(p.rM.slice_bytes, p.rW.slice_bytes);
  return p;
}

size_t norm_bwd_workspace_bytes(int64_t out, int64_t in, int64_t r, int dtype) {
  size_t b = make_norm_bwd_plan(out, in, r, dtype, false).bytes;
  if (in % 8 == 0 && r % 8 == 0 && in < (int64_t(1) << 21) && r <= (int64_t(1) << 20))
    b = std::max(b, make_norm_bwd_plan(out, in, r, dtype, true).bytes);
  return b;
}

hipError_t launch_norm_bwd(const NormBwdPlan& p, const NormBwdArgs& a) {
  return a.dtype == 0 ? launch_norm_bwd_t<0>(p, a) : launch_norm_bwd_t<1>(p, a);
}

}  // namespace dora
