// DoRA magnitude compose, forward and backward, for gfx950.
//
// Both directions are one-pass HBM streams over [T x out] matrices with a
// per-column scale pair (g - 1, g*s) derived from the fp32 vectors m and n
// (press summary of arXiv:2603.22276, paragraphs on the fused compose kernel
// and on stability near g = 1).  Arithmetic is fp32 with a single rounding of
// each stored element.
//
// Layout of the fast path: a thread owns 8 consecutive columns (one 16-byte
// chunk per row), computes its 8 scale pairs once and walks ROWS rows of its
// token block, so every row access is a fully coalesced 16-byte load or store
// and m/n are read once per thread rather than once per element.  Blocks are
// numbered column-block fastest so neighbouring workgroups stream neighbouring
// 4 KiB row segments.  The general path (row length not a multiple of 8, or
// unaligned pointers) does the same with one column per thread.
//
// The magnitude gradient sum_t dy*(base + s*lora) is reduced without atomics:
// each thread writes the fp32 sum over its ROWS tokens for its columns to a
// [token-blocks x out] partial buffer, and dmag_finalize adds the partials in
// a fixed order in fp64 and divides by n.  Results are bitwise reproducible.
#include "compose_kernels.hpp"
#include "dora_common.hpp"

namespace dora {

namespace {

constexpr int kThreads = 256;

// Per-column scale pair.  g - 1 = (m - n) / n: the subtraction is exact when
// m / n lies in [1/2, 2] (Sterbenz), so a column with m != n keeps a nonzero
// base correction even when |g - 1| is below one fp32 ulp of 1.
__device__ inline void column_scales(float m, float n, float s, float& gm1, float& gs) {
  gm1 = (m - n) / n;
  gs = (m / n) * s;
}

template <int DT, int ROWS, int UNROLL>
__global__ __launch_bounds__(kThreads) void compose_fwd_vec(const Chunk* base, const Chunk* lora,
                                                            const float* mag, const float* norm, float s,
                                                            int64_t T, int64_t out8, int ncb, int add_base,
                                                            Chunk* y) {
  const int64_t bid = blockIdx.x;
  const int64_t c8 = (bid % ncb) * kThreads + threadIdx.x;
  if (c8 >= out8) return;
  const int64_t t0 = (bid / ncb) * ROWS;
  const int64_t t1 = (t0 + ROWS < T) ? t0 + ROWS : T;

  float gm1[8], gs[8];
  {
    const f32x4* m4 = reinterpret_cast<const f32x4*>(mag) + 2 * c8;
    const f32x4* n4 = reinterpret_cast<const f32x4*>(norm) + 2 * c8;
    f32x4 ma = m4[0], mb = m4[1], na = n4[0], nb = n4[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      column_scales(ma[j], na[j], s, gm1[j], gs[j]);
      column_scales(mb[j], nb[j], s, gm1[j + 4], gs[j + 4]);
    }
  }

  auto compose = [&](const Chunk& cb, const Chunk& cl) -> Chunk {
    float b[8], l[8], o[8];
    chunk_to_f32<DT>(cb, b);
    chunk_to_f32<DT>(cl, l);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float d = __builtin_fmaf(gs[j], l[j], gm1[j] * b[j]);
      o[j] = add_base ? b[j] + d : d;
    }
    return f32_to_chunk<DT>(o);
  };

  int64_t t = t0;
  for (; t + UNROLL <= t1; t += UNROLL) {
    Chunk cb[UNROLL], cl[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t idx = (t + u) * out8 + c8;
      cb[u] = base[idx];
      cl[u] = lora[idx];
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) y[(t + u) * out8 + c8] = compose(cb[u], cl[u]);
  }
  for (; t < t1; ++t) {
    const int64_t idx = t * out8 + c8;
    Chunk cb = base[idx], cl = lora[idx];
    y[idx] = compose(cb, cl);
  }
}

template <int DT, int ROWS>
__global__ __launch_bounds__(kThreads) void compose_fwd_gen(const typename Dt<DT>::T* base,
                                                            const typename Dt<DT>::T* lora, const float* mag,
                                                            const float* norm, float s, int64_t T, int64_t out,
                                                            int ncb, int add_base, typename Dt<DT>::T* y) {
  const int64_t bid = blockIdx.x;
  const int64_t c = (bid % ncb) * kThreads + threadIdx.x;
  if (c >= out) return;
  const int64_t t0 = (bid / ncb) * ROWS;
  const int64_t t1 = (t0 + ROWS < T) ? t0 + ROWS : T;
  float gm1, gs;
  column_scales(mag[c], norm[c], s, gm1, gs);
  for (int64_t t = t0; t < t1; ++t) {
    const int64_t idx = t * out + c;
    const float b = Dt<DT>::to_f(base[idx]);
    const float l = Dt<DT>::to_f(lora[idx]);
    const float d = __builtin_fmaf(gs, l, gm1 * b);
    y[idx] = Dt<DT>::from_f(add_base ? b + d : d);
  }
}

template <int DT, int ROWS, int UNROLL>
__global__ __launch_bounds__(kThreads) void compose_bwd_vec(const Chunk* dy, const Chunk* base, const Chunk* lora,
                                                            const float* mag, const float* norm, float s,
                                                            int64_t T, int64_t out8, int ncb, int add_base,
                                                            Chunk* d_lora, Chunk* d_base, float* partial) {
  const int64_t bid = blockIdx.x;
  const int64_t c8 = (bid % ncb) * kThreads + threadIdx.x;
  if (c8 >= out8) return;
  const int64_t rb = bid / ncb;
  const int64_t t0 = rb * ROWS;
  const int64_t t1 = (t0 + ROWS < T) ? t0 + ROWS : T;

  // d_base scale: g - 1 for the delta output, g for the full output.
  float gb[8], gs[8];
  {
    const f32x4* m4 = reinterpret_cast<const f32x4*>(mag) + 2 * c8;
    const f32x4* n4 = reinterpret_cast<const f32x4*>(norm) + 2 * c8;
    f32x4 ma = m4[0], mb = m4[1], na = n4[0], nb = n4[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float gm1a, gm1b;
      column_scales(ma[j], na[j], s, gm1a, gs[j]);
      column_scales(mb[j], nb[j], s, gm1b, gs[j + 4]);
      gb[j] = add_base ? ma[j] / na[j] : gm1a;
      gb[j + 4] = add_base ? mb[j] / nb[j] : gm1b;
    }
  }
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;

  auto step = [&](const Chunk& cd, const Chunk& cb, const Chunk& cl, int64_t idx) {
    float d[8], b[8], l[8], ol[8], ob[8];
    chunk_to_f32<DT>(cd, d);
    chunk_to_f32<DT>(cb, b);
    chunk_to_f32<DT>(cl, l);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ol[j] = gs[j] * d[j];
      ob[j] = gb[j] * d[j];
      acc[j] = __builtin_fmaf(d[j], __builtin_fmaf(s, l[j], b[j]), acc[j]);
    }
    d_lora[idx] = f32_to_chunk<DT>(ol);
    if (d_base) d_base[idx] = f32_to_chunk<DT>(ob);
  };

  int64_t t = t0;
  for (; t + UNROLL <= t1; t += UNROLL) {
    Chunk cd[UNROLL], cb[UNROLL], cl[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t idx = (t + u) * out8 + c8;
      cd[u] = dy[idx];
      cb[u] = base[idx];
      cl[u] = lora[idx];
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) step(cd[u], cb[u], cl[u], (t + u) * out8 + c8);
  }
  for (; t < t1; ++t) {
    const int64_t idx = t * out8 + c8;
    Chunk cd = dy[idx], cb = base[idx], cl = lora[idx];
    step(cd, cb, cl, idx);
  }
  f32x4* p = reinterpret_cast<f32x4*>(partial + rb * out8 * 8) + 2 * c8;
  p[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
  p[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

template <int DT, int ROWS>
__global__ __launch_bounds__(kThreads) void compose_bwd_gen(const typename Dt<DT>::T* dy,
                                                            const typename Dt<DT>::T* base,
                                                            const typename Dt<DT>::T* lora, const float* mag,
                                                            const float* norm, float s, int64_t T, int64_t out,
                                                            int ncb, int add_base, typename Dt<DT>::T* d_lora,
                                                            typename Dt<DT>::T* d_base, float* partial) {
  const int64_t bid = blockIdx.x;
  const int64_t c = (bid % ncb) * kThreads + threadIdx.x;
  if (c >= out) return;
  const int64_t rb = bid / ncb;
  const int64_t t0 = rb * ROWS;
  const int64_t t1 = (t0 + ROWS < T) ? t0 + ROWS : T;
  const float m = mag[c], n = norm[c];
  float gm1, gs;
  column_scales(m, n, s, gm1, gs);
  const float gb = add_base ? m / n : gm1;
  float acc = 0.0f;
  for (int64_t t = t0; t < t1; ++t) {
    const int64_t idx = t * out + c;
    const float d = Dt<DT>::to_f(dy[idx]);
    const float b = Dt<DT>::to_f(base[idx]);
    const float l = Dt<DT>::to_f(lora[idx]);
    d_lora[idx] = Dt<DT>::from_f(gs * d);
    if (d_base) d_base[idx] = Dt<DT>::from_f(gb * d);
    acc = __builtin_fmaf(d, __builtin_fmaf(s, l, b), acc);
  }
  partial[rb * out + c] = acc;
}

// d_mag[c] = (sum over token blocks of partial[., c]) / n[c].  A block covers
// 64 columns with 4 groups of threads; group q adds blocks q, q+4, ... in fp64,
// then the four group sums combine as (g0 + g1) + (g2 + g3).
__global__ __launch_bounds__(kThreads) void dmag_finalize(const float* partial, int64_t nrb, int64_t out,
                                                          const float* norm, float* d_mag) {
  __shared__ double red[4][64];
  const int lc = threadIdx.x % 64;
  const int grp = threadIdx.x / 64;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 64 + lc;
  double sum = 0.0;
  if (c < out) {
    for (int64_t rb = grp; rb < nrb; rb += 4) sum += static_cast<double>(partial[rb * out + c]);
  }
  red[grp][lc] = sum;
  __syncthreads();
  if (grp == 0 && c < out) {
    const double tot = (red[0][lc] + red[1][lc]) + (red[2][lc] + red[3][lc]);
    d_mag[c] = static_cast<float>(tot / static_cast<double>(norm[c]));
  }
}

constexpr int kFwdRows = 16;
constexpr int kFwdUnroll = 4;
constexpr int kBwdUnroll = 4;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

template <int DT>
hipError_t launch_compose_fwd_t(const ComposeArgs& a, bool vec) {
  if (vec) {
    const int64_t out8 = a.out / 8;
    const int ncb = static_cast<int>(cdiv(out8, kThreads));
    const int64_t nblk = ncb * cdiv(a.T, kFwdRows);
    hipLaunchKernelGGL((compose_fwd_vec<DT, kFwdRows, kFwdUnroll>), dim3(nblk), dim3(kThreads), 0, a.stream,
                       static_cast<const Chunk*>(a.base), static_cast<const Chunk*>(a.lora), a.mag, a.norm, a.s,
                       a.T, out8, ncb, a.add_base, static_cast<Chunk*>(a.y));
  } else {
    using T = typename Dt<DT>::T;
    const int ncb = static_cast<int>(cdiv(a.out, kThreads));
    const int64_t nblk = ncb * cdiv(a.T, kFwdRows);
    hipLaunchKernelGGL((compose_fwd_gen<DT, kFwdRows>), dim3(nblk), dim3(kThreads), 0, a.stream,
                       static_cast<const T*>(a.base), static_cast<const T*>(a.lora), a.mag, a.norm, a.s, a.T,
                       a.out, ncb, a.add_base, static_cast<T*>(a.y));
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_compose_bwd_t(const ComposeArgs& a, bool vec) {
  const int64_t nrb = cdiv(a.T, kBwdRows);
  if (nrb > 0) {
    if (vec) {
      const int64_t out8 = a.out / 8;
      const int ncb = static_cast<int>(cdiv(out8, kThreads));
      hipLaunchKernelGGL((compose_bwd_vec<DT, kBwdRows, kBwdUnroll>), dim3(ncb * nrb), dim3(kThreads), 0,
                         a.stream, static_cast<const Chunk*>(a.dy), static_cast<const Chunk*>(a.base),
                         static_cast<const Chunk*>(a.lora), a.mag, a.norm, a.s, a.T, out8, ncb, a.add_base,
                         static_cast<Chunk*>(a.d_lora), static_cast<Chunk*>(a.d_base), a.partial);
    } else {
      using T = typename Dt<DT>::T;
      const int ncb = static_cast<int>(cdiv(a.out, kThreads));
      hipLaunchKernelGGL((compose_bwd_gen<DT, kBwdRows>), dim3(ncb * nrb), dim3(kThreads), 0, a.stream,
                         static_cast<const T*>(a.dy), static_cast<const T*>(a.base), static_cast<const T*>(a.lora),
                         a.mag, a.norm, a.s, a.T, a.out, ncb, a.add_base, static_cast<T*>(a.d_lora),
                         static_cast<T*>(a.d_base), a.partial);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(dmag_finalize, dim3(cdiv(a.out, 64)), dim3(kThreads), 0, a.stream, a.partial, nrb, a.out,
                     a.norm, a.d_mag);
  return hipGetLastError();
}

hipError_t launch_compose_fwd(const ComposeArgs& a, bool vec) {
  return a.dtype == 0 ? launch_compose_fwd_t<0>(a, vec) : launch_compose_fwd_t<1>(a, vec);
}

hipError_t launch_compose_bwd(const ComposeArgs& a, bool vec) {
  return a.dtype == 0 ? launch_compose_bwd_t<0>(a, vec) : launch_compose_bwd_t<1>(a, vec);
}

}  // namespace dora
