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
#include <algorithm>

#include "compose_kernels.hpp"
#include "dora_common.hpp"

namespace dora {

namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte global access; NT selects the nontemporal (streaming) cache policy.
template <bool NT>
__device__ inline Chunk ld16(const Chunk* p) {
  if constexpr (NT) {
    return __builtin_bit_cast(Chunk, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
  } else {
    return *p;
  }
}

template <bool NT>
__device__ inline void st16(Chunk* p, const Chunk& c) {
  if constexpr (NT) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, c), reinterpret_cast<u32x4*>(p));
  } else {
    *p = c;
  }
}

// Per-column scale pair.  g - 1 = (m - n) / n: the subtraction is exact when
// m / n lies in [1/2, 2] (Sterbenz), so a column with m != n keeps a nonzero
// base correction even when |g - 1| is below one fp32 ulp of 1.
__device__ inline void column_scales(float m, float n, float s, float& gm1, float& gs) {
  gm1 = (m - n) / n;
  gs = (m / n) * s;
}

template <int DT, int NTH, int ROWS, int UNROLL, bool NTL, bool NTS>
__global__ __launch_bounds__(NTH) void compose_fwd_vec(const Chunk* base, const Chunk* lora, const float* mag,
                                                       const float* norm, float s, int64_t T, int64_t out8,
                                                       int ncb, int add_base, Chunk* y) {
  const int64_t bid = blockIdx.x;
  const int64_t c8 = (bid % ncb) * NTH + threadIdx.x;
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
      cb[u] = ld16<NTL>(base + idx);
      cl[u] = ld16<NTL>(lora + idx);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) st16<NTS>(y + (t + u) * out8 + c8, compose(cb[u], cl[u]));
  }
  for (; t < t1; ++t) {
    const int64_t idx = t * out8 + c8;
    Chunk cb = ld16<NTL>(base + idx), cl = ld16<NTL>(lora + idx);
    st16<NTS>(y + idx, compose(cb, cl));
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

template <int DT, int NTH, int ROWS, int UNROLL, bool NTL, bool NTS>
__global__ __launch_bounds__(NTH) void compose_bwd_vec(const Chunk* dy, const Chunk* base, const Chunk* lora,
                                                       const float* mag, const float* norm, float s, int64_t T,
                                                       int64_t out8, int ncb, int add_base, Chunk* d_lora,
                                                       Chunk* d_base, float* partial) {
  const int64_t bid = blockIdx.x;
  const int64_t c8 = (bid % ncb) * NTH + threadIdx.x;
  if (c8 >= out8) return;
  // Token blocks in reverse order: the forward that precedes the backward in a
  // training step reads base and lora from first row to last, so their last
  // rows are the ones still in the last-level cache when the backward starts.
  const int64_t rb = (T + ROWS - 1) / ROWS - 1 - bid / ncb;
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
    st16<NTS>(d_lora + idx, f32_to_chunk<DT>(ol));
    if (d_base) st16<NTS>(d_base + idx, f32_to_chunk<DT>(ob));
  };

  int64_t t = t0;
  for (; t + UNROLL <= t1; t += UNROLL) {
    Chunk cd[UNROLL], cb[UNROLL], cl[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t idx = (t + u) * out8 + c8;
      cd[u] = ld16<NTL>(dy + idx);
      cb[u] = ld16<NTL>(base + idx);
      cl[u] = ld16<NTL>(lora + idx);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) step(cd[u], cb[u], cl[u], (t + u) * out8 + c8);
  }
  for (; t < t1; ++t) {
    const int64_t idx = t * out8 + c8;
    Chunk cd = ld16<NTL>(dy + idx), cb = ld16<NTL>(base + idx), cl = ld16<NTL>(lora + idx);
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
// COLS columns with GRPS groups of threads; group q adds blocks q, q + GRPS, ...
// into two fp64 accumulators (even and odd steps), and the group sums combine
// in a fixed pairwise tree, so the order depends only on the sizes.
template <int COLS, int GRPS>
__global__ __launch_bounds__(COLS* GRPS) void dmag_finalize(const float* partial, int64_t nrb, int64_t out,
                                                           const float* norm, float* d_mag) {
  __shared__ double red[GRPS][COLS];
  const int lc = threadIdx.x % COLS;
  const int grp = threadIdx.x / COLS;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * COLS + lc;
  double s0 = 0.0, s1 = 0.0;
  if (c < out) {
    int64_t rb = grp;
#pragma unroll 4
    for (; rb + GRPS < nrb; rb += 2 * GRPS) {
      s0 += static_cast<double>(partial[rb * out + c]);
      s1 += static_cast<double>(partial[(rb + GRPS) * out + c]);
    }
    if (rb < nrb) s0 += static_cast<double>(partial[rb * out + c]);
  }
  red[grp][lc] = s0 + s1;
  __syncthreads();
#pragma unroll
  for (int w = GRPS / 2; w >= 1; w >>= 1) {
    if (grp < w) red[grp][lc] += red[grp + w][lc];
    __syncthreads();
  }
  if (grp == 0 && c < out) d_mag[c] = static_cast<float>(red[0][lc] / static_cast<double>(norm[c]));
}

// Launch shapes of the 16-byte paths (threads, tokens per block, rows per batch
// of loads, nontemporal loads / stores) and of the magnitude-gradient finalize.
// Cache policies measured on MI355X at T = out = 8192 with the kernels run in
// the order of a training step (a 134 MB weight read, forward, backward): the
// outputs of one kernel are still being written back while the next runs, so
// the best pair is nontemporal stores in the forward and nontemporal loads and
// stores in the backward (~74% of peak HBM bandwidth over both, against ~67%
// with default policies).
// Short token blocks: consecutive workgroups then cover adjacent memory and
// the resident set sweeps HBM compactly (4-row blocks measured about 15%
// faster than 16-row blocks on data not in the caches).
constexpr int kFwdThreads = 256, kFwdRows = 2, kFwdUnroll = 2;
constexpr bool kFwdNtLoad = false, kFwdNtStore = true;
constexpr int kBwdThreads = 256, kBwdUnroll = 4;
constexpr bool kBwdNtLoad = true, kBwdNtStore = true;
constexpr int kFinCols = 32, kFinGroups = 16;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

template <int DT>
hipError_t launch_compose_fwd_t(const ComposeArgs& a, bool vec) {
  if (vec) {
    const int64_t out8 = a.out / 8;
    const int ncb = static_cast<int>(cdiv(out8, kFwdThreads));
    const int64_t nblk = ncb * cdiv(a.T, kFwdRows);
    hipLaunchKernelGGL((compose_fwd_vec<DT, kFwdThreads, kFwdRows, kFwdUnroll, kFwdNtLoad, kFwdNtStore>), dim3(nblk),
                       dim3(kFwdThreads), 0, a.stream,
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

template <int DT, int ROWS>
void launch_compose_bwd_rows(const ComposeArgs& a, bool vec, int64_t nrb) {
  if (vec) {
    const int64_t out8 = a.out / 8;
    const int ncb = static_cast<int>(cdiv(out8, kBwdThreads));
    hipLaunchKernelGGL((compose_bwd_vec<DT, kBwdThreads, ROWS, kBwdUnroll, kBwdNtLoad, kBwdNtStore>),
                       dim3(ncb * nrb), dim3(kBwdThreads), 0, a.stream, static_cast<const Chunk*>(a.dy),
                       static_cast<const Chunk*>(a.base), static_cast<const Chunk*>(a.lora), a.mag, a.norm, a.s, a.T,
                       out8, ncb, a.add_base, static_cast<Chunk*>(a.d_lora), static_cast<Chunk*>(a.d_base), a.partial);
  } else {
    using T = typename Dt<DT>::T;
    const int ncb = static_cast<int>(cdiv(a.out, kThreads));
    hipLaunchKernelGGL((compose_bwd_gen<DT, ROWS>), dim3(ncb * nrb), dim3(kThreads), 0, a.stream,
                       static_cast<const T*>(a.dy), static_cast<const T*>(a.base), static_cast<const T*>(a.lora),
                       a.mag, a.norm, a.s, a.T, a.out, ncb, a.add_base, static_cast<T*>(a.d_lora),
                       static_cast<T*>(a.d_base), a.partial);
  }
}

template <int DT>
hipError_t launch_compose_bwd_t(const ComposeArgs& a, bool vec) {
  const int rows = compose_bwd_rows(a.T, a.out);
  const int64_t nrb = cdiv(a.T, rows);
  if (nrb > 0) {
    if (rows == kBwdRowsWide)
      launch_compose_bwd_rows<DT, kBwdRowsWide>(a, vec, nrb);
    else
      launch_compose_bwd_rows<DT, kBwdRowsNarrow>(a, vec, nrb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((dmag_finalize<kFinCols, kFinGroups>), dim3(cdiv(a.out, kFinCols)), dim3(kFinCols * kFinGroups),
                     0, a.stream, a.partial, nrb, a.out, a.norm, a.d_mag);
  return hipGetLastError();
}

hipError_t launch_compose_fwd(const ComposeArgs& a, bool vec) {
  return a.dtype == 0 ? launch_compose_fwd_t<0>(a, vec) : launch_compose_fwd_t<1>(a, vec);
}

int compose_bwd_rows(int64_t T, int64_t out) {
  const int64_t ncb = cdiv(cdiv(out, 8), kBwdThreads);
  return ncb * cdiv(T, kBwdRowsWide) >= 512 ? kBwdRowsWide : kBwdRowsNarrow;
}

size_t compose_bwd_workspace(int64_t T, int64_t out) {
  if (T <= 0 || out <= 0) return 0;
  return static_cast<size_t>(cdiv(T, compose_bwd_rows(T, out))) * static_cast<size_t>(out) * 4;
}

int64_t compose_max_grid(int64_t T, int64_t out, bool vec) {
  const int64_t ncb_fwd = vec ? cdiv(out / 8, kFwdThreads) : cdiv(out, kThreads);
  const int64_t ncb_bwd = vec ? cdiv(out / 8, kBwdThreads) : cdiv(out, kThreads);
  const int64_t fwd = ncb_fwd * cdiv(T, kFwdRows), bwd = ncb_bwd * cdiv(T, compose_bwd_rows(T, out));
  return std::max({fwd, bwd, cdiv(out, kFinCols)});
}

hipError_t launch_compose_bwd(const ComposeArgs& a, bool vec) {
  return a.dtype == 0 ? launch_compose_bwd_t<0>(a, vec) : launch_compose_bwd_t<1>(a, vec);
}

}  // namespace dora
