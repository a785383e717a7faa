// Factored DoRA weight norm for gfx950.
//
//   n_i^2 = ||W0_i||^2 + 2 s B_i U_i^T + s^2 B_i G B_i^T,  U = W0 A^T, G = A A^T
//
// (press summary of arXiv:2603.22276, paragraph on the "factored norm": base,
// cross and Gram terms replace the out x in matrix B*A; scratch is
// O(out*r + r*r)).
//
// Kernels, in launch order:
//   gram_kernel    split-K partials of G over upper-triangular 64x64 tiles
//                  (G is symmetric), MFMA 32x32x16 with fp32 accumulation;
//   gram_finalize  fixed-order fp64 sum of the partials, G' = (s/2) G split
//                  into two storage-dtype matrices G'hi + G'lo;
//   wstream_kernel one pass over W0.  A workgroup owns 128 rows x 128 rank
//                  columns and a slice of the augmented K axis
//                    [ W0 | B | B ] . [ A | G'hi | G'lo ]^T
//                  so its accumulator holds U + B G' = U + (s/2) B G for those
//                  rows and columns.  The epilogue reduces B_ij * acc_ij over its
//                  columns (cross + Gram share one dot product:
//                  2s * sum_j B_ij (U + (s/2) B G)_ij = cross_i + gram_i), and
//                  the loader squares the W0 chunks it moves to LDS for the base
//                  term.  U is never written to memory.
//   norm_finalize  n_i = sqrt(max(sum of partials, 0)) in fp64, rounded to fp32.
//
// All reductions are in fixed order, so the result is bitwise reproducible.
#include <algorithm>

#include "dora_common.hpp"
#include "norm_kernels.hpp"

namespace dora {

namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align16(size_t x) { return (x + 15) & ~static_cast<size_t>(15); }

// MFMA tile of a workgroup: BM x BN outputs, K stage BK, WM x WN waves each
// owning (BM/WM) x (BN/WN) outputs as 32x32 MFMA tiles.  LDS rows are padded
// by 8 elements (16 bytes) so the 16-byte fragment reads of 16 consecutive
// rows fall in distinct bank groups.
template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int TM = BM / (WM * 32), TN = BN / (WN * 32);
  static constexpr int LDK = BK + 8;
  static constexpr int CPR = BK / 8;
  static constexpr int RPP = NT / CPR;
  static constexpr int XCH = BM / RPP, YCH = BN / RPP;
  static constexpr int LDS_ELEMS = 2 * (BM + BN) * LDK;
  static_assert(BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "wave tile");
  static_assert(NT % CPR == 0 && BM % RPP == 0 && BN % RPP == 0, "loader mapping");
};

using TileW = Tile<128, 128, 64, 2, 2>;
using TileG = Tile<64, 64, 64, 2, 2>;

// A row-major operand panel: rows x klen valid elements, ld elements per row.
struct Operand {
  const void* p;
  int64_t ld, rows, klen;
};

template <int DT, bool VEC>
__device__ inline Chunk load_chunk(const Operand& op, int64_t row, int64_t k) {
  using T = typename Dt<DT>::T;
  if (row >= op.rows || k >= op.klen) return zero_chunk();
  const T* src = static_cast<const T*>(op.p) + row * op.ld + k;
  if (VEC) return *reinterpret_cast<const Chunk*>(src);
  typename Dt<DT>::V8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (k + j < op.klen) ? src[j] : static_cast<T>(0.0f);
  return __builtin_bit_cast(Chunk, v);
}

// Stage map of the fused W stream: stage st covers BK columns of one segment of
// the augmented K axis.
struct WStages {
  const void *W0, *A, *B, *Ghi, *Glo;
  int64_t out, in, r, S1, S2;
  template <int BK>
  __device__ inline void get(int64_t st, Operand& X, Operand& Y, int64_t& k0, bool& seg_w) const {
    if (st < S1) {
      X = Operand{W0, in, out, in};
      Y = Operand{A, in, r, in};
      k0 = st * BK;
      seg_w = true;
    } else if (st < S1 + S2) {
      X = Operand{B, r, out, r};
      Y = Operand{Ghi, r, r, r};
      k0 = (st - S1) * BK;
      seg_w = false;
    } else {
      X = Operand{B, r, out, r};
      Y = Operand{Glo, r, r, r};
      k0 = (st - S1 - S2) * BK;
      seg_w = false;
    }
  }
};

struct GStages {
  const void* A;
  int64_t in, r;
  template <int BK>
  __device__ inline void get(int64_t st, Operand& X, Operand& Y, int64_t& k0, bool& seg_w) const {
    X = Operand{A, in, r, in};
    Y = X;
    k0 = st * BK;
    seg_w = false;
  }
};

// acc[i][j] += X[m0 + rows, K stages] . Y[n0 + cols, K stages]^T over stages
// [st0, st1).  Double-buffered LDS; the next stage's global loads are issued
// before the current stage's MFMAs.  With want_base, the squares of the X
// chunks of W0 stages are summed into bsum (thread rows lrow + i*RPP).
template <int DT, bool VEC, class TL, class Stages>
__device__ inline void mainloop(const Stages& sm, int64_t st0, int64_t st1, int64_t m0, int64_t n0,
                                typename Dt<DT>::T* smem, f32x16 (&acc)[TL::TM][TL::TN], float (&bsum)[TL::XCH],
                                bool want_base) {
  using T = typename Dt<DT>::T;
  using V8 = typename Dt<DT>::V8;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const int lrow = tid / TL::CPR, lkc = tid % TL::CPR;
  T* Xs[2] = {smem, smem + (TL::BM + TL::BN) * TL::LDK};
  T* Ys[2] = {Xs[0] + TL::BM * TL::LDK, Xs[1] + TL::BM * TL::LDK};

  Chunk xr[TL::XCH], yr[TL::YCH];
  auto gload = [&](int64_t st) -> bool {
    Operand X, Y;
    int64_t k0;
    bool seg_w;
    sm.template get<TL::BK>(st, X, Y, k0, seg_w);
    const int64_t k = k0 + lkc * 8;
#pragma unroll
    for (int i = 0; i < TL::XCH; ++i) xr[i] = load_chunk<DT, VEC>(X, m0 + lrow + i * TL::RPP, k);
#pragma unroll
    for (int i = 0; i < TL::YCH; ++i) yr[i] = load_chunk<DT, VEC>(Y, n0 + lrow + i * TL::RPP, k);
    return seg_w;
  };
  auto lstore = [&](int buf, bool seg_w) {
    if (want_base && seg_w) {
#pragma unroll
      for (int i = 0; i < TL::XCH; ++i) {
        float f[8];
        chunk_to_f32<DT>(xr[i], f);
#pragma unroll
        for (int j = 0; j < 8; ++j) bsum[i] = __builtin_fmaf(f[j], f[j], bsum[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < TL::XCH; ++i)
      *reinterpret_cast<Chunk*>(Xs[buf] + (lrow + i * TL::RPP) * TL::LDK + lkc * 8) = xr[i];
#pragma unroll
    for (int i = 0; i < TL::YCH; ++i)
      *reinterpret_cast<Chunk*>(Ys[buf] + (lrow + i * TL::RPP) * TL::LDK + lkc * 8) = yr[i];
  };

  if (st0 >= st1) return;
  lstore(0, gload(st0));
  __syncthreads();
  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;
  for (int64_t st = st0; st < st1; ++st) {
    const int buf = static_cast<int>((st - st0) & 1);
    const bool have_next = st + 1 < st1;
    bool next_w = false;
    if (have_next) next_w = gload(st + 1);
    const T* xs = Xs[buf] + (wm * TL::TM * 32 + frow) * TL::LDK + fk;
    const T* ys = Ys[buf] + (wn * TL::TN * 32 + frow) * TL::LDK + fk;
#pragma unroll
    for (int kk = 0; kk < TL::BK / 16; ++kk) {
      V8 a[TL::TM], b[TL::TN];
#pragma unroll
      for (int i = 0; i < TL::TM; ++i) a[i] = *reinterpret_cast<const V8*>(xs + i * 32 * TL::LDK + kk * 16);
#pragma unroll
      for (int j = 0; j < TL::TN; ++j) b[j] = *reinterpret_cast<const V8*>(ys + j * 32 * TL::LDK + kk * 16);
#pragma unroll
      for (int i = 0; i < TL::TM; ++i)
#pragma unroll
        for (int j = 0; j < TL::TN; ++j) acc[i][j] = Dt<DT>::mfma32(a[i], b[j], acc[i][j]);
    }
    if (have_next) lstore(buf ^ 1, next_w);
    __syncthreads();
  }
}

// Workgroups are dealt to the 8 XCDs round-robin by index; renumber them so
// each XCD receives a contiguous range of the logical work list (one K slice of
// A per XCD's L2, and the rank tiles of a row block together).  gridDim.x is a
// multiple of 8.
__device__ inline int64_t xcd_logical_index() {
  const int64_t b = blockIdx.x;
  return (b & 7) * (gridDim.x >> 3) + (b >> 3);
}

struct GramArgs {
  const void* A;
  int64_t in, r, Sg;
  int nTg, nUpper, splitG;
  float* gpart;
};

template <int DT, bool VEC>
__global__ __launch_bounds__(TileG::NT) void gram_kernel(GramArgs a) {
  using TL = TileG;
  __shared__ __attribute__((aligned(16))) typename Dt<DT>::T smem[TL::LDS_ELEMS];
  const int64_t v = xcd_logical_index();
  if (v >= static_cast<int64_t>(a.nUpper) * a.splitG) return;
  int u = static_cast<int>(v % a.nUpper);
  const int sp = static_cast<int>(v / a.nUpper);
  int ti = 0;
  while (u >= a.nTg - ti) {
    u -= a.nTg - ti;
    ++ti;
  }
  const int tj = ti + u;
  const int64_t m0 = static_cast<int64_t>(ti) * TL::BM, n0 = static_cast<int64_t>(tj) * TL::BN;
  const int64_t st0 = a.Sg * sp / a.splitG, st1 = a.Sg * (sp + 1) / a.splitG;

  f32x16 acc[TL::TM][TL::TN];
#pragma unroll
  for (int i = 0; i < TL::TM; ++i)
#pragma unroll
    for (int j = 0; j < TL::TN; ++j) acc[i][j] = f32x16{};
  float bsum[TL::XCH] = {};
  mainloop<DT, VEC, TL>(GStages{a.A, a.in, a.r}, st0, st1, m0, n0, smem, acc, bsum, false);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  float* dst = a.gpart + static_cast<int64_t>(sp) * a.r * a.r;
#pragma unroll
  for (int i = 0; i < TL::TM; ++i)
#pragma unroll
    for (int j = 0; j < TL::TN; ++j) {
      const int64_t col = n0 + wn * TL::TN * 32 + j * 32 + (lane & 31);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm * TL::TM * 32 + i * 32 + 8 * (q / 4) + 4 * (lane >> 5) + (q % 4);
        if (row < a.r && col < a.r) dst[row * a.r + col] = acc[i][j][q];
      }
    }
}

// G'[a][b] = (s/2) * sum_sp Gpart[sp][a][b] in fp64 (entries below the tiled
// diagonal are read from their mirror), then G'hi = round(G'), G'lo =
// round(G' - G'hi).  G'hi + G'lo carries about 16 (bf16) or 22 (fp16)
// significant bits of G'.
template <int DT>
__global__ __launch_bounds__(256) void gram_finalize(const float* gpart, int splitG, int64_t r, float half_s,
                                                     typename Dt<DT>::T* ghi, typename Dt<DT>::T* glo) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= r * r) return;
  const int64_t ra = idx / r, rb = idx % r;
  const int64_t src = (ra / TileG::BM <= rb / TileG::BN) ? idx : rb * r + ra;
  double sum = 0.0;
  for (int sp = 0; sp < splitG; ++sp) sum += static_cast<double>(gpart[static_cast<int64_t>(sp) * r * r + src]);
  const double gp = static_cast<double>(half_s) * sum;
  const typename Dt<DT>::T hi = Dt<DT>::from_d(gp);
  const double rem = gp - static_cast<double>(Dt<DT>::to_f(hi));
  ghi[idx] = hi;
  glo[idx] = Dt<DT>::from_d(rem);
}

struct WArgs {
  WStages sm;
  int64_t nRB, S, total;
  int nTiles, nSplit;
  float* base_part;   // [nSplit][out]
  float* cross_part;  // [nSplit][nTiles][out]
};

template <int DT, bool VEC>
__global__ __launch_bounds__(TileW::NT, 2) void wstream_kernel(WArgs a) {
  using TL = TileW;
  __shared__ __attribute__((aligned(16))) typename Dt<DT>::T smem[TL::LDS_ELEMS];
  __shared__ float red[TL::WN][TL::BM];
  const int64_t v = xcd_logical_index();
  if (v >= a.total) return;
  const int nt = static_cast<int>(v % a.nTiles);
  const int64_t rb = (v / a.nTiles) % a.nRB;
  const int sp = static_cast<int>(v / (static_cast<int64_t>(a.nTiles) * a.nRB));
  const int64_t m0 = rb * TL::BM, n0 = static_cast<int64_t>(nt) * TL::BN;
  const int64_t st0 = a.S * sp / a.nSplit, st1 = a.S * (sp + 1) / a.nSplit;
  const int64_t out = a.sm.out, r = a.sm.r;

  f32x16 acc[TL::TM][TL::TN];
#pragma unroll
  for (int i = 0; i < TL::TM; ++i)
#pragma unroll
    for (int j = 0; j < TL::TN; ++j) acc[i][j] = f32x16{};
  float bsum[TL::XCH] = {};
  const bool want_base = (nt == 0);
  mainloop<DT, VEC, TL>(a.sm, st0, st1, m0, n0, smem, acc, bsum, want_base);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  using T = typename Dt<DT>::T;
  const T* B = static_cast<const T*>(a.sm.B);

  // rs[i][q] = sum over this lane's columns of B[row][col] * acc[row][col]
  float rs[TL::TM][16];
#pragma unroll
  for (int i = 0; i < TL::TM; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) rs[i][q] = 0.0f;
#pragma unroll
  for (int j = 0; j < TL::TN; ++j) {
    const int64_t col = n0 + wn * TL::TN * 32 + j * 32 + (lane & 31);
    const bool cv = col < r;
#pragma unroll
    for (int i = 0; i < TL::TM; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm * TL::TM * 32 + i * 32 + 8 * (q / 4) + 4 * (lane >> 5) + (q % 4);
        const float bv = (cv && row < out) ? Dt<DT>::to_f(B[row * r + col]) : 0.0f;
        rs[i][q] = __builtin_fmaf(bv, acc[i][j][q], rs[i][q]);
      }
  }
  // reduce over the 32 columns held by each half-wave
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1)
#pragma unroll
    for (int i = 0; i < TL::TM; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) rs[i][q] += __shfl_xor(rs[i][q], off, 64);
  if ((lane & 31) == 0) {
#pragma unroll
    for (int i = 0; i < TL::TM; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) red[wn][wm * TL::TM * 32 + i * 32 + 8 * (q / 4) + 4 * (lane >> 5) + (q % 4)] = rs[i][q];
  }
  // base term: the 8 loader lanes of a row are consecutive
  if (want_base) {
#pragma unroll
    for (int i = 0; i < TL::XCH; ++i) {
      float b = bsum[i];
#pragma unroll
      for (int off = 1; off < TL::CPR; off <<= 1) b += __shfl_xor(b, off, 64);
      const int64_t row = m0 + tid / TL::CPR + i * TL::RPP;
      if ((tid % TL::CPR) == 0 && row < out) a.base_part[static_cast<int64_t>(sp) * out + row] = b;
    }
  }
  __syncthreads();
  if (tid < TL::BM && m0 + tid < out) {
    float c = 0.0f;
#pragma unroll
    for (int w = 0; w < TL::WN; ++w) c += red[w][tid];
    a.cross_part[(static_cast<int64_t>(sp) * a.nTiles + nt) * out + m0 + tid] = c;
  }
}

__global__ __launch_bounds__(256) void norm_finalize(const float* base_part, const float* cross_part, int nSplit,
                                                     int nTiles, int64_t out, float s, float* norm_out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= out) return;
  double b = 0.0, c = 0.0;
  for (int sp = 0; sp < nSplit; ++sp) b += static_cast<double>(base_part[static_cast<int64_t>(sp) * out + i]);
  for (int q = 0; q < nSplit * nTiles; ++q) c += static_cast<double>(cross_part[static_cast<int64_t>(q) * out + i]);
  const double n2 = b + 2.0 * static_cast<double>(s) * c;
  norm_out[i] = static_cast<float>(n2 > 0.0 ? sqrt(n2) : 0.0);
}

constexpr int kSlotsW = 512;  // resident W-stream workgroups: 256 CUs x 2

template <int DT>
hipError_t launch_norm_t(const NormPlan& p, const NormArgs& a, bool vec) {
  char* ws = static_cast<char*>(a.ws);
  using T = typename Dt<DT>::T;
  T* ghi = reinterpret_cast<T*>(ws + p.off_ghi);
  T* glo = reinterpret_cast<T*>(ws + p.off_glo);
  if (p.r > 0) {
    GramArgs g{a.A, p.in, p.r, p.Sg, p.nTg, p.nUpper, p.splitG, reinterpret_cast<float*>(ws + p.off_gpart)};
    const int64_t n = static_cast<int64_t>(p.nUpper) * p.splitG;
    const dim3 grid(static_cast<unsigned>(cdiv(n, 8) * 8));
    if (vec)
      hipLaunchKernelGGL((gram_kernel<DT, true>), grid, dim3(TileG::NT), 0, a.stream, g);
    else
      hipLaunchKernelGGL((gram_kernel<DT, false>), grid, dim3(TileG::NT), 0, a.stream, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gram_finalize<DT>), dim3(static_cast<unsigned>(cdiv(p.r * p.r, 256))), dim3(256), 0, a.stream,
                       g.gpart, p.splitG, p.r, a.s * 0.5f, ghi, glo);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  WArgs w;
  w.sm = WStages{a.W0, a.A, a.B, ghi, glo, p.out, p.in, p.r, p.S1, p.S2};
  w.nRB = p.nRB;
  w.S = p.S;
  w.nTiles = p.nTiles;
  w.nSplit = p.nSplit;
  w.total = p.nRB * p.nTiles * p.nSplit;
  w.base_part = reinterpret_cast<float*>(ws + p.off_base);
  w.cross_part = reinterpret_cast<float*>(ws + p.off_cross);
  const dim3 grid(static_cast<unsigned>(cdiv(w.total, 8) * 8));
  if (vec)
    hipLaunchKernelGGL((wstream_kernel<DT, true>), grid, dim3(TileW::NT), 0, a.stream, w);
  else
    hipLaunchKernelGGL((wstream_kernel<DT, false>), grid, dim3(TileW::NT), 0, a.stream, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(norm_finalize, dim3(static_cast<unsigned>(cdiv(p.out, 256))), dim3(256), 0, a.stream,
                     w.base_part, w.cross_part, p.nSplit, p.nTiles, p.out, a.s, a.norm_out);
  return hipGetLastError();
}

}  // namespace

size_t norm_scratch_bound(int64_t out, int64_t r) {
  return static_cast<size_t>(4 * (out * r + r * r) + 64 * out + 256);
}

NormPlan make_norm_plan(int64_t out, int64_t in, int64_t r, int dtype) {
  NormPlan p;
  p.out = out;
  p.in = in;
  p.r = r;
  p.dtype = dtype;
  if (out <= 0) return p;
  const int64_t e = 2;  // bytes per storage element (bf16, fp16)
  p.nRB = cdiv(out, TileW::BM);
  p.nTiles = static_cast<int>(std::max<int64_t>(1, cdiv(r, TileW::BN)));
  p.S1 = cdiv(in, TileW::BK);
  p.S2 = cdiv(r, TileW::BK);
  p.S = p.S1 + 2 * p.S2;
  // K splits: minimise (rounds of resident workgroups) x (stages per workgroup),
  // keeping at least 4 stages per workgroup; ties go to fewer splits.
  {
    const int64_t per = p.nRB * p.nTiles;
    const int64_t maxs = std::max<int64_t>(1, std::min<int64_t>(64, p.S / 4));
    int64_t best = -1, bestc = 0;
    for (int64_t k = 1; k <= maxs; ++k) {
      const int64_t cost = cdiv(per * k, kSlotsW) * cdiv(std::max<int64_t>(p.S, 1), k);
      if (best < 0 || cost < bestc) {
        best = k;
        bestc = cost;
      }
    }
    p.nSplit = static_cast<int>(best);
  }
  if (r > 0) {
    p.nTg = static_cast<int>(cdiv(r, TileG::BM));
    p.nUpper = p.nTg * (p.nTg + 1) / 2;
    p.Sg = cdiv(in, TileG::BK);
    p.splitG = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(cdiv(256, p.nUpper), std::max<int64_t>(1, p.Sg / 4))));
  }
  auto layout = [&]() {
    size_t off = 0;
    p.off_gpart = off;
    off += align16(static_cast<size_t>(p.splitG) * r * r * 4);
    p.off_ghi = off;
    off += align16(static_cast<size_t>(r * r * e));
    p.off_glo = off;
    off += align16(static_cast<size_t>(r * r * e));
    p.off_base = off;
    off += align16(static_cast<size_t>(p.nSplit) * out * 4);
    p.off_cross = off;
    off += align16(static_cast<size_t>(p.nSplit) * p.nTiles * out * 4);
    p.bytes = off;
  };
  layout();
  // stay inside the factored memory bound: fewer Gram splits first, then fewer K splits
  const size_t bound = norm_scratch_bound(out, r);
  while (p.bytes > bound && p.splitG > 1) {
    --p.splitG;
    layout();
  }
  while (p.bytes > bound && p.nSplit > 1) {
    --p.nSplit;
    layout();
  }
  return p;
}

hipError_t launch_norm(const NormPlan& p, const NormArgs& a, bool vec) {
  if (p.out <= 0) return hipSuccess;
  return p.dtype == 0 ? launch_norm_t<0>(p, a, vec) : launch_norm_t<1>(p, a, vec);
}

}  // namespace dora
