// Factored DoRA weight norm for gfx950.
//
//   n_i^2 = ||W0_i||^2 + 2 s B_i U_i^T + s^2 B_i G B_i^T,  U = W0 A^T, G = A A^T
//
// (press summary of arXiv:2603.22276, paragraph on the "factored norm": base,
// cross and Gram terms replace the out x in matrix B*A; scratch is
// O(out*r + r*r)).
//
// Kernels, in launch order:
//   gram_dma          (16-byte path) split-K partials of G = A A^T on the
//   gram_partial      (general path) upper-triangular tiles (G is symmetric),
//                     MFMA 32x32x16 with fp32 accumulation;
//   gram_finalize     fixed-order sum of the partials, then G' = (s/2) G split
//                     into two storage-dtype matrices G'hi + G'lo (written with
//                     their mirror images);
//   wstream_k64       (16-byte path, rank tiles of 128, 256 and 384; 128-byte
//   wstream_general    row segments, DMA waves beside the MFMA waves; general
//                     path: register-staged loads) one pass per rank tile
//                     over W0.  A workgroup owns a block of rows
//                     x a block of rank columns x a slice of the augmented K axis
//                       [ W0 | B | B ] . [ A | G'hi | G'lo ]^T
//                     so its accumulator holds U + B G' = U + (s/2) B G for those
//                     rows and columns.  The epilogue reduces B_ij * acc_ij over
//                     its columns, since 2s * sum_j B_ij (U + (s/2) B G)_ij =
//                     cross_i + gram_i, and the W0 elements the waves read for
//                     the MFMAs are also squared for the base term.  U is never
//                     written to memory.  On the 16-byte path the last
//                     workgroup of each row block also finalizes its norms;
//   norm_finalize     (general path) n_i = sqrt(max(sum of partials, 0)) in
//                     fp64, rounded to fp32.
//
// All reductions are in fixed order, so the result is bitwise reproducible.
#include <algorithm>

#include "dma_common.hpp"
#include "dora_common.hpp"
#include "norm_kernels.hpp"

namespace dora {

namespace {

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align16(size_t x) { return (x + 15) & ~static_cast<size_t>(15); }

// Workgroup numbering (xcd_logical_index, dma_common.hpp): each XCD receives a
// contiguous range of the logical work list (one K slice of A per XCD's L2, and
// the rank tiles of a row block together).

// ---------------------------------------------------------------------------
// Gram matrix

constexpr int kGramU = 8;  // K steps per batch of fragment loads

// One entry g' of G' = scale * G as the storage-dtype pair hi = round(g'),
// lo = round(g' - hi), written at (row, col) and, for an entry of an
// off-diagonal tile, at its mirror (col, row).  Used when a single K split
// covers the whole K axis (no partial sums to add): the Gram kernel then
// writes G'hi/G'lo itself and the plan holds no fp32 partials.
template <int DT>
__device__ inline void gram_store_pair(typename Dt<DT>::T* ghi, typename Dt<DT>::T* glo, int64_t r, int64_t row,
                                       int64_t col, float gp, bool mirror) {
  using T = typename Dt<DT>::T;
  const T hi = Dt<DT>::from_f(gp);
  const T lo = Dt<DT>::from_f(gp - Dt<DT>::to_f(hi));
  ghi[row * r + col] = hi;
  glo[row * r + col] = lo;
  if (mirror) {
    ghi[col * r + row] = hi;
    glo[col * r + row] = lo;
  }
}

// Split-K partial products of G on its upper-triangular 32x32 tiles (G is
// symmetric).  Workgroup (tile, split) = 4 waves; each wave accumulates a
// quarter of the split's K steps with MFMA 32x32x16, its operand fragments
// loaded straight from global memory (A is small and L2/MALL resident) in
// batches of kGramU steps; the four wave partials are summed in LDS in a fixed
// order and stored as the split's 32x32 tile.
template <int DT, bool DIRECT>
__global__ __launch_bounds__(256) void gram_partial(const typename Dt<DT>::T* A, int64_t in, int64_t r, int nT,
                                                    int splitG, float* gpart, float scale, typename Dt<DT>::T* ghi,
                                                    typename Dt<DT>::T* glo) {
  using T = typename Dt<DT>::T;
  using V8 = typename Dt<DT>::V8;
  __shared__ float red[4][32 * 32];
  const int nUpper = nT * (nT + 1) / 2;
  // XCD-aware: with splitG a multiple of 8 each XCD takes whole K splits, so
  // its L2 holds one K slice of A
  const int64_t v = xcd_logical_index();
  if (v >= static_cast<int64_t>(nUpper) * splitG) return;
  int u = static_cast<int>(v % nUpper);
  const int sp = static_cast<int>(v / nUpper);
  int ti = 0;
  while (u >= nT - ti) {
    u -= nT - ti;
    ++ti;
  }
  const int tj = ti + u;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t xr = static_cast<int64_t>(ti) * 32 + (lane & 31);
  const int64_t yr = static_cast<int64_t>(tj) * 32 + (lane & 31);
  const int64_t nk = cdiv(in, 16);
  const int64_t part = static_cast<int64_t>(sp) * 4 + wave;
  const int64_t kb0 = nk * part / (4 * splitG), kb1 = nk * (part + 1) / (4 * splitG);
  const int koff = (lane >> 5) * 8;

  // clamped, unconditional loads; out-of-range rows and K are selected to zero
  const int64_t xrc = xr < r ? xr : r - 1, yrc = yr < r ? yr : r - 1;
  auto frag = [&](int64_t row, int64_t rowc, int64_t k) -> V8 {
    const bool ok = row < r && k < in;
    V8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const T t = A[rowc * in + (k + j < in ? k + j : in - 1)];
      v[j] = (ok && k + j < in) ? t : static_cast<T>(0.0f);
    }
    return v;
  };

  f32x16 acc = {};
  int64_t kb = kb0;
  for (; kb + kGramU <= kb1; kb += kGramU) {
    V8 x[kGramU], y[kGramU];
#pragma unroll
    for (int q = 0; q < kGramU; ++q) {
      x[q] = frag(xr, xrc, (kb + q) * 16 + koff);
      y[q] = frag(yr, yrc, (kb + q) * 16 + koff);
    }
#pragma unroll
    for (int q = 0; q < kGramU; ++q) acc = Dt<DT>::mfma32(x[q], y[q], acc);
  }
  for (; kb < kb1; ++kb) acc = Dt<DT>::mfma32(frag(xr, xrc, kb * 16 + koff), frag(yr, yrc, kb * 16 + koff), acc);

#pragma unroll
  for (int q = 0; q < 16; ++q) red[wave][(8 * (q / 4) + 4 * (lane >> 5) + (q % 4)) * 32 + (lane & 31)] = acc[q];
  __syncthreads();
  float* dst = gpart + static_cast<int64_t>(sp) * r * r;
  for (int e = threadIdx.x; e < 1024; e += 256) {
    const int64_t row = static_cast<int64_t>(ti) * 32 + e / 32, col = static_cast<int64_t>(tj) * 32 + e % 32;
    if (row < r && col < r) {
      const float g = (red[0][e] + red[1][e]) + (red[2][e] + red[3][e]);
      if constexpr (DIRECT)
        gram_store_pair<DT>(ghi, glo, r, row, col, scale * g, ti != tj);
      else
        dst[row * r + col] = g;
    }
  }
}

// G'[a][b] = (s/2) * (sum over splits of the partials, in split order) for the
// entries of the upper tiles, split into G'hi = round(G') and G'lo =
// round(G' - G'hi) in the storage dtype and written at (a, b) and its mirror
// (b, a).  G'hi + G'lo carries about 16 (bf16) or 22 (fp16) significant bits.
// One workgroup per 8-row strip of an upper 32 x 32 tile (tr <= tc), one entry
// per thread: the direct writes run 64 bytes along a row, the mirror goes
// through LDS and is written in 16-byte runs.  Loads past r read a valid
// address and are dropped, so every thread issues the same loads.
template <int DT>
__global__ __launch_bounds__(256) void gram_finalize(const float* gpart, int splitG, int64_t r, float half_s,
                                                     typename Dt<DT>::T* ghi, typename Dt<DT>::T* glo) {
  using T = typename Dt<DT>::T;
  __shared__ float tile[8][33];
  const int nT = static_cast<int>((r + 31) / 32);
  int u = static_cast<int>(blockIdx.x >> 2);
  int tr = 0;
  while (u >= nT - tr) {
    u -= nT - tr;
    ++tr;
  }
  const int tc = tr + u;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t row0 = static_cast<int64_t>(tr) * 32 + (blockIdx.x & 3) * 8, col0 = static_cast<int64_t>(tc) * 32;
  const int64_t row = row0 + ty, col = col0 + tx;
  const bool inside = row < r && col < r;
  const float* src = gpart + (inside ? row * r + col : 0);
  const int64_t stride = r * r;
  float g = 0.0f;
  // groups of up to kFinSplits partials, all loaded before they are summed
  // pairwise; the groups are added in order
  constexpr int kFinSplits = 32;
  for (int s0 = 0; s0 < splitG; s0 += kFinSplits) {
    float a[kFinSplits];
#pragma unroll
    for (int k = 0; k < kFinSplits; ++k) {
      const int sp = s0 + k < splitG ? s0 + k : splitG - 1;
      a[k] = src[sp * stride];
    }
#pragma unroll
    for (int k = 0; k < kFinSplits; ++k)
      if (s0 + k >= splitG) a[k] = 0.0f;
#pragma unroll
    for (int w = 1; w < kFinSplits; w *= 2)
#pragma unroll
      for (int k = 0; k < kFinSplits; k += 2 * w) a[k] += a[k + w];
    g += a[0];
  }
  const float gp = half_s * g;
  if (inside) {
    const T hi = Dt<DT>::from_f(gp);
    ghi[row * r + col] = hi;
    glo[row * r + col] = Dt<DT>::from_f(gp - Dt<DT>::to_f(hi));
  }
  if (tr == tc) return;  // the diagonal tile holds both halves itself
  tile[ty][tx] = gp;
  __syncthreads();
  const int ii = threadIdx.x & 7, jj = threadIdx.x >> 3;
  const int64_t mrow = col0 + jj, mcol = row0 + ii;  // mirror of (row0 + ii, col0 + jj)
  if (mrow < r && mcol < r) {
    const float z = tile[ii][jj];
    const T hi = Dt<DT>::from_f(z);
    ghi[mrow * r + mcol] = hi;
    glo[mrow * r + mcol] = Dt<DT>::from_f(z - Dt<DT>::to_f(hi));
  }
}

// ---------------------------------------------------------------------------
// Shared pieces of the W stream

// A row-major operand panel: rows x klen valid elements, ld elements per row.
struct Operand {
  const void* p;
  int64_t ld, rows, klen;
};

// Stage map of the fused W stream: stage st covers BK columns of one segment of
// the augmented K axis [W0 | B | B] . [A | G'hi | G'lo]^T.
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

struct WArgs {
  WStages sm;
  int64_t nRB, S, total;
  int nTiles, nSplit;
  float* base_part;   // [nSplit][out]
  float* cross_part;  // [nSplit][nTiles][out]
  int skip_base;      // the base term comes from a cache: no squares, no base partials
  float* acc_part = nullptr;  // [nSplit][out][r]: store the accumulators U + B G' instead of reducing them
  // Norm finalize in the epilogue: the last workgroup of each row block (a
  // counter per row block, zeroed by the Gram kernel of the same call) sums
  // the partials and writes the norm.  Null: a separate norm_finalize launch.
  unsigned* fin_count = nullptr;
  float* norm_out = nullptr;
  const float* base_sq = nullptr;
  float s = 0.0f;
};

// Partials per sum that the finalizes load all at once before adding them.
constexpr int kFinParts = 8;

// sum_{q < n} p[q * stride] in fp64, in order, each load at device scope (it
// reads through this XCD's L2 to the device-coherent level, so it sees the
// partials that workgroups on other XCDs wrote through with device-scope
// stores); loads go out in groups of 8 before the group is added.
__device__ inline double ordered_sum_device(const float* p, int n, int64_t stride) {
  double acc = 0.0;
  int q = 0;
  for (; q + 8 <= n; q += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = __hip_atomic_load(p + static_cast<int64_t>(q + u) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += static_cast<double>(v[u]);
  }
  for (; q < n; ++q)
    acc += static_cast<double>(
        __hip_atomic_load(p + static_cast<int64_t>(q) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return acc;
}

// Epilogue shared by both W-stream kernels.  The MFMAs take the rank-side
// fragment as their first operand, so acc[i][j] is the transposed 32x32 tile:
// lane l holds W0 row m0 + wm*TM*32 + i*32 + l%32 (the tile column) and, in
// register q, rank column n0 + wn*TN*32 + j*32 + 8*(q/4) + 4*(l/32) + q%4 of
// U + B G'.  Each lane therefore needs B[row][4 consecutive columns] per
// register group (one 8-byte load on the 16-byte path), sums its products in
// registers, adds the other half-wave's sum, and the waves along the rank axis
// are combined in LDS in a fixed order.
template <int DT, int TM, int TN, int WM, int WN, int BM, bool VEC>
__device__ inline void cross_epilogue(const WArgs& a, int sp, int nt, int64_t m0, int64_t n0,
                                      const f32x16 (&acc)[TM][TN], float (*red)[BM]) {
  using T = typename Dt<DT>::T;
  using T4 = T __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t out = a.sm.out, r = a.sm.r;
  const T* B = static_cast<const T*>(a.sm.B);
  const int h = lane >> 5;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t row = m0 + wm * TM * 32 + i * 32 + (lane & 31);
    const bool rv = row < out;
    // clamped, unconditional loads (no divergent branches around them); the
    // products of rows or columns outside the matrices are selected away
    const int64_t rowc = rv ? row : out - 1;
    float rs = 0.0f;
    if (r > 0) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        T4 b4[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t col = n0 + wn * TN * 32 + j * 32 + 8 * g + 4 * h;
          if (VEC) {
            // r is a multiple of 8: a 4-column group is wholly inside or outside
            const int64_t colc = col < r ? col : r - 4;
            b4[g] = *reinterpret_cast<const T4*>(B + rowc * r + colc);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) b4[g][e] = B[rowc * r + (col + e < r ? col + e : r - 1)];
          }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t col = n0 + wn * TN * 32 + j * 32 + 8 * g + 4 * h;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float t = __builtin_fmaf(Dt<DT>::to_f(b4[g][e]), acc[i][j][4 * g + e], rs);
            rs = (rv && col + e < r) ? t : rs;
          }
        }
      }
    }
    rs += __shfl_xor(rs, 32, 64);
    if (h == 0) red[wn][wm * TM * 32 + i * 32 + (lane & 31)] = rs;
  }
  __syncthreads();
  if (tid < BM && m0 + tid < out) {
    float c = 0.0f;
#pragma unroll
    for (int w = 0; w < WN; ++w) c += red[w][tid];
    a.cross_part[(static_cast<int64_t>(sp) * a.nTiles + nt) * out + m0 + tid] = c;
  }
}

// ---------------------------------------------------------------------------
// Epilogues shared by the W stream's 16-byte path (wstream_k64, below).

// Epilogue of the 16-byte path for the norm backward: the workgroup's split-K
// partial of U + B G' itself, written to acc_part[sp][row][col] in fp32.  Lane
// l of wave (wm, wn) holds, for tile (i, j), row m0 + 32*(wm*TMW + i) + l%32
// and in register q rank column n0 + 32*(wn*TN + j) + 16*(l/32) + q (the
// rank-side panel is fetched in the fragment row order), so each lane writes
// 16 consecutive floats per tile; r % 8 == 0 makes each half of them wholly
// inside or outside the matrix.
template <class TL>
__device__ inline void dma_store_acc(const WArgs& a, int sp, int64_t m0, int64_t n0,
                                     const f32x16 (&acc)[TL::TMW][TL::TN]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const int h = lane >> 5, frow = lane & 31;
  const int64_t out = a.sm.out, r = a.sm.r;
  float* part = a.acc_part + static_cast<int64_t>(sp) * out * r;
#pragma unroll
  for (int i = 0; i < TL::TMW; ++i) {
    const int64_t row = m0 + 32 * (wm * TL::TMW + i) + frow;
    if (row >= out) continue;
#pragma unroll
    for (int j = 0; j < TL::TN; ++j) {
      const int64_t col = n0 + 32 * (wn * TL::TN + j) + 16 * h;
      if (col >= r) continue;
      float* dst = part + row * r + col;
      *reinterpret_cast<f32x4*>(dst) = f32x4{acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[i][j][4], acc[i][j][5], acc[i][j][6], acc[i][j][7]};
      if (col + 8 < r) {
        *reinterpret_cast<f32x4*>(dst + 8) = f32x4{acc[i][j][8], acc[i][j][9], acc[i][j][10], acc[i][j][11]};
        *reinterpret_cast<f32x4*>(dst + 12) = f32x4{acc[i][j][12], acc[i][j][13], acc[i][j][14], acc[i][j][15]};
      }
    }
  }
}

// Epilogue of the 16-byte path: the cross term's row sums
// sum_c B[m][c] * (W0 A^T + B G')[m][c] over the workgroup's rank columns.
// The B tile (BM rows x BN rank columns) is brought into the free stage area
// by DMA, in passes of as many 32-row blocks as fit.  Row m of a pass sits at
// m * BN * 2 bytes, its logical 16-byte chunk c in slot (c & ~15) | ((c ^ m) & 15),
// so the reads of 16 consecutive rows at one chunk hit 16 distinct bank
// groups.  A lane needs, per rank tile, the 16 consecutive B columns matching
// its accumulator registers: two 16-byte LDS reads, whose slots depend on the
// lane only (tile rows start on multiples of 32).  Rank columns past r hold
// zero in both operands; a chunk there is still left out of the sum.
template <int DT, class TL>
__device__ inline void dma_cross_epilogue(const WArgs& a, int sp, int nt, int64_t m0, int64_t n0,
                                          const f32x16 (&acc)[TL::TMW][TL::TN], const float (&bs)[TL::NP],
                                          bool want_base, float (*red)[TL::BM], char* smem, uint32_t lds0,
                                          __amdgpu_buffer_rsrc_t rb) {
  constexpr int CPR = TL::BN / 8;  // 16-byte chunks per B-tile row
  constexpr int RPP = TL::RPP;     // rows per pass
  constexpr int NPASS = (TL::BM + RPP - 1) / RPP;
  constexpr int INSTR = RPP * CPR / 64;  // 1 KiB DMA instructions per pass
  static_assert(CPR % 16 == 0 && RPP % 32 == 0, "swizzle groups of 16 chunks, passes of whole row tiles");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const int h = lane >> 5, frow = lane & 31;
  const int64_t out = a.sm.out, r = a.sm.r;
  // waves past the NW tile waves (DMA-only waves) hold no accumulators: they
  // take part in the barriers only
  const bool worker = wave < TL::NW;
  const int cols_here = static_cast<int>(std::min<int64_t>(std::max<int64_t>(r - n0, 0), TL::BN));
  // byte offsets within a row of the lane's chunks (tile j, chunk k of two)
  uint32_t cofs[TL::TN][2];
#pragma unroll
  for (int j = 0; j < TL::TN; ++j)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = wn * TL::TN * 4 + j * 4 + 2 * h + k;
      cofs[j][k] = static_cast<uint32_t>((c & ~15) | ((c ^ frow) & 15)) * 16u;
    }
  const uint32_t lrow = lds0 + static_cast<uint32_t>(frow * CPR * 16);
  float rs[TL::TMW][2];
#pragma unroll
  for (int i = 0; i < TL::TMW; ++i) rs[i][0] = rs[i][1] = 0.0f;

#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    const int row_base = pass * RPP;
    __syncthreads();  // stage buffers (or the previous pass) no longer read
    if (worker && cols_here > 0) {
      for (int q = wave; q < INSTR; q += TL::NW) {
        const int sl = q * 64 + lane;
        const int rl = sl / CPR, p = sl % CPR;
        const int c = (p & ~15) | ((p ^ rl) & 15);  // logical chunk held by slot p
        const int col = c * 8;
        const uint32_t off =
            col < cols_here ? static_cast<uint32_t>(((row_base + rl) * r + n0 + col) * 2) : kOob;
        dma16(rb, smem + q * 1024, off);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
    if (worker && cols_here > 0) {
#pragma unroll
      for (int i = 0; i < TL::TMW; ++i) {
        const int r32 = wm * TL::TMW * 32 + i * 32;  // first tile row within the workgroup tile
        if (r32 < row_base || r32 >= row_base + RPP) continue;
        const uint32_t rbase = lrow + static_cast<uint32_t>((r32 - row_base) * CPR * 16);
#pragma unroll
        for (int j = 0; j < TL::TN; ++j) {
          u32x4 w[2];
          w[0] = lds_read16(rbase + cofs[j][0]);
          w[1] = lds_read16(rbase + cofs[j][1]);
          lds_wait();
          tie(w[0]);
          tie(w[1]);
          const int c0 = wn * TL::TN * 4 + j * 4 + 2 * h;
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const typename Dt<DT>::V8 b = __builtin_bit_cast(typename Dt<DT>::V8, w[k]);
            float u0 = Dt<DT>::to_f(b[0]) * acc[i][j][8 * k];
            float u1 = Dt<DT>::to_f(b[1]) * acc[i][j][8 * k + 1];
#pragma unroll
            for (int e = 2; e < 8; e += 2) {
              u0 = __builtin_fmaf(Dt<DT>::to_f(b[e]), acc[i][j][8 * k + e], u0);
              u1 = __builtin_fmaf(Dt<DT>::to_f(b[e + 1]), acc[i][j][8 * k + e + 1], u1);
            }
            rs[i][k] += (c0 + k) * 8 < cols_here ? u0 + u1 : 0.0f;
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TL::TMW; ++i) {
    float v = rs[i][0] + rs[i][1];
    v += __shfl_xor(v, 32, 64);
    if (worker && h == 0) red[wn][wm * TL::TMW * 32 + i * 32 + frow] = v;
  }
  if (want_base) {
    // wave wn holds the squares of pairs p = wn + WN*t (tile p/KS); at most one
    // t of a wave falls on a given tile
#pragma unroll
    for (int i = 0; i < TL::TMW; ++i) {
      float b = 0.0f;
#pragma unroll
      for (int t = 0; t < TL::NP; ++t)
        if ((wn + TL::WN * t) / TL::KS == i) b = bs[t];
      b += __shfl_xor(b, 32, 64);
      if (worker && h == 0) red[TL::WN + wn][wm * TL::TMW * 32 + i * 32 + frow] = b;
    }
  }
  __syncthreads();
  const bool fused = a.fin_count != nullptr;
  if (tid < TL::BM && m0 + tid < out) {
    float c = 0.0f;
#pragma unroll
    for (int w = 0; w < TL::WN; ++w) c += red[w][tid];
    float* cp = a.cross_part + (static_cast<int64_t>(sp) * a.nTiles + nt) * out + m0 + tid;
    if (fused)  // written through to the device-coherent level
      __hip_atomic_store(cp, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *cp = c;
    if (want_base) {
      float b = 0.0f;
#pragma unroll
      for (int w = 0; w < TL::WN; ++w) b += red[TL::WN + w][tid];
      float* bp = a.base_part + static_cast<int64_t>(sp) * out + m0 + tid;
      if (fused)
        __hip_atomic_store(bp, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        *bp = b;
    }
  }
  if (!fused) return;
  // The last of the row block's nSplit * nTiles workgroups computes its norms
  // (the sums of norm_finalize, in the same order).  Every thread's partial
  // stores are complete before the workgroup's counter increment; the loads of
  // the last workgroup follow its increment.
  wait_vmcnt<0>();
  __syncthreads();
  int* flag = reinterpret_cast<int*>(&red[0][0]);
  if (tid == 0) {
    const unsigned total = static_cast<unsigned>(a.nSplit) * static_cast<unsigned>(a.nTiles);
    const unsigned old = __hip_atomic_fetch_add(a.fin_count + m0 / TL::BM, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    *flag = old == total - 1 ? 1 : 0;
  }
  __syncthreads();
  if (*flag && tid < TL::BM && m0 + tid < out) {
    const int64_t i = m0 + tid;
    const int nc = a.nSplit * a.nTiles;
    double b, c;
    if (a.nSplit <= kFinParts && nc <= kFinParts) {
      // every partial of both sums in flight before the first addition (one
      // round trip to the device-coherent level); the additions keep split order
      // (unconditional loads of clamped indices: a load under a condition
      // would be waited for on its own)
      float vb[kFinParts], vc[kFinParts];
      const float* bp = a.base_sq ? a.base_sq + i : a.base_part + i;
      const int nb = a.base_sq ? 1 : a.nSplit;
#pragma unroll
      for (int q = 0; q < kFinParts; ++q) {
        vb[q] = __hip_atomic_load(bp + static_cast<int64_t>(q < nb ? q : nb - 1) * out, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        vc[q] = __hip_atomic_load(a.cross_part + i + static_cast<int64_t>(q < nc ? q : nc - 1) * out,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      b = 0.0;
      c = 0.0;
#pragma unroll
      for (int q = 0; q < kFinParts; ++q) {
        b += q < nb ? static_cast<double>(vb[q]) : 0.0;
        c += q < nc ? static_cast<double>(vc[q]) : 0.0;
      }
    } else {
      b = a.base_sq ? static_cast<double>(a.base_sq[i]) : ordered_sum_device(a.base_part + i, a.nSplit, out);
      c = ordered_sum_device(a.cross_part + i, nc, out);
    }
    const double n2 = b + 2.0 * static_cast<double>(a.s) * c;
    a.norm_out[i] = static_cast<float>(n2 > 0.0 ? sqrt(n2) : 0.0);
  }
}

// ---------------------------------------------------------------------------
// Gram matrix, 16-byte path: split-K partials of G = A A^T on the upper 64x64
// blocks (G is symmetric).  Workgroup (block, split) = 4 waves, one 32x32
// sub-tile each.  K stages of 64 go global -> LDS by DMA: one wave
// instruction moves 8 rows x 128 bytes (whole cache lines), lane l taking row
// l/8 and the logical 16-byte chunk (l%8) ^ ((row/2)%8), which lands in LDS
// slot l%8; the fragment reads of 16 consecutive rows at one logical chunk then
// hit 16 distinct bank groups.  Rows past r and K past in read zero.
constexpr int kGramStage = 2 * 64 * 128;  // X and Y panels, 64 rows x 128 bytes
constexpr int kGramL = 4;                 // DMA instructions per wave per stage

template <int DT, int kGramNS, bool DIRECT>
__global__ __launch_bounds__(256) void gram_dma(const typename Dt<DT>::T* A, int in, int r, int nB, int splitG,
                                                float* gpart, float scale, typename Dt<DT>::T* ghi,
                                                typename Dt<DT>::T* glo, unsigned* fin_count, int n_count) {
  using V8 = typename Dt<DT>::V8;
  static_assert(kGramNS >= 3 && kGramNS <= 8 && (kGramNS - 2) * kGramL < 64, "ring slots");
  __shared__ __attribute__((aligned(1024))) char smem[kGramNS * kGramStage];
  const int nUpper = nB * (nB + 1) / 2;
  // XCD-aware: consecutive logical indices share a K split, so each XCD's L2
  // holds one K slice of A
  const int v = static_cast<int>(xcd_logical_index());
  // the W stream's per-row-block counters of this call start at zero
  if (v == 0 && fin_count)
    for (int i = threadIdx.x; i < n_count; i += 256) fin_count[i] = 0u;
  if (v >= nUpper * splitG) return;
  int u = v % nUpper;
  const int sp = v / nUpper;
  int bi = 0;
  while (u >= nB - bi) {
    u -= nB - bi;
    ++bi;
  }
  const int bj = bi + u;
  const int x0 = bi * 64, y0 = bj * 64;
  const int nk = (in + 63) / 64;
  const int st0 = static_cast<int>(static_cast<int64_t>(nk) * sp / splitG);
  const int st1 = static_cast<int>(static_cast<int64_t>(nk) * (sp + 1) / splitG);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_t*)smem));

  auto rsrc = [&](int row0) {
    const int nrows = std::min(std::max(r - row0, 0), 64);
    const char* p = reinterpret_cast<const char*>(A) + (nrows > 0 ? static_cast<int64_t>(row0) * in * 2 : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), static_cast<short>(0), nrows * in * 2,
                                             kBufferWord3);
  };
  const __amdgpu_buffer_rsrc_t rx = rsrc(x0), ry = rsrc(y0);
  // this wave's DMA instructions: X groups 2*wave, 2*wave + 1; Y likewise
  uint32_t off[2];
  int kc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = (2 * wave + q) * 8 + (lane >> 3);
    kc[q] = ((lane & 7) ^ ((row >> 1) & 7)) * 8;
    off[q] = static_cast<uint32_t>(row) * static_cast<uint32_t>(in) * 2u + kc[q] * 2u;
  }
  auto issue = [&](int st, int slot) {
    const uint32_t kb = static_cast<uint32_t>(st) * 128u;
    const int krem = in - st * 64;
    char* base = smem + slot * kGramStage;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t o = (kc[q] < krem) ? off[q] + kb : kOob;
      dma16(rx, base + (2 * wave + q) * 1024, o);
      dma16(ry, base + 8192 + (2 * wave + q) * 1024, o);
    }
  };

  // fragment addresses: lane l reads row 32*w + l%32, logical chunk 2*step + l/32
  const int frow = lane & 31, fh = lane >> 5, fsw = (frow >> 1) & 7;
  uint32_t xq[4], yq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    xq[q] = lds0 + static_cast<uint32_t>((wm * 32 + frow) * 128 + (((2 * q + fh) ^ fsw) * 16));
    yq[q] = lds0 + 8192u + static_cast<uint32_t>((wn * 32 + frow) * 128 + (((2 * q + fh) ^ fsw) * 16));
  }

  f32x16 acc0 = {}, acc1 = {};
#pragma unroll
  for (int i = 0; i < kGramNS - 1; ++i)
    if (st0 + i < st1) issue(st0 + i, i);
#define DORA_GSTAGE(U)                                                                    \
  if constexpr ((U) < kGramNS) {                                                          \
    const int st = sb + (U);                                                              \
    if (st >= st1) break;                                                                 \
    if (st + kGramNS - 2 < st1)                                                           \
      wait_vmcnt<(kGramNS - 2) * kGramL>();                                               \
    else                                                                                  \
      wait_vmcnt<0>();                                                                    \
    __builtin_amdgcn_s_barrier();                                                         \
    if (st + kGramNS - 1 < st1) issue(st + kGramNS - 1, ((U) + kGramNS - 1) % kGramNS);   \
    constexpr int so = (U) * kGramStage;                                                  \
    constexpr int sw = so & ~32767, si = so & 32767;                                      \
    u32x4 fx[4], fy[4];                                                                   \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                       \
      fx[q] = lds_read16_at<si>(xq[q] + sw);                                              \
      fy[q] = lds_read16_at<si>(yq[q] + sw);                                              \
    }                                                                                     \
    lds_wait();                                                                           \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                       \
      tie(fx[q]);                                                                         \
      tie(fy[q]);                                                                         \
    }                                                                                     \
    acc0 = Dt<DT>::mfma32(__builtin_bit_cast(V8, fx[0]), __builtin_bit_cast(V8, fy[0]), acc0); \
    acc1 = Dt<DT>::mfma32(__builtin_bit_cast(V8, fx[1]), __builtin_bit_cast(V8, fy[1]), acc1); \
    acc0 = Dt<DT>::mfma32(__builtin_bit_cast(V8, fx[2]), __builtin_bit_cast(V8, fy[2]), acc0); \
    acc1 = Dt<DT>::mfma32(__builtin_bit_cast(V8, fx[3]), __builtin_bit_cast(V8, fy[3]), acc1); \
  }
  for (int sb = st0; sb < st1; sb += kGramNS) {
    DORA_GSTAGE(0)
    DORA_GSTAGE(1)
    DORA_GSTAGE(2)
    DORA_GSTAGE(3)
    DORA_GSTAGE(4)
    DORA_GSTAGE(5)
    DORA_GSTAGE(6)
    DORA_GSTAGE(7)
  }
#undef DORA_GSTAGE

  // acc register q of lane l: G[x0 + 32*wm + 8*(q/4) + 4*(l/32) + q%4][y0 + 32*wn + l%32]
  float* dst = gpart + static_cast<int64_t>(sp) * r * r;
  const int col = y0 + wn * 32 + frow;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int row = x0 + wm * 32 + 8 * (q / 4) + 4 * fh + (q % 4);
    if (row < r && col < r) {
      if constexpr (DIRECT)
        gram_store_pair<DT>(ghi, glo, r, row, col, scale * (acc0[q] + acc1[q]), bi != bj);
      else
        dst[static_cast<int64_t>(row) * r + col] = acc0[q] + acc1[q];
    }
  }
}


// ---------------------------------------------------------------------------
// W stream with 128-byte row segments (rank tiles of 128, 256 and 384).
//
// With 64-byte row segments every L1 -> L2 request is 64 bytes, and the L1's
// table of pending requests then bounds the stream (it is full most of the
// time at the measured L2 latency).  Here a stage is 64 K columns: every DMA
// row segment is a whole 128-byte line.  The A panel (384
// rank rows, L2 resident) and the W0 panel (128 rows, streamed from HBM) sit
// in separate rings: two A slots, three W0 slots (the W0 panel is 128 or 256
// rows, the A panel 32 * TN * 4 rank rows).
//
// The loads of a stage (64 KiB per workgroup) take the texture path about a
// thousand cycles to accept, and a wave that issues them cannot issue MFMAs
// meanwhile.  So the roles are split: 8 tile waves only read LDS and run
// MFMAs, 4 DMA waves (one per SIMD) only issue loads.  After the barrier
// that opens stage u, the DMA waves issue A(u + 1) and then W0(u + 2) into
// the slots stage u - 1 used, and wait for A(u + 1) (their loads complete in
// order, so W0(u + 2) stays in flight: W0 has two stages to arrive, A one)
// before the barrier of stage u + 1.  Every stage issues the same loads per
// DMA wave (stages past the slice get out-of-range offsets: zeros into a slot
// no stage reads again), so one vmcnt value serves every wait.  Tile: 64 * TMW
// rows x 128 * TN ranks, tile waves 2 along the rows x 4 along the ranks
// (32 * TMW x 32 * TN each), four MFMA K steps per stage with the next step's
// fragments read during the current step's MFMAs.
template <int TN_, int TMW_>
struct K64Tile {
  static constexpr int TMW = TMW_, TN = TN_, WM = 2, WN = 4, NW = 8, NDMA = 4, NT = 64 * (NW + NDMA);
  static constexpr int BM = 32 * TMW * WM, BN = 32 * TN * WN;  // 128 x 384
  static constexpr int BK = 64, KS = BK / 16, ROWB = BK * 2;   // 128-byte rows
  static constexpr int RPI = 1024 / ROWB;                      // rows per 1 KiB DMA instruction
  static constexpr int XI = BM / RPI, YI = BN / RPI, XQ = XI / NDMA, YQ = YI / NDMA, L = 2 * XQ + YQ;
  static constexpr int A_BYTES = BN * ROWB, W_BYTES = BM * ROWB;  // one slot of each ring
  static constexpr int NA = 2, NWS = 3;
  static constexpr int A_OFF = 0, W_OFF = NA * A_BYTES;
  static constexpr int AREA = 160 * 1024, LDS_BYTES = AREA;
  static constexpr int NPAIR = TMW * KS, NP = (NPAIR + WN - 1) / WN;
  static constexpr int RED_BYTES = 2 * WN * BM * 4, RED_OFF = AREA - RED_BYTES;
  static constexpr int RPP_FIT = (AREA - RED_BYTES) / (BN * 2) / 32 * 32;
  static constexpr int RPP = RPP_FIT < BM ? RPP_FIT : BM;
  static_assert(TMW <= 4 && TN <= 3, "fragment reads of one K step: at most four W0 and three rank tiles");
  static_assert(XI % NDMA == 0 && YI % NDMA == 0, "whole DMA groups per DMA wave");
  static_assert(W_OFF + NWS * W_BYTES <= RED_OFF, "rings below the epilogue's row sums");
  static_assert(L < 64, "vmcnt range");
};

template <int DT, class TL>
__global__ __launch_bounds__(TL::NT, 1) void wstream_k64(WArgs a) {
  using V8 = typename Dt<DT>::V8;
  __shared__ __attribute__((aligned(1024))) char smem[TL::LDS_BYTES];
  float(*red)[TL::BM] = reinterpret_cast<float(*)[TL::BM]>(smem + TL::RED_OFF);

  const uint32_t v = static_cast<uint32_t>(xcd_logical_index());
  if (v >= static_cast<uint32_t>(a.total)) return;
  const uint32_t nTiles = static_cast<uint32_t>(a.nTiles), nRB = static_cast<uint32_t>(a.nRB);
  const int nt = static_cast<int>(v % nTiles);
  const uint32_t rb = (v / nTiles) % nRB;
  const int sp = static_cast<int>(v / (nTiles * nRB));
  const int64_t m0 = static_cast<int64_t>(rb) * TL::BM, n0 = static_cast<int64_t>(nt) * TL::BN;
  const int S1 = static_cast<int>(a.sm.S1), S12 = S1 + static_cast<int>(a.sm.S2);
  const int st0 = static_cast<int>(a.S * sp / a.nSplit), st1 = static_cast<int>(a.S * (sp + 1) / a.nSplit);
  // The W0 stages of the slice go in a rotated order, by a different amount
  // for each row block: the row blocks of a split then read different column
  // offsets at any moment rather than all the same one (which cost about a
  // quarter of the stream's rate).  The Gram stages stay last, in order.
  const int nW = std::max(0, std::min(st1, S1) - st0);
  const int rot = nW > 0 ? static_cast<int>((rb * 37u) % static_cast<uint32_t>(nW)) : 0;
  const int in = static_cast<int>(a.sm.in), r = static_cast<int>(a.sm.r);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool dma_wave = wave >= TL::NW;
  const int dw = dma_wave ? wave - TL::NW : 0;  // index among the DMA waves
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const bool want_base = (nt == 0) && !a.skip_base;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_t*)smem));

  auto rsrc = [](const void* base, int64_t row0, int64_t rows, int64_t ld, int64_t max_rows) {
    const int64_t nrows = std::min<int64_t>(std::max<int64_t>(rows - row0, 0), max_rows);
    const char* p = static_cast<const char*>(base) + (nrows > 0 ? row0 * ld * 2 : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), static_cast<short>(0),
                                             static_cast<int>(nrows * ld * 2), kBufferWord3);
  };
  const int64_t out = a.sm.out;
  const __amdgpu_buffer_rsrc_t rxW = rsrc(a.sm.W0, m0, out, in, TL::BM);
  const __amdgpu_buffer_rsrc_t ryA = rsrc(a.sm.A, n0, r, in, TL::BN);
  const __amdgpu_buffer_rsrc_t rxB = rsrc(a.sm.B, m0, out, r, TL::BM);
  const __amdgpu_buffer_rsrc_t ryH = rsrc(a.sm.Ghi, n0, r, r, TL::BN);
  const __amdgpu_buffer_rsrc_t ryL = rsrc(a.sm.Glo, n0, r, r, TL::BN);

  // DMA geometry: instruction q of DMA wave d moves panel rows
  // 8*(q*NDMA + d) .. + 7, 128 bytes each; lane l takes row l/8 of them and the
  // logical chunk (l%8) ^ ((row/2)%8), which lands in LDS slot l%8 (so the
  // fragment reads of 16 consecutive rows at one logical chunk hit 16 distinct
  // bank groups).  Group rows start on multiples of 32*q + 8*d: the chunk
  // depends on the lane and the wave's parity only.  The A panel is fetched in
  // the fragment row order sigma (rows 16..31 of a 32-row tile hold rank rows
  // sigma(p)); 32*q keeps a row's place within its 32-row tile.
  auto sigma = [](int p) { return 16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3); };
  const int prow = dw * TL::RPI + (lane >> 3);         // panel row of instruction 0
  const int lc = (lane & 7) ^ ((prow >> 1) & 7);      // logical chunk fetched
  const int kc = lc * 8;                               // its first K element
  const int yr0 = (prow & ~31) + sigma(prow & 31);
  const uint32_t ldA = static_cast<uint32_t>(in) * 2u, ldB = static_cast<uint32_t>(r) * 2u;
  const uint32_t lxA = static_cast<uint32_t>(prow) * ldA + kc * 2u, lxB = static_cast<uint32_t>(prow) * ldB + kc * 2u;
  const uint32_t lyA = static_cast<uint32_t>(yr0) * ldA + kc * 2u, lyB = static_cast<uint32_t>(yr0) * ldB + kc * 2u;
  // smallest rank (within the tile) among the eight panel rows of A-panel
  // instruction q: rows 8m .. 8m + 7 of a 32-row tile hold ranks 4m .. 4m + 3
  // and 16 + 4m .. 16 + 4m + 3
  int a_rank0[TL::YQ];
#pragma unroll
  for (int q = 0; q < TL::YQ; ++q) {
    const int p0 = 8 * (q * TL::NDMA + dw);
    a_rank0[q] = (p0 & ~31) + 4 * ((p0 & 31) >> 3);
  }

  // Fragment reads: lane l reads row 32*i + l%32 of its wave's tiles at
  // logical chunk 2*step + l/32, stored at chunk (2*step + l/32) ^ ((l%32)/2 % 8).
  const int frow = lane & 31, fh = lane >> 5, fsw = (frow >> 1) & 7;
  const uint32_t xrow = lds0 + static_cast<uint32_t>(TL::W_OFF + (wm * TL::TMW * 32 + frow) * TL::ROWB);
  const uint32_t yrow = lds0 + static_cast<uint32_t>(TL::A_OFF + (wn * TL::TN * 32 + frow) * TL::ROWB);
  uint32_t co[TL::KS];
#pragma unroll
  for (int k = 0; k < TL::KS; ++k) co[k] = static_cast<uint32_t>(((2 * k + fh) ^ fsw) * 16);

  f32x16 acc[TL::TMW][TL::TN];
#pragma unroll
  for (int i = 0; i < TL::TMW; ++i)
#pragma unroll
    for (int j = 0; j < TL::TN; ++j) acc[i][j] = f32x16{};
  float bs[TL::NP];
#pragma unroll
  for (int t = 0; t < TL::NP; ++t) bs[t] = 0.0f;

  // the segment of stage st: resources, row pitch, per-lane offsets, K offset
  // and whether this lane's chunk lies past the segment (or the stage past st1)
#define K64_SEL(ST)                                                                      \
  const int dstep_ = (ST);                                                               \
  const int drw_ = dstep_ - st0 + rot;                                                   \
  const int dst_ = dstep_ - st0 < nW ? st0 + (drw_ < nW ? drw_ : drw_ - nW) : dstep_;    \
  const bool dw_ = dst_ < S1, dh_ = dst_ < S12;                                          \
  const __amdgpu_buffer_rsrc_t drx_ = dw_ ? rxW : rxB;                                   \
  const __amdgpu_buffer_rsrc_t dry_ = dw_ ? ryA : (dh_ ? ryH : ryL);                     \
  const uint32_t dld_ = dw_ ? ldA : ldB, dlx_ = dw_ ? lxA : lxB, dly_ = dw_ ? lyA : lyB; \
  const int dkst_ = dst_ - (dw_ ? 0 : (dh_ ? S1 : S12));                                 \
  const int dkrem_ = (dw_ ? in : r) - dkst_ * TL::BK;                                    \
  const uint32_t dkb_ = static_cast<uint32_t>(dkst_) * static_cast<uint32_t>(TL::ROWB);  \
  const bool doob_ = dstep_ >= st1 || (dkrem_ < TL::BK && kc >= dkrem_);
  // DMA of the A (rank-side) panel of stage ST into A slot SA; an instruction
  // whose eight panel rows all hold ranks past r is not issued (its LDS rows
  // only feed accumulator columns past r, which no epilogue reads)
#define K64_ISSUE_A(ST, SA)                                                              \
  {                                                                                      \
    K64_SEL(ST)                                                                          \
    _Pragma("unroll") for (int q = 0; q < TL::YQ; ++q) {                                 \
      if (n0 + a_rank0[q] >= r) continue;                                                \
      const uint32_t o_ = dly_ + static_cast<uint32_t>(q * TL::NDMA * TL::RPI) * dld_ + dkb_; \
      dma16(dry_, smem + TL::A_OFF + (SA) * TL::A_BYTES + (q * TL::NDMA + dw) * 1024, doob_ ? kOob : o_); \
    }                                                                                    \
  }
  // DMA of the W0 (row-side) panel of stage ST into W slot SW
#define K64_ISSUE_W(ST, SWS)                                                             \
  {                                                                                      \
    K64_SEL(ST)                                                                          \
    _Pragma("unroll") for (int q = 0; q < TL::XQ; ++q) {                                 \
      const uint32_t o_ = dlx_ + static_cast<uint32_t>(q * TL::NDMA * TL::RPI) * dld_ + dkb_; \
      dma16(drx_, smem + TL::W_OFF + (SWS) * TL::W_BYTES + (q * TL::NDMA + dw) * 1024, doob_ ? kOob : o_); \
    }                                                                                    \
  }
  // fragments of K step K of the stage in A slot SA / W slot SWS
#define K64_READS(X, Y, SA, SWS, K)                                                      \
  {                                                                                      \
    const uint32_t xb_ = xrow + (SWS) * TL::W_BYTES + co[K];                             \
    const uint32_t yb_ = yrow + (SA) * TL::A_BYTES + co[K];                              \
    X[0] = lds_read16_at<0>(xb_);                                                        \
    if constexpr (TL::TMW > 1) X[1 % TL::TMW] = lds_read16_at<32 * TL::ROWB>(xb_);       \
    if constexpr (TL::TMW > 2) X[2 % TL::TMW] = lds_read16_at<64 * TL::ROWB>(xb_);       \
    if constexpr (TL::TMW > 3) X[3 % TL::TMW] = lds_read16_at<96 * TL::ROWB>(xb_);       \
    Y[0] = lds_read16_at<0>(yb_);                                                        \
    if constexpr (TL::TN > 1) Y[1 % TL::TN] = lds_read16_at<32 * TL::ROWB>(yb_);         \
    if constexpr (TL::TN > 2) Y[2 % TL::TN] = lds_read16_at<64 * TL::ROWB>(yb_);         \
  }
#define K64_MFMAS(X, Y)                                                                  \
  _Pragma("unroll") for (int i = 0; i < TL::TMW; ++i) _Pragma("unroll") for (int j = 0; j < TL::TN; ++j) \
      acc[i][j] = Dt<DT>::mfma32(__builtin_bit_cast(V8, Y[j]), __builtin_bit_cast(V8, X[i]), acc[i][j]);
#define K64_SQUARES(X, C)                                                                \
  _Pragma("unroll") for (int t = 0; t < TL::NP; ++t)                                     \
    _Pragma("unroll") for (int i = 0; i < TL::TMW; ++i)                                  \
      if (wn + TL::WN * t == TL::KS * i + (C)) {                                         \
        bs[t] = sq2<DT>(X[i][0], bs[t]);                                                 \
        bs[t] = sq2<DT>(X[i][1], bs[t]);                                                 \
        bs[t] = sq2<DT>(X[i][2], bs[t]);                                                 \
        bs[t] = sq2<DT>(X[i][3], bs[t]);                                                 \
      }
  // One stage of a DMA wave: U is the stage's index within a loop turn of 6
  // (A slot U % 2, W slot U % 3).
#define K64_DMA_STAGE(U)                                                                 \
  {                                                                                      \
    const int st = sb + (U);                                                             \
    if (st >= st1) break;                                                                \
    __builtin_amdgcn_s_barrier();                                                        \
    K64_ISSUE_A(st + 1, ((U) + 1) % TL::NA)                                              \
    K64_ISSUE_W(st + 2, ((U) + 2) % TL::NWS)                                             \
    wait_vmcnt<TL::XQ>();                                                                \
  }
  // One stage of a tile wave
#define K64_STAGE(U)                                                                     \
  {                                                                                      \
    constexpr int sa = (U) % TL::NA, sws = (U) % TL::NWS;                                \
    const int st = sb + (U);                                                             \
    if (st >= st1) break;                                                                \
    __builtin_amdgcn_s_barrier();                                                        \
    const bool base_here = want_base && st < S1;                                         \
    u32x4 xa[TL::TMW], ya[TL::TN], xn[TL::TMW], yn[TL::TN];                              \
    K64_READS(xa, ya, sa, sws, 0)                                                        \
    lds_wait();                                                                          \
    _Pragma("unroll") for (int i = 0; i < TL::TMW; ++i) tie(xa[i]);                      \
    _Pragma("unroll") for (int j = 0; j < TL::TN; ++j) tie(ya[j]);                       \
    K64_READS(xn, yn, sa, sws, 1)                                                        \
    K64_MFMAS(xa, ya)                                                                    \
    if (base_here) { K64_SQUARES(xa, 0) }                                                \
    lds_wait();                                                                          \
    _Pragma("unroll") for (int i = 0; i < TL::TMW; ++i) tie(xn[i]);                      \
    _Pragma("unroll") for (int j = 0; j < TL::TN; ++j) tie(yn[j]);                       \
    K64_READS(xa, ya, sa, sws, 2)                                                        \
    K64_MFMAS(xn, yn)                                                                    \
    if (base_here) { K64_SQUARES(xn, 1) }                                                \
    lds_wait();                                                                          \
    _Pragma("unroll") for (int i = 0; i < TL::TMW; ++i) tie(xa[i]);                      \
    _Pragma("unroll") for (int j = 0; j < TL::TN; ++j) tie(ya[j]);                       \
    K64_READS(xn, yn, sa, sws, 3)                                                        \
    K64_MFMAS(xa, ya)                                                                    \
    if (base_here) { K64_SQUARES(xa, 2) }                                                \
    lds_wait();                                                                          \
    _Pragma("unroll") for (int i = 0; i < TL::TMW; ++i) tie(xn[i]);                      \
    _Pragma("unroll") for (int j = 0; j < TL::TN; ++j) tie(yn[j]);                       \
    K64_MFMAS(xn, yn)                                                                    \
    if (base_here) { K64_SQUARES(xn, 3) }                                                \
  }

  // Both roles pass one barrier per stage of the slice.
  if (st0 < st1) {
    if (dma_wave) {
      // prologue: A(st0), W0(st0), W0(st0 + 1), in that order; stage st0's
      // panels have landed before its barrier
      K64_ISSUE_A(st0, 0)
      K64_ISSUE_W(st0, 0)
      K64_ISSUE_W(st0 + 1, 1)
      wait_vmcnt<TL::XQ>();
      for (int sb = st0; sb < st1; sb += 6) {
        K64_DMA_STAGE(0)
        K64_DMA_STAGE(1)
        K64_DMA_STAGE(2)
        K64_DMA_STAGE(3)
        K64_DMA_STAGE(4)
        K64_DMA_STAGE(5)
      }
    } else {
      for (int sb = st0; sb < st1; sb += 6) {
        K64_STAGE(0)
        K64_STAGE(1)
        K64_STAGE(2)
        K64_STAGE(3)
        K64_STAGE(4)
        K64_STAGE(5)
      }
    }
  }
  // stages past the slice were issued as out-of-range loads: drain them
  // before the stage area is reused (the epilogue's first barrier)
  wait_vmcnt<0>();
#undef K64_DMA_STAGE
#undef K64_STAGE
#undef K64_SQUARES
#undef K64_MFMAS
#undef K64_READS
#undef K64_ISSUE_W
#undef K64_ISSUE_A
#undef K64_SEL

  if (a.acc_part) {  // norm backward: keep U + B G' (DMA waves hold no accumulators)
    if (!dma_wave) dma_store_acc<TL>(a, sp, m0, n0, acc);
    return;
  }
  dma_cross_epilogue<DT, TL>(a, sp, nt, m0, n0, acc, bs, want_base, red, smem, lds0, rxB);
}

// ---------------------------------------------------------------------------
// W stream, general path (row lengths not multiples of 8, or unaligned
// pointers): register-staged loads with element-wise bounds, LDS rows padded
// by 8 elements, double buffered.

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

template <int DT>
__device__ inline Chunk load_chunk_any(const Operand& op, int64_t row, int64_t k) {
  using T = typename Dt<DT>::T;
  if (row >= op.rows || k >= op.klen) return zero_chunk();
  const T* src = static_cast<const T*>(op.p) + row * op.ld + k;
  typename Dt<DT>::V8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (k + j < op.klen) ? src[j] : static_cast<T>(0.0f);
  return __builtin_bit_cast(Chunk, v);
}

template <int DT>
__global__ __launch_bounds__(TileW::NT, 2) void wstream_general(WArgs a) {
  using TL = TileW;
  using T = typename Dt<DT>::T;
  using V8 = typename Dt<DT>::V8;
  __shared__ __attribute__((aligned(16))) T smem[TL::LDS_ELEMS];
  __shared__ float red[TL::WN][TL::BM];
  const int64_t v = xcd_logical_index();
  if (v >= a.total) return;
  const int nt = static_cast<int>(v % a.nTiles);
  const int64_t rb = (v / a.nTiles) % a.nRB;
  const int sp = static_cast<int>(v / (static_cast<int64_t>(a.nTiles) * a.nRB));
  const int64_t m0 = rb * TL::BM, n0 = static_cast<int64_t>(nt) * TL::BN;
  const int64_t st0 = a.S * sp / a.nSplit, st1 = a.S * (sp + 1) / a.nSplit;
  const bool want_base = (nt == 0) && !a.skip_base;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const int lrow = tid / TL::CPR, lkc = tid % TL::CPR;
  // buffer b: X panel at smem + b*(BM+BN)*LDK, Y panel right after it
  auto Xs = [&](int b) { return smem + b * (TL::BM + TL::BN) * TL::LDK; };
  auto Ys = [&](int b) { return smem + b * (TL::BM + TL::BN) * TL::LDK + TL::BM * TL::LDK; };

  f32x16 acc[TL::TM][TL::TN];
#pragma unroll
  for (int i = 0; i < TL::TM; ++i)
#pragma unroll
    for (int j = 0; j < TL::TN; ++j) acc[i][j] = f32x16{};
  float bsum[TL::XCH] = {};

  Chunk xr[TL::XCH], yr[TL::YCH];
  auto gload = [&](int64_t st) -> bool {
    Operand X, Y;
    int64_t k0;
    bool seg_w;
    a.sm.template get<TL::BK>(st, X, Y, k0, seg_w);
    const int64_t k = k0 + lkc * 8;
#pragma unroll
    for (int i = 0; i < TL::XCH; ++i) xr[i] = load_chunk_any<DT>(X, m0 + lrow + i * TL::RPP, k);
#pragma unroll
    for (int i = 0; i < TL::YCH; ++i) yr[i] = load_chunk_any<DT>(Y, n0 + lrow + i * TL::RPP, k);
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
      *reinterpret_cast<Chunk*>(Xs(buf) + (lrow + i * TL::RPP) * TL::LDK + lkc * 8) = xr[i];
#pragma unroll
    for (int i = 0; i < TL::YCH; ++i)
      *reinterpret_cast<Chunk*>(Ys(buf) + (lrow + i * TL::RPP) * TL::LDK + lkc * 8) = yr[i];
  };

  if (st0 < st1) {
    lstore(0, gload(st0));
    __syncthreads();
    const int frow = lane & 31;
    const int fk = (lane >> 5) * 8;
    for (int64_t st = st0; st < st1; ++st) {
      const int buf = static_cast<int>((st - st0) & 1);
      const bool have_next = st + 1 < st1;
      bool next_w = false;
      if (have_next) next_w = gload(st + 1);
      const T* xs = Xs(buf) + (wm * TL::TM * 32 + frow) * TL::LDK + fk;
      const T* ys = Ys(buf) + (wn * TL::TN * 32 + frow) * TL::LDK + fk;
#pragma unroll
      for (int kk = 0; kk < TL::BK / 16; ++kk) {
        V8 x[TL::TM], y[TL::TN];
#pragma unroll
        for (int i = 0; i < TL::TM; ++i) x[i] = *reinterpret_cast<const V8*>(xs + i * 32 * TL::LDK + kk * 16);
#pragma unroll
        for (int j = 0; j < TL::TN; ++j) y[j] = *reinterpret_cast<const V8*>(ys + j * 32 * TL::LDK + kk * 16);
#pragma unroll
        for (int i = 0; i < TL::TM; ++i)
#pragma unroll
          for (int j = 0; j < TL::TN; ++j) acc[i][j] = Dt<DT>::mfma32(y[j], x[i], acc[i][j]);
      }
      if (have_next) lstore(buf ^ 1, next_w);
      __syncthreads();
    }
  }

  if (want_base) {
    const int64_t out = a.sm.out;
#pragma unroll
    for (int i = 0; i < TL::XCH; ++i) {
      float b = bsum[i];
#pragma unroll
      for (int off = 1; off < TL::CPR; off <<= 1) b += __shfl_xor(b, off, 64);
      const int64_t row = m0 + lrow + i * TL::RPP;
      if (lkc == 0 && row < out) a.base_part[static_cast<int64_t>(sp) * out + row] = b;
    }
  }
  cross_epilogue<DT, TL::TM, TL::TN, TL::WM, TL::WN, TL::BM, false>(a, sp, nt, m0, n0, acc, red);
}

// ---------------------------------------------------------------------------

// Row square norms c_i = sum_k W0_ik^2: the base term alone, for a cache of
// the frozen W0.  One wave per row.  On the 16-byte path lane l reads chunks
// l, l + 64, .. of 8 elements (four in flight) and squares the four packed
// pairs of a chunk into four fp32 sums, two squares per dot2 instruction; the
// general path deals elements l, l + 64, .. to the four sums in turn.  A sum
// holds at most ceil(in / 256) + 1 squares; the 256 sums of a wave are
// combined in fp64 and rounded to fp32 once.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void row_sqnorm(const typename Dt<DT>::T* W0, int64_t out, int64_t in, float* sq) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= out) return;
  const typename Dt<DT>::T* w = W0 + row * in;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (VEC) {
    const u32x4* p = reinterpret_cast<const u32x4*>(w);
    const int64_t nc = in / 8;
    int64_t c = lane;
    for (; c + 192 < nc; c += 256) {
      const u32x4 v0 = p[c], v1 = p[c + 64], v2 = p[c + 128], v3 = p[c + 192];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[q] = sq2<DT>(v0[q], acc[q]);
        acc[q] = sq2<DT>(v1[q], acc[q]);
        acc[q] = sq2<DT>(v2[q], acc[q]);
        acc[q] = sq2<DT>(v3[q], acc[q]);
      }
    }
    for (; c < nc; c += 64) {
      const u32x4 v = p[c];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = sq2<DT>(v[q], acc[q]);
    }
  } else {
    int q = 0;
    for (int64_t k = lane; k < in; k += 64) {
      const float x = Dt<DT>::to_f(w[k]);
      acc[q] = __builtin_fmaf(x, x, acc[q]);
      q = (q + 1) & 3;
    }
  }
  double d = (static_cast<double>(acc[0]) + static_cast<double>(acc[1])) +
             (static_cast<double>(acc[2]) + static_cast<double>(acc[3]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) d += __shfl_xor(d, o, 64);
  if (lane == 0) sq[row] = static_cast<float>(d);
}

// sum_{q < n} p[q * stride] in fp64, in order; the loads go out in groups of
// 8 before the group is added, so a row's partials are fetched in parallel
// rather than one dependent load at a time.
__device__ inline double ordered_sum(const float* p, int n, int64_t stride) {
  double acc = 0.0;
  int q = 0;
  for (; q + 8 <= n; q += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[static_cast<int64_t>(q + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += static_cast<double>(v[u]);
  }
  for (; q < n; ++q) acc += static_cast<double>(p[static_cast<int64_t>(q) * stride]);
  return acc;
}

// n_i from the partials; the base term from base_sq[i] when a cache is given.
// Up to kFinParts partials of each sum are loaded before either is added (one
// memory round trip for both sums); the additions keep split order.
__global__ __launch_bounds__(256) void norm_finalize(const float* base_part, const float* cross_part,
                                                     const float* base_sq, int nSplit, int nTiles, int64_t out,
                                                     float s, float* norm_out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= out) return;
  const int nc = nSplit * nTiles;
  double b, c;
  if (nSplit <= kFinParts && nc <= kFinParts) {
    float vb[kFinParts], vc[kFinParts];
    const float bq = base_sq ? base_sq[i] : 0.0f;
#pragma unroll
    for (int q = 0; q < kFinParts; ++q) {
      vb[q] = !base_sq && q < nSplit ? base_part[i + static_cast<int64_t>(q) * out] : 0.0f;
      vc[q] = q < nc ? cross_part[i + static_cast<int64_t>(q) * out] : 0.0f;
    }
    b = static_cast<double>(bq);
    c = 0.0;
#pragma unroll
    for (int q = 0; q < kFinParts; ++q) {
      if (q < nSplit) b += static_cast<double>(vb[q]);
      if (q < nc) c += static_cast<double>(vc[q]);
    }
  } else {
    b = base_sq ? static_cast<double>(base_sq[i]) : ordered_sum(base_part + i, nSplit, out);
    c = ordered_sum(cross_part + i, nc, out);
  }
  const double n2 = b + 2.0 * static_cast<double>(s) * c;
  norm_out[i] = static_cast<float>(n2 > 0.0 ? sqrt(n2) : 0.0);
}

// Rank tile width of the 16-byte path: 128*TN columns, TN in 1..3, choosing the
// least padding of r and then the widest tile (fewest passes over W0).  Tiles
// of 512 are not used: at r = 512, two passes of 256-wide tiles measured 94 us
// at 8192^2 against 110-114 us for one pass of a 512-wide tile, whose rank
// panel does not fit two ring slots beside the W0 ring at 128-byte segments.
int dma_tn(int64_t r) {
  int best = 1;
  int64_t best_pad = -1;
  for (int tn = 1; tn <= 3; ++tn) {
    const int64_t w = 128 * tn;
    const int64_t pad = cdiv(std::max<int64_t>(r, 1), w) * w;
    if (best_pad < 0 || pad <= best_pad) {
      best = tn;
      best_pad = pad;
    }
  }
  return best;
}

// Rank tiles of 128, 256 and 384: 256 x 128, 128 x 256 and 128 x 384 (W0 rows x ranks).
template <int TN> struct K64Of;
template <> struct K64Of<1> { using T = K64Tile<1, 4>; };
template <> struct K64Of<2> { using T = K64Tile<2, 2>; };
template <> struct K64Of<3> { using T = K64Tile<3, 2>; };

int dma_rows(int tn) {
  switch (tn) {
    case 1: return K64Of<1>::T::BM;
    case 2: return K64Of<2>::T::BM;
    default: return K64Of<3>::T::BM;
  }
}

int dma_bk(int tn) {
  switch (tn) {
    case 1: return K64Of<1>::T::BK;
    case 2: return K64Of<2>::T::BK;
    default: return K64Of<3>::T::BK;
  }
}

template <int DT, int TN>
void launch_dma(const WArgs& w, hipStream_t stream) {
  static_assert(TN >= 1 && TN <= 3, "rank tiles of 128, 256 and 384");
  using TL = typename K64Of<TN>::T;
  const dim3 grid(static_cast<unsigned>(cdiv(w.total, 8) * 8));
  hipLaunchKernelGGL((wstream_k64<DT, TL>), grid, dim3(TL::NT), 0, stream, w);
}

// Workgroups of gram_finalize: four 8-row strips per upper 32 x 32 tile.
int64_t gram_finalize_blocks(int64_t r) {
  const int64_t nT = cdiv(r, 32);
  return 2 * nT * (nT + 1);
}

// G' = scale * A A^T as the pair G'hi + G'lo in the plan's workspace regions.
template <int DT>
hipError_t launch_gram_t(const NormPlan& p, const void* Av, float scale, char* ws, bool vec, hipStream_t stream,
                         unsigned* fin_count = nullptr) {
  using T = typename Dt<DT>::T;
  if (p.r <= 0) return hipSuccess;
  T* ghi = reinterpret_cast<T*>(ws + p.off_ghi);
  T* glo = reinterpret_cast<T*>(ws + p.off_glo);
  const T* A = static_cast<const T*>(Av);
  float* gpart = reinterpret_cast<float*>(ws + p.off_gpart);
  const int nUpper = p.nTg * (p.nTg + 1) / 2;
  const dim3 ggrid(static_cast<unsigned>(cdiv(static_cast<int64_t>(nUpper) * p.splitG, 8) * 8));
  if (p.gram_direct) {  // one K split: the Gram kernel writes G'hi/G'lo itself
    if (vec)
      hipLaunchKernelGGL((gram_dma<DT, 4, true>), ggrid, dim3(256), 0, stream, A, static_cast<int>(p.in),
                         static_cast<int>(p.r), p.nTg, 1, nullptr, scale, ghi, glo, fin_count,
                         static_cast<int>(p.nRB));
    else
      hipLaunchKernelGGL((gram_partial<DT, true>), ggrid, dim3(256), 0, stream, A, p.in, p.r, p.nTg, 1, nullptr,
                         scale, ghi, glo);
    return hipGetLastError();
  }
  if (vec)
    hipLaunchKernelGGL((gram_dma<DT, 4, false>), ggrid, dim3(256), 0, stream, A, static_cast<int>(p.in),
                       static_cast<int>(p.r), p.nTg, p.splitG, gpart, scale, nullptr, nullptr, fin_count,
                       static_cast<int>(p.nRB));
  else
    hipLaunchKernelGGL((gram_partial<DT, false>), ggrid, dim3(256), 0, stream, A, p.in, p.r, p.nTg, p.splitG, gpart,
                       scale, nullptr, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gram_finalize<DT>), dim3(static_cast<unsigned>(gram_finalize_blocks(p.r))), dim3(256), 0,
                     stream, gpart, p.splitG, p.r, scale, ghi, glo);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_norm_t(const NormPlan& p, const NormArgs& a, bool vec) {
  if (vec && p.strip) return launch_norm_strip(p, a);
  char* ws = static_cast<char*>(a.ws);
  using T = typename Dt<DT>::T;
  T* ghi = reinterpret_cast<T*>(ws + p.off_ghi);
  T* glo = reinterpret_cast<T*>(ws + p.off_glo);
  // 16-byte path with an adapter: the W stream's epilogue finalizes the norm
  // (per-row-block counters in the workspace, zeroed by the Gram kernel)
  const bool fuse = vec && p.r > 0 && p.in > 0;
  unsigned* fin_count = fuse ? reinterpret_cast<unsigned*>(ws + p.off_count) : nullptr;
  {
    const hipError_t e = launch_gram_t<DT>(p, a.A, a.s * 0.5f, ws, vec, a.stream, fin_count);
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
  w.skip_base = a.base_sq != nullptr;
  w.fin_count = fin_count;
  w.norm_out = a.norm_out;
  w.base_sq = a.base_sq;
  w.s = a.s;
  if (vec) {
    switch (p.tn) {
      case 1: launch_dma<DT, 1>(w, a.stream); break;
      case 2: launch_dma<DT, 2>(w, a.stream); break;
      default: launch_dma<DT, 3>(w, a.stream); break;
    }
  } else {
    const dim3 grid(static_cast<unsigned>(cdiv(w.total, 8) * 8));
    hipLaunchKernelGGL((wstream_general<DT>), grid, dim3(TileW::NT), 0, a.stream, w);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fuse) return e;
  hipLaunchKernelGGL(norm_finalize, dim3(static_cast<unsigned>(cdiv(p.out, 256))), dim3(256), 0, a.stream,
                     w.base_part, w.cross_part, a.base_sq, p.nSplit, p.nTiles, p.out, a.s, a.norm_out);
  return hipGetLastError();
}

// Norm backward, d_B: d_B[i][j] = s * c_i * (sum of the split partials of
// U + s B G, added in split order in fp32), rounded once to the storage dtype.
// Four consecutive elements of one row per thread and step (r % 8 == 0).
template <int DT>
__global__ __launch_bounds__(256) void nbwd_finalize_b(const float* part, int nSplit, int64_t out, int64_t r,
                                                       const float* c, float s, void* dB) {
  using T = typename Dt<DT>::T;
  using T4 = T __attribute__((ext_vector_type(4)));
  const int64_t n = out * r, n4 = n / 4;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n4;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    f32x4 sum = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int p = 0; p < nSplit; ++p) sum += reinterpret_cast<const f32x4*>(part + static_cast<int64_t>(p) * n)[e];
    const float sc = s * c[(e * 4) / r];
    T4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = Dt<DT>::from_f(sc * sum[q]);
    reinterpret_cast<T4*>(dB)[e] = o;
  }
}

template <int DT>
hipError_t launch_norm_bwd_db_t(const NormPlan& p, const void* W0, const void* A, const void* B, float s,
                                const float* c, void* dB, void* wsv, float* acc_part, hipStream_t stream) {
  char* ws = static_cast<char*>(wsv);
  using T = typename Dt<DT>::T;
  hipError_t e = launch_gram_t<DT>(p, A, s, ws, true, stream);  // G' = s G
  if (e != hipSuccess) return e;
  WArgs w;
  w.sm = WStages{W0, A, B, reinterpret_cast<T*>(ws + p.off_ghi), reinterpret_cast<T*>(ws + p.off_glo), p.out, p.in,
                 p.r, p.S1, p.S2};
  w.nRB = p.nRB;
  w.S = p.S;
  w.nTiles = p.nTiles;
  w.nSplit = p.nSplit;
  w.total = p.nRB * p.nTiles * p.nSplit;
  w.base_part = nullptr;
  w.cross_part = nullptr;
  w.skip_base = 1;
  w.acc_part = acc_part;
  switch (p.tn) {
    case 1: launch_dma<DT, 1>(w, stream); break;
    case 2: launch_dma<DT, 2>(w, stream); break;
    default: launch_dma<DT, 3>(w, stream); break;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = std::min<int64_t>(cdiv(p.out * p.r / 4, 256), 4096);
  hipLaunchKernelGGL((nbwd_finalize_b<DT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, acc_part,
                     p.nSplit, p.out, p.r, c, s, dB);
  return hipGetLastError();
}

}  // namespace

size_t norm_bwd_acc_bytes(const NormPlan& p) { return static_cast<size_t>(p.nSplit) * p.out * p.r * 4; }

hipError_t launch_norm_bwd_db(const NormPlan& p, const void* W0, const void* A, const void* B, float s,
                              const float* c, void* dB, void* ws, float* acc_part, hipStream_t stream) {
  if (p.out <= 0 || p.r <= 0) return hipSuccess;
  return p.dtype == 0 ? launch_norm_bwd_db_t<0>(p, W0, A, B, s, c, dB, ws, acc_part, stream)
                      : launch_norm_bwd_db_t<1>(p, W0, A, B, s, c, dB, ws, acc_part, stream);
}

size_t norm_scratch_bound(int64_t out, int64_t r) {
  return static_cast<size_t>(4 * (out * r + r * r) + 64 * out);
}

int64_t norm_max_grid(const NormPlan& p) {
  const int64_t nUpper = static_cast<int64_t>(p.nTg) * (p.nTg + 1) / 2;
  const int64_t gram = p.r > 0 ? std::max(cdiv(nUpper * p.splitG, 8) * 8, gram_finalize_blocks(p.r)) : 0;
  const int64_t stream = cdiv(p.nRB * p.nTiles * p.nSplit, 8) * 8;
  return std::max({gram, stream, cdiv(p.out, 256), p.strip ? cdiv_strip(p.out) : int64_t(0)});
}

NormPlan make_norm_plan(int64_t out, int64_t in, int64_t r, int dtype, bool vec, bool store_acc) {
  NormPlan p;
  p.out = out;
  p.in = in;
  p.r = r;
  p.dtype = dtype;
  p.vec = vec;
  if (out <= 0) return p;
  const int64_t e = 2;  // bytes per storage element (bf16, fp16)
  int64_t bm, bn, bk, slots;
  if (vec) {
    slots = 256;
    p.tn = dma_tn(r);
    // A rank tile of 128 takes 256-row blocks.  Where those, at the most K
    // splits the plan allows (at least 8 stages each), leave CUs without a
    // workgroup, the forward takes the 256-wide tile of 128-row blocks
    // instead: twice the workgroups, with MFMAs on the padded ranks that stay
    // below each stage's HBM time.  4096^2, r = 64: 24.5 / 26.3 us against
    // 25.4 / 27.1 (warm / cold).  The store mode of the norm backward keeps
    // the 128-wide tile (its cold call measured 2.5 us slower with this one).
    if (p.tn == 1 && !store_acc && r <= 128) {
      const int64_t S = cdiv(in, dma_bk(1)) + 2 * cdiv(r, dma_bk(1));
      const int64_t maxs = std::max<int64_t>(1, std::min<int64_t>(64, S / 8));
      if (cdiv(out, dma_rows(1)) * maxs < slots) p.tn = 2;
    }
    bm = dma_rows(p.tn);
    bn = 128 * p.tn;
    bk = dma_bk(p.tn);
  } else {
    p.tn = 0;
    bm = TileW::BM;
    bn = TileW::BN;
    bk = TileW::BK;
    slots = 512;
  }
  p.nRB = cdiv(out, bm);
  p.nTiles = static_cast<int>(std::max<int64_t>(1, cdiv(r, bn)));
  p.S1 = cdiv(in, bk);
  p.S2 = cdiv(r, bk);
  p.S = p.S1 + 2 * p.S2;
  // K splits: minimise (rounds of resident workgroups) x (stages per workgroup
  // + a fixed cost of about 8 stages of 32 for the pipeline fill and the
  // epilogue), keeping at least 8 stages per workgroup; ties go to fewer splits.
  {
    const int64_t fixed = 8 * 32 / bk;
    const int64_t per = p.nRB * p.nTiles;
    const int64_t maxs = std::max<int64_t>(1, std::min<int64_t>(64, p.S / 8));
    int64_t best = -1, bestc = 0;
    for (int64_t k = 1; k <= maxs; ++k) {
      const int64_t cost = cdiv(per * k, slots) * (cdiv(std::max<int64_t>(p.S, 1), k) + fixed);
      if (best < 0 || cost < bestc) {
        best = k;
        bestc = cost;
      }
    }
    p.nSplit = static_cast<int>(best);
    // Store mode (the norm backward keeps each split's accumulators, nSplit x
    // out x r fp32, and reads them back): split K only as far as it takes to
    // give the 256 CUs a workgroup each, since every split adds a full slice.
    if (store_acc)
      p.nSplit = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(maxs, slots / std::max<int64_t>(per, 1))));
  }
  if (r > 0) {
    // Gram: upper tiles (64x64 on the 16-byte path, 32x32 otherwise) x K
    // splits; about 512 workgroups, at most 32 splits with at least 2 K
    // stages of 64 per workgroup (general path: 16 splits, 8 K steps of 16
    // per wave).  At small r the few upper tiles need the splits: r = 64 and
    // 128 at in = 8192 take 32 splits (1.4 us faster than 16).
    const int64_t tile = vec ? 64 : 32;
    p.nTg = static_cast<int>(cdiv(r, tile));
    const int64_t nUpper = static_cast<int64_t>(p.nTg) * (p.nTg + 1) / 2;
    const int64_t max_split = std::max<int64_t>(1, vec ? cdiv(in, 64) / 2 : cdiv(in, 16) / (4 * 8));
    int64_t sg = std::max<int64_t>(1, std::min<int64_t>({cdiv(512, nUpper), vec ? 32 : 16, max_split}));
    if (sg >= 8) sg = sg / 8 * 8;  // whole K splits per XCD
    p.splitG = static_cast<int>(sg);
  }
  auto layout = [&]() {
    size_t off = 0;
    p.off_gpart = off;
    if (!p.gram_direct) off += align16(static_cast<size_t>(p.splitG) * r * r * 4);
    p.off_ghi = off;
    off += align16(static_cast<size_t>(r * r * e));
    p.off_glo = off;
    off += align16(static_cast<size_t>(r * r * e));
    p.off_base = off;
    off += align16(static_cast<size_t>(p.nSplit) * out * 4);
    p.off_cross = off;
    off += static_cast<size_t>(p.nSplit) * p.nTiles * out * 4;
    p.off_count = off;  // the fused finalize's counter per row block, right after the cross partials
    off = align16(off + static_cast<size_t>(p.nRB) * 4);
    p.bytes = off;
  };
  layout();
  const size_t bound = norm_scratch_bound(out, r);
  while (p.bytes > bound && p.splitG > 1) {
    --p.splitG;
    layout();
  }
  if (p.bytes > bound && p.splitG == 1) {
    // r large against out: no fp32 partials, the Gram kernel writes G'hi/G'lo
    p.gram_direct = true;
    layout();
  }
  while (p.bytes > bound && p.nSplit > 1) {
    --p.nSplit;
    layout();
  }
  p.strip = vec && norm_strip_fits(out, in, r);
  return p;
}

size_t norm_workspace_bytes(int64_t out, int64_t in, int64_t r, int dtype) {
  size_t b = make_norm_plan(out, in, r, dtype, false).bytes;
  if (in % 8 == 0 && r % 8 == 0) b = std::max(b, make_norm_plan(out, in, r, dtype, true).bytes);
  return b;
}

hipError_t launch_row_sqnorm(const void* W0, int64_t out, int64_t in, int dtype, bool vec, float* sq,
                             hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(cdiv(out, 4))), block(256);
  if (dtype == 0) {
    const auto* w = static_cast<const Dt<0>::T*>(W0);
    if (vec)
      hipLaunchKernelGGL((row_sqnorm<0, true>), grid, block, 0, stream, w, out, in, sq);
    else
      hipLaunchKernelGGL((row_sqnorm<0, false>), grid, block, 0, stream, w, out, in, sq);
  } else {
    const auto* w = static_cast<const Dt<1>::T*>(W0);
    if (vec)
      hipLaunchKernelGGL((row_sqnorm<1, true>), grid, block, 0, stream, w, out, in, sq);
    else
      hipLaunchKernelGGL((row_sqnorm<1, false>), grid, block, 0, stream, w, out, in, sq);
  }
  return hipGetLastError();
}

hipError_t launch_norm(const NormPlan& p, const NormArgs& a) {
  if (p.out <= 0) return hipSuccess;
  return p.dtype == 0 ? launch_norm_t<0>(p, a, p.vec) : launch_norm_t<1>(p, a, p.vec);
}

}  // namespace dora
