// Compose forward with the adapter's second projection fused in, for gfx950:
//
//   y = (g - 1) * base + g * s * (h B^T)   (+ base),   g_j = m_j / n_j,
//
// with h = x A^T [T x r] and B [out x r] (press summary of arXiv:2603.22276:
// the fused kernel's gains come from fewer memory accesses).  lora = h B^T
// lives only in the MFMA accumulators: the kernel reads base once, writes y
// once, and reads h and B (small, L2 / last-level-cache resident) per tile.
//
// Kernels:
//   lora_fwd_dma      (16-byte path) a workgroup owns 32*TM tokens x 128*TN
//                     output columns and the whole K = r axis.  K stages of 32
//                     go global -> LDS by DMA into an NS-slot ring (h rows as
//                     the X panel, B rows as the Y panel in the fragment row
//                     order), MFMA 32x32x16 with fp32 accumulation, then an
//                     epilogue straight from the accumulators: the tile's base
//                     block comes into the freed ring by DMA, and a lane,
//                     holding one token row and 16 consecutive output columns
//                     per 32x32 tile, reads its base from LDS and writes y as
//                     two 16-byte chunks per tile;
//   lora_fwd_general  (general path) one thread per output element, the r-term
//                     dot product in order in fp32.
#include <algorithm>

#include "dma_common.hpp"
#include "dora_common.hpp"
#include "lora_compose_kernels.hpp"

namespace dora {

namespace {

inline int64_t lcdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile geometry: NW = WM*4 waves in a WM x 4 grid (WM along the tokens, 4 along
// the output columns); a wave owns TMW = TM/WM token tiles x TN column tiles of
// 32 and keeps their accumulators in registers.  A K stage holds one segment of
// BK elements (ROWB = 2*BK bytes, CPR 16-byte chunks) of each panel row; one
// wave DMA instruction moves RPI = 1024/ROWB rows, lane l taking row l/CPR and
// the logical chunk (l%CPR) ^ ((row/SWP)%CPR), SWP = 16/CPR, which lands in LDS
// slot l%CPR; the fragment reads of 16 consecutive rows at one logical chunk
// then hit 16 distinct bank groups.
template <int TN_, int TM_, int NS_, int WM_, int BK_ = 32>
struct LoraTile {
  static constexpr int TN = TN_, TM = TM_, NS = NS_, WM = WM_;
  static constexpr int WN = 4, NW = WM * WN, NT = NW * 64;
  static constexpr int TMW = TM / WM;
  static constexpr int BM = 32 * TM, BN = 32 * WN * TN;
  static constexpr int BK = BK_, ROWB = 2 * BK, CPR = ROWB / 16, RPI = 1024 / ROWB, SWP = 16 / CPR;
  static constexpr int KS = BK / 16;  // MFMA K steps per stage, done in pairs
  static constexpr int X_BYTES = BM * ROWB, Y_BYTES = BN * ROWB, STAGE_BYTES = X_BYTES + Y_BYTES;
  static constexpr int XQ = BM / RPI / NW, YQ = BN / RPI / NW;
  static constexpr int L = XQ + YQ;  // DMA instructions per wave and stage
  static constexpr int LDS_BYTES = NS * STAGE_BYTES;
  static_assert(TM % WM == 0, "token tiles split over the waves");
  static_assert((BM / RPI) % NW == 0 && (BN / RPI) % NW == 0, "panels split into whole DMA groups per wave");
  static_assert(LDS_BYTES + 2 * BN * 4 <= 160 * 1024, "LDS: ring and column scales");
  static_assert(BM * BN * 2 <= LDS_BYTES, "the epilogue's base block fits the ring");
  static_assert(BK == 32 || BK == 64, "64- or 128-byte row segments");
  static_assert(NS >= 2 && NS <= 8 && (NS - 2) * L < 64, "ring depth and vmcnt range");
};

// 256 tokens x 256 columns, 8 waves, one workgroup per CU.  K stages of 64
// (128-byte row segments, whole cache lines) in two ring slots of 64 KB: the
// DMA of stage u + 1 overlaps the MFMAs of stage u.
using LoraTileMain = LoraTile<2, 8, 2, 2, 64>;

// Column tiles per group of the tile order (below): the largest power of two
// from 4 to 16 whose B slice (group x 256 rows x r) stays within 1.5 MiB, well
// inside an XCD's 4 MiB L2.  Wider groups make the concurrent tiles of an XCD
// cover longer runs of each base row.  Measured at T x out (r), warm / cold us:
// 4096^2 (64) 19.6 / 21.6 with 16 against 22.9 / 24.3 with 4; 8192^2 (384)
// 93.2 / 100.8 with 8 against 95.0 / 103.2; at 10240 x 27648 (512), whose
// B slice of 16 tiles is 4 MiB, 16 and 8 were 7-19 us slower cold than 4.
inline uint32_t lora_group_cols(int64_t r) {
  const int64_t slice = 256 * std::max<int64_t>(r, 1) * 2;  // bytes of B per column tile
  uint32_t g = 16;
  while (g > 4 && static_cast<int64_t>(g) * slice > (int64_t(3) << 19)) g /= 2;
  return g;
}

struct LoraArgs {
  const void *base, *h, *B;
  const float *mag, *norm;
  void* y;
  float s;
  int add_base;
  int64_t T, out, r;
  int nRB, nTiles, S;
  uint32_t group;  // column tiles per group of the tile order
};

// Wait for the current stage's DMA while the n younger stages already issued
// (at most NS-2) stay in flight; n is wave-uniform.
template <class TL, int N = TL::NS - 2>
__device__ inline void lora_wait_younger(int n) {
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= N)
      wait_vmcnt<N * TL::L>();
    else
      lora_wait_younger<TL, N - 1>(n);
  }
}

template <int DT, class TL>
__global__ __launch_bounds__(TL::NT, 2) void lora_fwd_dma(LoraArgs a) {
  using V8 = typename Dt<DT>::V8;
  __shared__ __attribute__((aligned(1024))) char smem[TL::LDS_BYTES + 2 * TL::BN * 4];

  const uint32_t v = static_cast<uint32_t>(xcd_logical_index());
  const uint32_t total = static_cast<uint32_t>(a.nRB) * static_cast<uint32_t>(a.nTiles);
  if (v >= total) return;
  // Tile order: groups of a.group column tiles, token blocks within a group.
  // With the XCD-contiguous numbering an XCD then works on one group's B slice
  // (a.group x 256 rows of B stay in its L2) while it sweeps the token
  // blocks, instead of streaming all of B once per token block.
  const uint32_t nRB = static_cast<uint32_t>(a.nRB), nTl = static_cast<uint32_t>(a.nTiles);
  const uint32_t G = a.group;
  const uint32_t grp = v / (G * nRB);
  const uint32_t gn = std::min<uint32_t>(G, nTl - grp * G);
  const uint32_t loc = v - grp * G * nRB;
  const int rb = static_cast<int>(loc / gn);
  const int nt = static_cast<int>(grp * G + loc % gn);
  const int64_t m0 = static_cast<int64_t>(rb) * TL::BM, n0 = static_cast<int64_t>(nt) * TL::BN;
  const int64_t T = a.T, out = a.out;
  const int r = static_cast<int>(a.r), S = a.S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_t*)smem));

  // Buffer resources, rebased to the tile's first row; rows past the operand
  // lie beyond num_records and read zero.  Offsets stay below 2^31 (at most
  // 256 rows of r <= 2^20 or out < 2^22 elements).
  auto rsrc = [](const void* base, int64_t row0, int64_t rows, int64_t ld, int64_t max_rows) {
    const int64_t nrows = std::min<int64_t>(std::max<int64_t>(rows - row0, 0), max_rows);
    const char* p = static_cast<const char*>(base) + (nrows > 0 ? row0 * ld * 2 : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), static_cast<short>(0),
                                             static_cast<int>(nrows * ld * 2), kBufferWord3);
  };
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.h, m0, T, r, TL::BM);
  const __amdgpu_buffer_rsrc_t ry = rsrc(a.B, n0, out, r, TL::BN);

  // Per-lane DMA geometry (as in the W stream of the factored norm): the Y
  // panel is fetched in the row order sigma of the fragment reads, so that
  // accumulator register q of a lane in half h holds column 16h + q of its tile.
  const int lrow = lane / TL::CPR, lslot = lane % TL::CPR;
  // instruction q of the wave starts at row (q*NW + wave)*RPI, and q*NW*RPI is
  // a multiple of SWP*CPR: the chunk depends on the wave's row of instruction 0
  const int lc = lslot ^ (((wave * TL::RPI + lrow) / TL::SWP) % TL::CPR);
  const int kc = lc * 8;
  auto sigma = [](int p) { return 16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3); };
  const int xr0 = wave * TL::RPI + lrow;
  const int yp = wave * TL::RPI + lrow;
  const int yr0 = (yp & ~31) + sigma(yp & 31);
  const uint32_t ld = static_cast<uint32_t>(r) * 2u;
  const uint32_t lx = static_cast<uint32_t>(xr0) * ld + kc * 2u, ly = static_cast<uint32_t>(yr0) * ld + kc * 2u;

  const int frow = lane & 31, fhalf = lane >> 5, fsw = (frow / TL::SWP) % TL::CPR;
  const uint32_t xrow = lds0 + static_cast<uint32_t>((wm * TL::TMW * 32 + frow) * TL::ROWB);
  const uint32_t yrow = lds0 + static_cast<uint32_t>(TL::X_BYTES + (wn * TL::TN * 32 + frow) * TL::ROWB);
  // K step k reads logical chunk 2k + fhalf of its rows
  uint32_t cofs[TL::KS];
#pragma unroll
  for (int k = 0; k < TL::KS; ++k) cofs[k] = static_cast<uint32_t>(((2 * k + fhalf) ^ fsw) * 16);

  f32x16 acc[TL::TMW][TL::TN];
#pragma unroll
  for (int i = 0; i < TL::TMW; ++i)
#pragma unroll
    for (int j = 0; j < TL::TN; ++j) acc[i][j] = f32x16{};

  // DMA of K stage ST into ring slot SLOT; lanes past r in the last stage get
  // an out-of-range offset (zeros).
  auto issue = [&](int st, int slot) {
    const uint32_t kb = static_cast<uint32_t>(st) * TL::ROWB;
    const int krem = r - st * TL::BK;
    const bool tail = krem < TL::BK && kc >= krem;
    char* so = smem + slot * TL::STAGE_BYTES;
#pragma unroll
    for (int q = 0; q < TL::XQ; ++q)
      dma16(rx, so + (q * TL::NW + wave) * 1024, tail ? kOob : lx + static_cast<uint32_t>(q * TL::NW * TL::RPI) * ld + kb);
#pragma unroll
    for (int q = 0; q < TL::YQ; ++q)
      dma16(ry, so + TL::X_BYTES + (q * TL::NW + wave) * 1024,
            tail ? kOob : ly + static_cast<uint32_t>(q * TL::NW * TL::RPI) * ld + kb);
  };

  // The epilogue's base block: BM rows of BN*2 bytes, row t's logical 16-byte
  // chunk c in slot c ^ (t % 32) (see the epilogue); DMA of rows [h*R, h*R + R),
  // R = BM / NS, which land in ring slot h.
  constexpr int EROWB = TL::BN * 2, ECPR = EROWB / 16, ERPI = 1024 / EROWB;
  static_assert(ECPR == 32 && ERPI * EROWB == 1024, "base rows of 32 chunks, two per DMA instruction");
  static_assert(TL::BM * EROWB == TL::NS * TL::STAGE_BYTES, "the base block fills the ring, one part per slot");
  const __amdgpu_buffer_rsrc_t rbase = rsrc(a.base, m0, T, out, TL::BM);
  auto issue_base = [&](int h) {
    constexpr int QH = TL::BM / ERPI / TL::NS;  // DMA instructions per slot
    const int erow = lane / ECPR, eslot = lane % ECPR;
#pragma unroll
    for (int q = h * QH + wave; q < (h + 1) * QH; q += TL::NW) {
      const int row = q * ERPI + erow;
      const int64_t col = n0 + 8 * (eslot ^ (row % ECPR));
      const uint32_t off = col < out ? static_cast<uint32_t>((static_cast<int64_t>(row) * out + col) * 2) : kOob;
      dma16(rbase, smem + q * 1024, off);
    }
  };

#pragma unroll
  for (int u = 0; u < TL::NS - 1; ++u)
    if (u < S) issue(u, u);

  constexpr int tstep = 32 * TL::ROWB;
  for (int sb = 0; sb < S; sb += TL::NS) {
#pragma unroll
    for (int u = 0; u < TL::NS; ++u) {
      const int st = sb + u;
      if (st >= S) break;
      lora_wait_younger<TL>(S - 1 - st);
      __builtin_amdgcn_s_barrier();
      if (st + TL::NS - 1 < S) issue(st + TL::NS - 1, (u + TL::NS - 1) % TL::NS);
      // last stage: the slot of the one before it is free; its part of the
      // base block comes in during this stage's MFMAs
      if (TL::NS == 2 && st == S - 1 && S >= 2) issue_base((u + 1) % 2);
      const uint32_t so = static_cast<uint32_t>(u * TL::STAGE_BYTES);
#pragma unroll
      for (int kp = 0; kp < TL::KS; kp += 2) {
      u32x4 x0[TL::TMW], y0[TL::TN], x1[TL::TMW], y1[TL::TN];
#pragma unroll
      for (int i = 0; i < TL::TMW; ++i) x0[i] = lds_read16(xrow + cofs[kp] + so + i * tstep);
#pragma unroll
      for (int j = 0; j < TL::TN; ++j) y0[j] = lds_read16(yrow + cofs[kp] + so + j * tstep);
#pragma unroll
      for (int i = 0; i < TL::TMW; ++i) x1[i] = lds_read16(xrow + cofs[kp + 1] + so + i * tstep);
#pragma unroll
      for (int j = 0; j < TL::TN; ++j) y1[j] = lds_read16(yrow + cofs[kp + 1] + so + j * tstep);
      lds_wait_keep<TL::TMW + TL::TN>();
#pragma unroll
      for (int i = 0; i < TL::TMW; ++i) tie(x0[i]);
#pragma unroll
      for (int j = 0; j < TL::TN; ++j) tie(y0[j]);
#pragma unroll
      for (int i = 0; i < TL::TMW; ++i)
#pragma unroll
        for (int j = 0; j < TL::TN; ++j)
          acc[i][j] = Dt<DT>::mfma32(__builtin_bit_cast(V8, y0[j]), __builtin_bit_cast(V8, x0[i]), acc[i][j]);
      lds_wait();
#pragma unroll
      for (int i = 0; i < TL::TMW; ++i) tie(x1[i]);
#pragma unroll
      for (int j = 0; j < TL::TN; ++j) tie(y1[j]);
#pragma unroll
      for (int i = 0; i < TL::TMW; ++i)
#pragma unroll
        for (int j = 0; j < TL::TN; ++j)
          acc[i][j] = Dt<DT>::mfma32(__builtin_bit_cast(V8, y1[j]), __builtin_bit_cast(V8, x1[i]), acc[i][j]);
      }
    }
  }

  // Epilogue.  The ring is free once every wave is past its last fragment
  // read; the tile's base block (BM rows x BN columns, 2 bytes each) then goes
  // global -> LDS by DMA, all of it in flight at once (a lane loading its own
  // rows of base one at a time leaves too few loads in flight to cover the
  // memory latency); with two ring slots the part in the next-to-last stage's
  // slot was issued during the last stage.  Row t of the block is BN*2 bytes,
  // its logical 16-byte chunk c in slot c ^ (t % 32): the reads below, 32 rows
  // at one logical chunk, then spread over the banks.  Columns past out read
  // zero.  The
  // column scales (g - 1, g*s) sit after the ring.  A lane then walks its
  // TMW token rows; per row it needs 2*TN chunks of 8 columns (16 consecutive
  // columns c0 .. c0 + 15 per column tile j, whole chunks since out % 8 == 0),
  // and the four stores that complete a row's 128-byte line of y follow each
  // other, so the L2 merges them before any write-back.  The whole block is in
  // LDS before the first store, so y may be base.
  using T16 = typename Dt<DT>::T;
  T16* y = static_cast<T16*>(a.y);
  float* sc = reinterpret_cast<float*>(smem + TL::LDS_BYTES);  // [2][BN]: g - 1, then g*s
  // every wave is past its last fragment read (each waited for its own LDS
  // reads): a bare barrier, so the base loads already in flight keep flying
  __builtin_amdgcn_s_barrier();
  {
    // the parts not issued during the last stage (all of them when S < 2)
    const int early = (TL::NS == 2 && S >= 2) ? (S - 2) % 2 : -1;
#pragma unroll
    for (int h = 0; h < TL::NS; ++h)
      if (h != early) issue_base(h);
  }
  if (tid < TL::BN) {
    const int64_t c = n0 + tid;
    float gm1 = 0.0f, gs = 0.0f;
    if (c < out) {
      const float m = a.mag[c], n = a.norm[c];
      gm1 = (m - n) / n;
      gs = (m / n) * a.s;
    }
    sc[tid] = gm1;
    sc[TL::BN + tid] = gs;
  }
  wait_vmcnt<0>();
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TL::TMW; ++i) {
    const int rl = wm * TL::TMW * 32 + i * 32 + frow;  // row within the block (rl % 32 == frow)
    const int64_t t = m0 + rl;
    u32x4 cb[TL::TN][2];
#pragma unroll
    for (int j = 0; j < TL::TN; ++j)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int c = (wn * TL::TN * 32 + j * 32 + 16 * fhalf) / 8 + k;  // logical chunk
        cb[j][k] = lds_read16(lds0 + static_cast<uint32_t>(rl * EROWB + ((c ^ frow) * 16)));
      }
    lds_wait();
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < TL::TN; ++j) {
      const int cl = wn * TL::TN * 32 + j * 32 + 16 * fhalf;  // first column within the tile
      const int64_t c0 = n0 + cl;
      if (c0 >= out) continue;
      const int64_t idx = t * out + c0;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (k == 1 && c0 + 8 >= out) continue;
        tie(cb[j][k]);
        // the chunk's 8 column scales, read from LDS where they are used
        const f32x4 g1a = *reinterpret_cast<const f32x4*>(sc + cl + 8 * k);
        const f32x4 g1b = *reinterpret_cast<const f32x4*>(sc + cl + 8 * k + 4);
        const f32x4 g2a = *reinterpret_cast<const f32x4*>(sc + TL::BN + cl + 8 * k);
        const f32x4 g2b = *reinterpret_cast<const f32x4*>(sc + TL::BN + cl + 8 * k + 4);
        float b[8], o[8];
        chunk_to_f32<DT>(__builtin_bit_cast(Chunk, cb[j][k]), b);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float gm1 = e < 4 ? g1a[e] : g1b[e - 4], gs = e < 4 ? g2a[e] : g2b[e - 4];
          const float d = __builtin_fmaf(gs, acc[i][j][8 * k + e], gm1 * b[e]);
          o[e] = a.add_base ? b[e] + d : d;
        }
        *reinterpret_cast<u32x4*>(y + idx + 8 * k) = __builtin_bit_cast(u32x4, f32_to_chunk<DT>(o));
      }
    }
  }
}

// General path: one thread per output element, lora_tj = sum_k h_tk B_jk in
// order in fp32, then the compose.
template <int DT>
__global__ __launch_bounds__(256) void lora_fwd_general(LoraArgs a) {
  using T16 = typename Dt<DT>::T;
  const T16* h = static_cast<const T16*>(a.h);
  const T16* B = static_cast<const T16*>(a.B);
  const T16* base = static_cast<const T16*>(a.base);
  T16* y = static_cast<T16*>(a.y);
  const int64_t n = a.T * a.out;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = e / a.out, j = e % a.out;
    float l = 0.0f;
    for (int64_t k = 0; k < a.r; ++k) l = __builtin_fmaf(Dt<DT>::to_f(h[t * a.r + k]), Dt<DT>::to_f(B[j * a.r + k]), l);
    const float m = a.mag[j], nn = a.norm[j];
    const float gm1 = (m - nn) / nn, gs = (m / nn) * a.s;
    const float b = Dt<DT>::to_f(base[e]);
    const float d = __builtin_fmaf(gs, l, gm1 * b);
    y[e] = Dt<DT>::from_f(a.add_base ? b + d : d);
  }
}

constexpr int kGenBlocks = 4096;

}  // namespace

int64_t lora_fwd_max_grid(int64_t T, int64_t out, bool vec) {
  if (!vec) return kGenBlocks;
  using TL = LoraTileMain;
  return lcdiv(lcdiv(T, TL::BM) * lcdiv(out, TL::BN), 8) * 8;
}

hipError_t launch_lora_fwd(const LoraFwdArgs& p, bool vec) {
  using TL = LoraTileMain;
  LoraArgs a{};
  a.base = p.base;
  a.h = p.h;
  a.B = p.B;
  a.mag = p.mag;
  a.norm = p.norm;
  a.y = p.y;
  a.s = p.s;
  a.add_base = p.add_base;
  a.T = p.T;
  a.out = p.out;
  a.r = p.r;
  if (vec) {
    a.nRB = static_cast<int>(lcdiv(p.T, TL::BM));
    a.nTiles = static_cast<int>(lcdiv(p.out, TL::BN));
    a.group = lora_group_cols(p.r);
    a.S = static_cast<int>(lcdiv(p.r, TL::BK));
    const dim3 grid(static_cast<unsigned>(lora_fwd_max_grid(p.T, p.out, true)));
    if (p.dtype == 0)
      hipLaunchKernelGGL((lora_fwd_dma<0, TL>), grid, dim3(TL::NT), 0, p.stream, a);
    else
      hipLaunchKernelGGL((lora_fwd_dma<1, TL>), grid, dim3(TL::NT), 0, p.stream, a);
  } else {
    const int64_t blocks = std::min<int64_t>(lcdiv(p.T * p.out, 256), kGenBlocks);
    if (p.dtype == 0)
      hipLaunchKernelGGL((lora_fwd_general<0>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, p.stream, a);
    else
      hipLaunchKernelGGL((lora_fwd_general<1>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, p.stream, a);
  }
  return hipGetLastError();
}

}  // namespace dora
