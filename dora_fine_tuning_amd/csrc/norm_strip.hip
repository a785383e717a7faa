// Factored weight norm for small adapters (r <= 32) on the 16-byte path, in
// one launch and without workspace.  The summary page's factored-norm
// paragraph splits ||W0_i + s B_i A||^2 into the base term ||W0_i||^2, the
// cross term 2 s B_i . (W0 A^T)_i and the Gram term s^2 B_i (A A^T) B_i^T.
// Here a workgroup owns a strip of 32 rows of W0 and runs over the whole
// input axis, so every sum of its rows ends inside it: no split-K partials,
// no counters, no finalize launch.  At this rank the Gram matrix is cheap
// enough for every workgroup to form it itself, in fp32 accumulators, from
// the A panel stages it already loads for the cross term; no other launch
// has to precede the W0 stream.
//
// Per K stage of 64: the strip's W0 rows (4 KiB) and the r rows of A (r x
// 128 bytes) go global -> LDS by DMA through two rings, each fed by one DMA
// wave (the W0 ring is deep, to keep ~44 KiB of HBM reads in flight per CU;
// the A panel comes from L2).  Four compute waves take one MFMA K step of 16
// each: U = W0 A^T (32 x 32 per rank tile), the upper 32 x 32 blocks of
// G = A A^T, and the squares of the W0 fragment.  After the stage loop each
// compute wave turns its part of U into a partial cross sum per row (B from
// global memory) and leaves its Gram blocks in LDS; the blocks are added in
// wave order and every row's quadratic form B_i G B_i^T is taken in fp32.
// The norm is sqrt(base + 2 s cross + s^2 gram) with the three sums combined
// in fp64.
#include <algorithm>

#include "dma_common.hpp"
#include "norm_kernels.hpp"

namespace dora {

namespace {

template <int NR_>
struct StripTile {
  static constexpr int NR = NR_;                // rank tiles of 32 (r <= 32 NR)
  static constexpr int RM = 32, RN = 32 * NR;   // W0 rows and A rows of a stage
  static constexpr int BK = 64, ROWB = 128;     // K per stage, bytes per LDS row
  static constexpr int NC = 4;                  // compute waves: K step w of every stage
  static constexpr int NT = 64 * (NC + 2);      // + the W0 DMA wave and the A DMA wave
  static constexpr int WI = RM * ROWB / 1024;   // 1 KiB DMA instructions per W0 stage
  static constexpr int AI = RN * ROWB / 1024;   // per A stage
  static constexpr int W_BYTES = RM * ROWB, A_BYTES = RN * ROWB;
  static constexpr int NWS = 12, NAS = NR == 1 ? 14 : 9;  // ring slots
  static constexpr int W_OFF = 0, A_OFF = NWS * W_BYTES;
  static constexpr int LDS_BYTES = A_OFF + NAS * A_BYTES;
  static constexpr int NG = NR * (NR + 1) / 2;  // upper 32 x 32 Gram blocks
  static constexpr int GS = 36;                 // floats per row of a Gram block in LDS (16-byte aligned, padded)
  static constexpr int G_FLOATS = NC * NG * 32 * GS;
  static constexpr int RED_OFF = G_FLOATS * 4;  // then base and cross sums [NC][32] each
  static_assert((NWS - 2) * WI < 64 && (NAS - 2) * AI < 64, "vmcnt range");
  static_assert(RED_OFF + 2 * NC * 32 * 4 <= LDS_BYTES, "epilogue fits in the ring area");
  static_assert(LDS_BYTES > 80 * 1024, "one workgroup per CU");
};

// Block g of the upper Gram blocks, row-major over (jb <= lb)
template <int NR>
__device__ constexpr int gram_jb(int g) {
  return NR == 1 ? 0 : (g < 2 ? 0 : 1);
}
template <int NR>
__device__ constexpr int gram_lb(int g) {
  return NR == 1 ? 0 : (g == 0 ? 0 : 1);
}

// One DMA wave's ring of NSL slots (NI 1 KiB instructions per stage): steps
// 0 .. NSL-2 in a prologue, then at each step's barrier the step NSL-1
// ahead into the slot the previous step freed, and a wait until the next
// step has landed.  Instruction q moves rows 8q .. 8q + 7 of the panel.  Step
// st loads K stage (st + start) mod S: the workgroups start at different K
// stages, so the rows' reads at any moment spread over many column offsets
// (all strips at one offset left the W0 stream near 4.6 TB/s warm; spread,
// near the 6 TB/s of a contiguous read).
template <int NSL, int NI>
__device__ inline void strip_dma_ring(__amdgpu_buffer_rsrc_t rs, char* ring, int slot_bytes, int nrows, int in, int S,
                                      int start, int lane) {
  auto issue = [&](int st, int slot) {
    const int kst = st + start < S ? st + start : st + start - S;  // the K stage loaded at step st
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int row = 8 * q + (lane >> 3);
      const int lc = (lane & 7) ^ ((row >> 1) & 7);
      const int k = kst * 64 + lc * 8;
      const uint32_t o = st < S && row < nrows && k < in ? static_cast<uint32_t>((row * in + k) * 2) : kOob;
      dma16(rs, ring + slot * slot_bytes + q * 1024, o);
    }
  };
  for (int d = 0; d < NSL - 1; ++d) issue(d, d);
  wait_vmcnt<(NSL - 2) * NI>();
  int slot = NSL - 1;
  for (int st = 0; st < S; ++st) {
    __builtin_amdgcn_s_barrier();
    issue(st + NSL - 1, slot);
    slot = slot + 1 == NSL ? 0 : slot + 1;
    wait_vmcnt<(NSL - 2) * NI>();
  }
}

template <int DT, class TL>
__global__ __launch_bounds__(TL::NT, 1) void norm_strip(const void* W0v, const void* Av, const void* Bv, int64_t out,
                                                       int in, int r, float s, const float* base_sq,
                                                       float* norm_out) {
  using T = typename Dt<DT>::T;
  using V8 = typename Dt<DT>::V8;
  __shared__ __attribute__((aligned(1024))) char smem[TL::LDS_BYTES];
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * TL::RM;
  const int S = (in + TL::BK - 1) / TL::BK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_t*)smem));
  const bool want_base = base_sq == nullptr;

  if (wave >= TL::NC) {
    // DMA waves.  Instruction q of a stage moves panel rows 8q .. 8q + 7, 128
    // bytes each; lane l takes row 8q + l/8 and the logical 16-byte chunk
    // (l%8) ^ ((row/2)%8), which lands in LDS slot l%8, so the fragment reads of
    // 16 consecutive rows at one logical chunk hit 16 distinct bank groups.
    // Rows past the operand lie beyond the buffer resource's range and K
    // chunks past in get an out-of-range offset: both read zero.  Stages past
    // the last are issued out of range too (zeros into slots no stage reads),
    // so every wait keeps the same count in flight.
    const bool wdma = wave == TL::NC;
    const int nrows = wdma ? static_cast<int>(std::min<int64_t>(out - row0, TL::RM)) : r;
    const char* base = wdma ? static_cast<const char*>(W0v) + row0 * in * 2 : static_cast<const char*>(Av);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base), static_cast<short>(0), nrows * in * 2, kBufferWord3);
    const int start = static_cast<int>((static_cast<int64_t>(blockIdx.x) * 37) % S);
    if (wdma)
      strip_dma_ring<TL::NWS, TL::WI>(rs, smem + TL::W_OFF, TL::W_BYTES, nrows, in, S, start, lane);
    else
      strip_dma_ring<TL::NAS, TL::AI>(rs, smem + TL::A_OFF, TL::A_BYTES, nrows, in, S, start, lane);
    wait_vmcnt<0>();  // the epilogue reuses the rings
    __syncthreads();
    __syncthreads();
  } else {
    // Compute wave w: K step w of each stage.  Lane l reads row l%32 of each
    // panel at logical chunk 2w + l/32, stored in slot (2w + l/32) ^ ((l%32)/2 % 8).
    const int frow = lane & 31, fh = lane >> 5;
    const uint32_t co = static_cast<uint32_t>(((2 * wave + fh) ^ ((frow >> 1) & 7)) * 16);
    const uint32_t wrow = lds0 + TL::W_OFF + frow * TL::ROWB + co;
    const uint32_t arow = lds0 + TL::A_OFF + frow * TL::ROWB + co;
    f32x16 U[TL::NR], G[TL::NG];
#pragma unroll
    for (int j = 0; j < TL::NR; ++j) U[j] = f32x16{};
#pragma unroll
    for (int g = 0; g < TL::NG; ++g) G[g] = f32x16{};
    float bs = 0.0f;
    int ws = 0, as = 0;
    for (int st = 0; st < S; ++st) {
      __builtin_amdgcn_s_barrier();
      u32x4 x = lds_read16(wrow + ws * TL::W_BYTES), a[TL::NR];
      a[0] = lds_read16(arow + as * TL::A_BYTES);
      if constexpr (TL::NR > 1) a[1 % TL::NR] = lds_read16_at<32 * TL::ROWB>(arow + as * TL::A_BYTES);
      lds_wait();
      tie(x);
#pragma unroll
      for (int j = 0; j < TL::NR; ++j) tie(a[j]);
#pragma unroll
      for (int j = 0; j < TL::NR; ++j)
        U[j] = Dt<DT>::mfma32(__builtin_bit_cast(V8, a[j]), __builtin_bit_cast(V8, x), U[j]);
#pragma unroll
      for (int g = 0; g < TL::NG; ++g)
        G[g] = Dt<DT>::mfma32(__builtin_bit_cast(V8, a[gram_jb<TL::NR>(g)]),
                              __builtin_bit_cast(V8, a[gram_lb<TL::NR>(g)]), G[g]);
      if (want_base) {
        bs = sq2<DT>(x[0], bs);
        bs = sq2<DT>(x[1], bs);
        bs = sq2<DT>(x[2], bs);
        bs = sq2<DT>(x[3], bs);
      }
      ws = ws + 1 == TL::NWS ? 0 : ws + 1;
      as = as + 1 == TL::NAS ? 0 : as + 1;
    }
    __syncthreads();  // every stage read and every DMA drained: the rings are free
    // Lane l holds, in register i of a 32 x 32 result, row 8(i/4) + 4(l/32) + i%4
    // of the A-side operand and column l%32 of the other: U[j] holds
    // U[strip row l%32][rank 32j + that row], G[g] holds G[32jb + that row][32lb + l%32].
    float* gp = reinterpret_cast<float*>(smem) + wave * TL::NG * 32 * TL::GS;
#pragma unroll
    for (int g = 0; g < TL::NG; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) gp[(g * 32 + 8 * (i / 4) + 4 * fh + i % 4) * TL::GS + frow] = G[g][i];
    // partial cross sum of row frow over this wave's K steps: sum_j B[row][j] U[row][j]
    float c = 0.0f;
    const int64_t row = row0 + frow;
    if (row < out) {
      const T* Brow = static_cast<const T*>(Bv) + row * r;
#pragma unroll
      for (int j = 0; j < TL::NR; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = 32 * j + 8 * q + 4 * fh;  // four consecutive ranks; r % 8 == 0
          if (col < r) {
            const uint2 bw = *reinterpret_cast<const uint2*>(Brow + col);
            const T* b4 = reinterpret_cast<const T*>(&bw);
#pragma unroll
            for (int t = 0; t < 4; ++t) c = __builtin_fmaf(Dt<DT>::to_f(b4[t]), U[j][4 * q + t], c);
          }
        }
    }
    c += __shfl_xor(c, 32, 64);
    bs += __shfl_xor(bs, 32, 64);
    float* red = reinterpret_cast<float*>(smem + TL::RED_OFF);
    if (fh == 0) {
      red[wave * 32 + frow] = bs;
      red[TL::NC * 32 + wave * 32 + frow] = c;
    }
    __syncthreads();
  }
  // Gram blocks: the compute waves' parts added in wave order, in place
  float* g0 = reinterpret_cast<float*>(smem);
  constexpr int GBLK = TL::NG * 32 * TL::GS;
  for (int e = tid; e < GBLK; e += TL::NT) {
    float v = g0[e];
#pragma unroll
    for (int w = 1; w < TL::NC; ++w) v += g0[w * GBLK + e];
    g0[e] = v;
  }
  __syncthreads();
  // Row i of the strip: eight threads, thread p taking rows 4p .. 4p + 3 of
  // every Gram block: q_i = sum over blocks of f * B_i,jb G_blk B_i,lb^T
  // (f = 2 off the diagonal, where the lower block is the upper's transpose).
  if (tid < TL::RM * 8) {
    const int i = tid >> 3, p = tid & 7;
    const int64_t row = row0 + i;
    float bf[TL::RN];
    if (row < out) {
      const T* Brow = static_cast<const T*>(Bv) + row * r;
#pragma unroll
      for (int c8 = 0; c8 < TL::RN / 8; ++c8) {
        if (c8 * 8 < r) {
          const uint4 bw = *reinterpret_cast<const uint4*>(Brow + c8 * 8);
          const T* b8 = reinterpret_cast<const T*>(&bw);
#pragma unroll
          for (int t = 0; t < 8; ++t) bf[c8 * 8 + t] = Dt<DT>::to_f(b8[t]);
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t) bf[c8 * 8 + t] = 0.0f;
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < TL::RN; ++t) bf[t] = 0.0f;
    }
    float qv = 0.0f;
#pragma unroll
    for (int g = 0; g < TL::NG; ++g) {
      const int jb = gram_jb<TL::NR>(g), lb = gram_lb<TL::NR>(g);
      float qb = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = 4 * p + t;
        const float* grow = g0 + (g * 32 + m) * TL::GS;
        float acc = 0.0f;
#pragma unroll
        for (int n4 = 0; n4 < 8; ++n4) {
          const float4 gv = *reinterpret_cast<const float4*>(grow + 4 * n4);
          acc = __builtin_fmaf(gv.x, bf[32 * lb + 4 * n4], acc);
          acc = __builtin_fmaf(gv.y, bf[32 * lb + 4 * n4 + 1], acc);
          acc = __builtin_fmaf(gv.z, bf[32 * lb + 4 * n4 + 2], acc);
          acc = __builtin_fmaf(gv.w, bf[32 * lb + 4 * n4 + 3], acc);
        }
        qb = __builtin_fmaf(bf[32 * jb + m], acc, qb);
      }
      qv += jb == lb ? qb : 2.0f * qb;
    }
    qv += __shfl_xor(qv, 1, 64);
    qv += __shfl_xor(qv, 2, 64);
    qv += __shfl_xor(qv, 4, 64);
    if (p == 0 && row < out) {
      const float* red = reinterpret_cast<const float*>(smem + TL::RED_OFF);
      float b = 0.0f, c = 0.0f;
#pragma unroll
      for (int w = 0; w < TL::NC; ++w) {
        b += red[w * 32 + i];
        c += red[TL::NC * 32 + w * 32 + i];
      }
      const double bb = want_base ? static_cast<double>(b) : static_cast<double>(base_sq[row]);
      const double sd = static_cast<double>(s);
      const double n2 = bb + 2.0 * sd * static_cast<double>(c) + sd * sd * static_cast<double>(qv);
      norm_out[row] = static_cast<float>(n2 > 0.0 ? sqrt(n2) : 0.0);
    }
  }
}

template <int DT>
hipError_t launch_strip_t(const NormPlan& p, const NormArgs& a) {
  using TL = StripTile<1>;
  static_assert(32 * TL::NR >= kStripMaxRank, "one rank tile covers every rank the strip path takes");
  const dim3 grid(static_cast<unsigned>(cdiv_strip(p.out)));
  hipLaunchKernelGGL((norm_strip<DT, TL>), grid, dim3(TL::NT), 0, a.stream, a.W0, a.A, a.B, p.out,
                     static_cast<int>(p.in), static_cast<int>(p.r), a.s, a.base_sq, a.norm_out);
  return hipGetLastError();
}

}  // namespace

bool norm_strip_fits(int64_t out, int64_t in, int64_t r) {
  return r > 0 && r <= kStripMaxRank && in > 0 && cdiv_strip(out) >= kStripMinBlocks &&
         static_cast<int64_t>(32) * in * 2 < (int64_t(1) << 31) && r * in * 2 < (int64_t(1) << 31);
}

hipError_t launch_norm_strip(const NormPlan& p, const NormArgs& a) {
  return p.dtype == 0 ? launch_strip_t<0>(p, a) : launch_strip_t<1>(p, a);
}

}  // namespace dora
