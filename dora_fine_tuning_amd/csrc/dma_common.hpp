// Device helpers of the direct global -> LDS (DMA) kernels on gfx950: buffer
// resources and 16-byte-per-lane loads into LDS, waits on the vector-memory
// counter, LDS fragment reads issued as inline assembly, the XCD-aware
// workgroup numbering, and packed squares for the base term.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dora_common.hpp"

namespace dora {

// Workgroups are dealt to the 8 XCDs round-robin by index; renumber them so
// each XCD receives a contiguous range of the logical work list.  gridDim.x is
// a multiple of 8.
__device__ inline int64_t xcd_logical_index() {
  const int64_t b = blockIdx.x;
  return (b & 7) * (gridDim.x >> 3) + (b >> 3);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kOob = 0xFFFFFF00u;   // buffer offset past any range: loads read zero
constexpr int kBufferWord3 = 0x00020000;  // raw (untyped) buffer resource, gfx9 family

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS fragment reads are issued as inline assembly: the compiler cannot tell
// them apart from the in-flight DMA writes into other stages and would
// otherwise wait for every outstanding load before each read.  lds_wait()
// completes them; tie() keeps the MFMAs that use a fragment after that wait.
__device__ inline u32x4 lds_read16(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ inline void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// wait until at most N LDS reads of this wave are outstanding (they complete in order)
template <int N>
__device__ inline void lds_wait_keep() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}
__device__ inline void tie(u32x4& v) { asm volatile("" : "+v"(v)); }
// One 16-byte-per-lane buffer load straight into LDS: lane l writes bytes
// [16l, 16l + 16) of the 1 KiB block at lds (wave-uniform); offsets at or past
// the resource's num_records read zero.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, char* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 16, off, 0, 0, 0);
}
// ds_read_b128 at a per-lane base plus a compile-time byte offset
template <int OFF>
__device__ inline u32x4 lds_read16_at(uint32_t base) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF) : "memory");
  return v;
}

// acc + x0^2 + x1^2 for the two storage-dtype values packed in w (one dot2 instruction)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <int DT>
__device__ inline float sq2(uint32_t w, float acc);
template <>
__device__ inline float sq2<0>(uint32_t w, float acc) {
  const bf16x2_t v = __builtin_bit_cast(bf16x2_t, w);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}
template <>
__device__ inline float sq2<1>(uint32_t w, float acc) {
  const f16x2_t v = __builtin_bit_cast(f16x2_t, w);
  return __builtin_amdgcn_fdot2(v, v, acc, false);
}

}  // namespace dora
