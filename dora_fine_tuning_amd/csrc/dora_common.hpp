// Device-side helpers shared by the DoRA kernels: storage-dtype traits, the
// gfx950 MFMA wrappers and 16-byte chunk conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Storage dtype traits.  DT 0 = bf16, 1 = fp16 (the ABI's dtype codes).
// Conversions to the storage type round to nearest even (v_cvt_pk_bf16_f32 /
// v_cvt_f16_f32 on gfx950).
template <int DT>
struct Dt;

template <>
struct Dt<0> {
  using T = __bf16;
  using V8 = bf16x8;
  __device__ static inline float to_f(T x) { return static_cast<float>(x); }
  __device__ static inline T from_f(float x) { return static_cast<T>(x); }
  __device__ static inline T from_d(double x) { return static_cast<T>(static_cast<float>(x)); }
  // D[32x32] += A[32x16] * B[16x32]; lane l holds A row l%32, k 8*(l/32)..+7 and
  // B column l%32, the same k; D element (8*(i/4) + 4*(l/32) + i%4, l%32) in reg i.
  __device__ static inline f32x16 mfma32(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Dt<1> {
  using T = _Float16;
  using V8 = f16x8;
  __device__ static inline float to_f(T x) { return static_cast<float>(x); }
  __device__ static inline T from_f(float x) { return static_cast<T>(x); }
  __device__ static inline T from_d(double x) { return static_cast<T>(x); }
  __device__ static inline f32x16 mfma32(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// A 16-byte chunk (8 storage elements) moved as one global/LDS access.
struct alignas(16) Chunk {
  uint32_t w[4];
};

template <int DT>
__device__ inline void chunk_to_f32(const Chunk& c, float (&f)[8]) {
  using V8 = typename Dt<DT>::V8;
  V8 v = __builtin_bit_cast(V8, c);
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = Dt<DT>::to_f(v[j]);
}

template <int DT>
__device__ inline Chunk f32_to_chunk(const float (&f)[8]) {
  using V8 = typename Dt<DT>::V8;
  V8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = Dt<DT>::from_f(f[j]);
  return __builtin_bit_cast(Chunk, v);
}

__device__ inline Chunk zero_chunk() {
  Chunk c;
  c.w[0] = c.w[1] = c.w[2] = c.w[3] = 0u;
  return c;
}

}  // namespace dora
