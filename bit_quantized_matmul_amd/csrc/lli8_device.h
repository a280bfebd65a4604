// Device-side helpers shared by the lli8 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lli8 {

enum : int { DT_F16 = 0, DT_BF16 = 1 };

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// 16-bit storage -> fp32 (exact for both formats).
template <int DT>
__device__ __forceinline__ float to_f32(uint32_t bits16) {
  if constexpr (DT == DT_F16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  } else {
    return __uint_as_float(bits16 << 16);
  }
}

// fp32 -> 16-bit storage, round to nearest even.
template <int DT>
__device__ __forceinline__ uint16_t from_f32(float v) {
  if constexpr (DT == DT_F16) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
  } else {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
  }
}

// Element e (0..7) of a 16-byte chunk of eight 16-bit values.
__device__ __forceinline__ uint32_t half_bits(const u32x4& c, int e) {
  uint32_t w = c[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// The int8 code of x for a row whose scale factor is s = fl32(127 / absmax):
// round(fl32(x * s)) with halves away from zero (roundf), kept in [-127, 127].
__device__ __forceinline__ int quant_code(float x, float s) {
  float v = x * s;
  float r = roundf(v);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, WAVE));
  return v;
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v |= __shfl_xor(v, off, WAVE);
  return v;
}

// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    int u = __shfl_up(v, off, WAVE);
    if (lane >= off) v += u;
  }
  return v;
}

}  // namespace lli8
