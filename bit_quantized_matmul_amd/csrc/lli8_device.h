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

// fl32(p / 127), correctly rounded.  For 2^-100 <= |p| < 2^101 and for zero
// one multiply by fl32(1/127) and one FMA correction give the same bits as
// the IEEE division (checked on the device against the division for every
// float in that range, both signs); other values (tiny, huge, inf, NaN) take
// the division itself.
// The multiply-and-correct form alone, for callers that know p is in
// range: p = fl32(c * s) with |c| <= 127 an integer and 2^-93 <= s < 2^94
// (div127_scale_ok) lies in it, or is zero.
__device__ __forceinline__ float div127_inrange(float p) {
  constexpr float r = 1.0f / 127.0f;
  const float q0 = p * r;
  const float e = __builtin_fmaf(-q0, 127.0f, p);  // exact remainder
  return __builtin_fmaf(e, r, q0);
}
__device__ __forceinline__ bool div127_scale_ok(float s) { return s >= 0x1p-93f && s < 0x1p94f; }

__device__ __forceinline__ float div127(float p) {
  constexpr float r = 1.0f / 127.0f;
  const float a = __builtin_fabsf(p);
  if (a < 0x1p101f && (a >= 0x1p-100f || a == 0.0f)) {
    const float q0 = p * r;
    const float e = __builtin_fmaf(-q0, 127.0f, p);  // exact remainder
    return __builtin_fmaf(e, r, q0);
  }
  return p / 127.0f;
}

// Element e (0..7) of a 16-byte chunk of eight 16-bit values.
__device__ __forceinline__ uint32_t half_bits(const u32x4& c, int e) {
  uint32_t w = c[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// A row whose absmax is below 2^-100 (only bf16 reaches it: the smallest fp16
// absmax is 2^-24) has its values and its absmax scaled by 2^64 first, exactly,
// so that 127 / absmax stays finite; wherever the plain factor is finite the
// codes are the same either way.
constexpr float TINY_ABSMAX = 0x1p-100f;
constexpr float PRESCALE = 0x1p64f;
__device__ __forceinline__ bool tiny_absmax(float m) { return m > 0.0f && m < TINY_ABSMAX; }
// s = fl32(127 / absmax), with the absmax prescaled when it is tiny
__device__ __forceinline__ float row_factor(float m) {
  return (m > 0.0f) ? 127.0f / (tiny_absmax(m) ? m * PRESCALE : m) : 0.0f;
}

// The int8 code of x for a row whose scale factor is s = fl32(127 / absmax):
// round(fl32(x * s)) with halves away from zero (roundf), kept in [-127, 127]
// (PRE: x prescaled, for a row with a tiny absmax).
template <bool PRE = false>
__device__ __forceinline__ int quant_code(float x, float s) {
  float v = (PRE ? x * PRESCALE : x) * s;
  float r = roundf(v);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

// Codes of the two 16-bit values of x for row factor s = fl32(127 / absmax),
// as two int16 in one dword.  v = fl32(|x| * s) <= 127.5 (for fp16 one
// v_fma_mix_f32 with a zero addend: the same single rounding of the exact
// product), and round-half-away(v) = floor(v + 0.5) for v >= 0, which
// v_cvt_rpi_i32_f32 computes.  Its result is the same whether or not the
// hardware rounds v + 0.5 to fp32 first: the one value where that rounding
// would reach the next integer, v = 0.5 - 2^-25, is not the product of any
// fp16 or bf16 value with the scale of any fp16 or bf16 absmax.  The sign of
// x is applied to both magnitudes at once with packed 16-bit arithmetic.
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int cvt_rpi(float v) {
  int r;
  asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

template <int DT, bool PRE = false>
__device__ __forceinline__ float scaled_abs(uint32_t bits16, float s) {
  if constexpr (DT == DT_F16)
    return __builtin_fmaf(__builtin_fabsf((float)__builtin_bit_cast(_Float16, (uint16_t)bits16)), s, 0.0f);
  else if constexpr (PRE)
    return (__uint_as_float((bits16 & 0x7FFFu) << 16) * PRESCALE) * s;
  else
    return __uint_as_float((bits16 & 0x7FFFu) << 16) * s;
}

template <int DT, bool PRE = false>
__device__ __forceinline__ uint32_t code_pair16(uint32_t x, float s) {
  const int mlo = cvt_rpi(scaled_abs<DT, PRE>(x & 0xFFFFu, s));
  const int mhi = cvt_rpi(scaled_abs<DT, PRE>(x >> 16, s));
  // the low 16 bits of each: a value of an excluded (outlier) column, scaled
  // by a row absmax taken without it, can run far past 16 bits, and its code
  // (discarded later) must not carry into its neighbour's half
  const i16x2 mag = __builtin_bit_cast(i16x2, __builtin_amdgcn_perm((uint32_t)mhi, (uint32_t)mlo, 0x05040100u));
  const i16x2 neg = __builtin_bit_cast(i16x2, x) >> 15;  // -1 where x < 0
  return __builtin_bit_cast(uint32_t, (i16x2)((mag ^ neg) - neg));
}

// Low bytes of the four int16 codes in two dwords, packed little-endian.
__device__ __forceinline__ uint32_t pack_codes16(uint32_t p01, uint32_t p23) {
  return __builtin_amdgcn_perm(p23, p01, 0x06040200u);
}

// Larger of each 16-bit half (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

// 0xFF in every byte whose bit is set in the low 4 bits of f.
__device__ __forceinline__ uint32_t byte_mask4(uint32_t f) {
  return ((f & 1u) * 0xFFu) | (((f >> 1) & 1u) * 0xFF00u) | (((f >> 2) & 1u) * 0xFF0000u) |
         (((f >> 3) & 1u) * 0xFF000000u);
}

// Threshold test on raw 16-bit values: |x| > tau  <=>  (bits & 0x7FFF) > t16,
// where t16 is the largest 15-bit magnitude whose value is <= tau (both
// formats order finite magnitudes like their bit patterns).  0xFFFF when the
// threshold disables the split (tau <= 0, +inf): no magnitude exceeds it.
template <int DT>
__device__ __forceinline__ uint32_t magnitude_threshold(float tau) {
  if (!(tau > 0.0f && tau <= 3.4028235e38f)) return 0xFFFFu;
  uint32_t bb = from_f32<DT>(tau);
  if (to_f32<DT>(bb) > tau) bb -= 1u;
  return bb & 0x7FFFu;
}

// Outlier flags (bit e) of the eight values of a chunk from their packed
// 15-bit magnitudes (m[d] holds values 2d and 2d + 1).
__device__ __forceinline__ uint32_t flags8(const uint32_t (&m)[4], uint32_t t16) {
  uint32_t f = 0u;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    f |= (((m[d] & 0xFFFFu) > t16) ? (1u << (2 * d)) : 0u) | (((m[d] >> 16) > t16) ? (2u << (2 * d)) : 0u);
  return f;
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

// Inclusive prefix sum across the wave, in registers (DPP, no LDS round
// trips): within each row of 16 lanes by row shifts of 1, 2, 4 and 8 lanes
// (lanes shifted in from outside the row read 0), then across rows by the
// gfx9 row broadcasts: lane 15 of rows 0 and 2 into rows 1 and 3, then lane
// 31 (the total of rows 0-1) into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2 and 3
  return v;
}

}  // namespace lli8
