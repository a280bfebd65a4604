// Vector-wise quantisation of a 16-bit matrix on its own: absmax or
// zero-point, one scale per row or per column ("Hugging Face integrates
// LLM.int8() ...", section "Quantization mechanics": both schemes, either
// way).  Not a step of the forward; the forward's own quantisers live in
// lli8_quant.hip and lli8_decode.hip.
//
//   absmax:     code = clamp(round_half_away(fl32(x * fl32(127 / amax))), +-127),
//               scale = amax (0 for an all-zero vector, codes 0); below 2^-100
//               x and amax are scaled by 2^64 first, as in the forward
//               (zero-point with a range below 254 / FLT_MAX is outside the
//               contract: its stored factor nd would overflow)
//   zero-point: lo = min(min x, 0), hi = max(max x, 0), nd = fl32(254 / fl32(hi - lo)),
//               zp = round_half_away(fl32(-lo * nd)) - 127,
//               code = clamp(round_half_away(fl32(x * nd)) + zp, +-127),
//               scale = nd, zero point = zp (0 and 0 for an all-zero vector)
//
// Both are HBM-bound codecs: read X once from memory, write the codes once.
// Absmax per row runs the weight quantiser of lli8_quant.hip (the same
// computation).  Otherwise row-wise: one wave per row, the row held in
// registers (rows up to 12288 values; longer ones take a statistics pass and
// then a code pass over the same row, in cache by then).  Column-wise: one
// workgroup per 32- or 64-column strip, 8 columns per thread, the strip's
// rows held in registers (up to 32 rows per thread: 4096 rows of a 32-column
// strip; more rows are walked twice, statistics then codes); one launch, no
// atomics, no scratch.
#include <type_traits>

#include "lli8_device.h"
#include "lli8_internal.h"

namespace lli8 {

namespace {

// Statistics of one vector -> (scale, zero point) of the chosen scheme.
template <int ZP>
__device__ __forceinline__ void finish_stats(float lo, float hi, float& scale, int& zp, float& mul) {
  if constexpr (ZP) {
    lo = fminf(lo, 0.0f);
    hi = fmaxf(hi, 0.0f);
    const float width = hi - lo;
    if (width > 0.0f) {
      const float nd = 254.0f / width;
      scale = nd;
      mul = nd;
      zp = (int)roundf(-lo * nd) - 127;
    } else {
      scale = 0.0f;
      mul = 0.0f;
      zp = 0;
    }
  } else {
    // absmax: zp, unused by the scheme, carries the exponent by which the
    // values are scaled first (64 for an absmax below 2^-100, where 127 /
    // amax would overflow: the same prescaling as the forward's quantisers)
    const float amax = fmaxf(fabsf(lo), fabsf(hi));
    scale = amax;
    mul = row_factor(amax);
    zp = tiny_absmax(amax) ? 64 : 0;
  }
}

// One code; mul = 0 marks an all-zero vector (code 0).  PRE = false: the
// caller knows the absmax prescale exponent zp is 0.
template <int ZP, bool PRE = true>
__device__ __forceinline__ int code_of(float x, float mul, int zp) {
  if (mul == 0.0f) return 0;
  const int q = ZP ? (int)roundf(x * mul) + zp : (int)roundf((PRE ? __builtin_ldexpf(x, zp) : x) * mul);
  return q < -127 ? -127 : (q > 127 ? 127 : q);
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) | ((uint32_t)(d & 0xFF) << 24);
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fminf(v, __shfl_xor(v, off, WAVE));
  return v;
}

// ------------------------------------------------------------ row-wise ----
// Block = 4 waves, wave = one row.  VEC: C % 8 == 0, 16-byte chunks.
template <int DT, int ZP, int VEC>
__global__ __launch_bounds__(256) void vw_rows_kernel(const uint16_t* __restrict__ X, int64_t R, int64_t C,
                                                      int8_t* __restrict__ codes, float* __restrict__ scale,
                                                      int32_t* __restrict__ zpo) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const uint16_t* row = X + r * C;
  float lo = 0.0f, hi = 0.0f;  // 0 is inside either scheme's range already
  if constexpr (VEC) {
    // four chunks' loads in flight together; chunks past the row load as 0.0
    const int64_t nch = C >> 3;
    for (int64_t c0 = lane; c0 < nch; c0 += 4 * 64) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t c = c0 + 64 * u;
        v[u] = c < nch ? *reinterpret_cast<const u32x4*>(row + 8 * c) : (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = to_f32<DT>(half_bits(v[u], e));
          lo = fminf(lo, x);
          hi = fmaxf(hi, x);
        }
    }
  } else {
    for (int64_t c = lane; c < C; c += 64) {
      const float x = to_f32<DT>(row[c]);
      lo = fminf(lo, x);
      hi = fmaxf(hi, x);
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  float sc, mul;
  int zp;
  finish_stats<ZP>(lo, hi, sc, zp, mul);
  if (lane == 0) {
    scale[r] = sc;
    if (ZP) zpo[r] = zp;
  }
  int8_t* crow = codes + r * C;
  auto put = [&](auto PREc) {
    constexpr bool PRE = decltype(PREc)::value;
    if constexpr (VEC) {
      const int64_t nch = C >> 3;
      for (int64_t c = lane; c < nch; c += 64) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * c);
        int q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = code_of<ZP, PRE>(to_f32<DT>(half_bits(v, e)), mul, zp);
        *reinterpret_cast<u32x2*>(crow + 8 * c) = (u32x2){pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7])};
      }
    } else {
      for (int64_t c = lane; c < C; c += 64) crow[c] = (int8_t)code_of<ZP, PRE>(to_f32<DT>(row[c]), mul, zp);
    }
  };
  // (absmax: the prescale only for a row with a tiny absmax; uniform per row)
  if (!ZP && zp != 0) put(std::true_type());
  else put(std::false_type());
}

// Zero-point statistics on raw 16-bit values: a key that orders fp16 and
// bf16 bit patterns like the values they encode (a negative value has every
// bit flipped, a positive one its sign bit set), two keys per dword.
__device__ __forceinline__ uint32_t order_keys16(uint32_t w) {
  const uint32_t neg = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, w) >> 15);  // 0xFFFF where negative
  return w ^ (neg | 0x80008000u);
}
__device__ __forceinline__ uint32_t key_bits16(uint32_t k) {  // inverse of one key
  return (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

// Two zero-point codes clamp(round_half_away(fl32(x * nd)) + zp, +-127) as
// int16 halves of one dword.  The magnitude is floor(|v| + 0.5) for
// v = fl32(x * nd), |v| <= 254, by one conversion; mantissa bit 0 of |v| is
// cleared first, after which the result is the same whether or not the
// conversion rounds |v| + 0.5 to fp32 (no tie k + 0.5 below 2^22 has that
// bit set, and the rounded sum is then exact).  zp2: the zero point in both
// halves.
template <int DT>
__device__ __forceinline__ uint32_t zp_code_pair16(uint32_t x, float nd, uint32_t zp2) {
  const int mlo = cvt_rpi(__uint_as_float(__float_as_uint(scaled_abs<DT>(x & 0xFFFFu, nd)) & ~1u));
  const int mhi = cvt_rpi(__uint_as_float(__float_as_uint(scaled_abs<DT>(x >> 16, nd)) & ~1u));
  const i16x2 mag = __builtin_bit_cast(i16x2, __builtin_amdgcn_perm((uint32_t)mhi, (uint32_t)mlo, 0x05040100u));
  const i16x2 neg = __builtin_bit_cast(i16x2, x) >> 15;  // -1 where x < 0
  const i16x2 q = ((mag ^ neg) - neg) + __builtin_bit_cast(i16x2, zp2);
  const i16x2 lim = {127, 127};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_elementwise_min(q, lim), -lim));
}

// Zero-point, rows of at most 512 * MAXC values (C % 8 == 0): the row is held
// in registers (MAXC 16-byte chunks per lane), so it is read from memory once
// and every code store comes after the only wait.  (The two-pass kernel above
// reloads a chunk after each store, and loads and stores share one
// completion counter, so each reload also waits for the previous store:
// 4096 x 4096 fp16 15.9 -> 14.5 us per kernel.)  The row's minimum and
// maximum are taken on ordering keys, both in one packed wave reduction, and
// the codes two at a time with packed 16-bit arithmetic.  Chunks past the row
// end re-read chunk 0, which changes no minimum or maximum, and store nothing.
template <int DT, int MAXC>
__global__ __launch_bounds__(256) void vw_rows_zp_kernel(const uint16_t* __restrict__ X, int64_t R, int64_t C,
                                                         int8_t* __restrict__ codes, float* __restrict__ scale,
                                                         int32_t* __restrict__ zpo) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const int64_t nch = C >> 3;
  const u32x4* rp = reinterpret_cast<const u32x4*>(X + r * C);
  u32x4 v[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int64_t c = lane + (int64_t)i * 64;
    v[i] = rp[c < nch ? c : 0];
  }
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < MAXC; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t k = order_keys16(v[i][d]);
      kmin = pk_min_u16(kmin, k);
      kmax = pk_max_u16(kmax, k);
    }
  // the largest key in the high half, the complement of the smallest in the
  // low half: one packed maximum over the wave reduces both
  uint32_t mm = (max(kmax & 0xFFFFu, kmax >> 16) << 16) | (0xFFFFu - min(kmin & 0xFFFFu, kmin >> 16));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mm = pk_max_u16(mm, (uint32_t)__shfl_xor((int)mm, off, WAVE));
  const float lo = to_f32<DT>(key_bits16(0xFFFFu - (mm & 0xFFFFu)));
  const float hi = to_f32<DT>(key_bits16(mm >> 16));
  float sc, mul;
  int zp;
  finish_stats<1>(lo, hi, sc, zp, mul);  // widens [lo, hi] to contain 0
  if (lane == 0) {
    scale[r] = sc;
    zpo[r] = zp;
  }
  const uint32_t zp2 = ((uint32_t)zp & 0xFFFFu) | ((uint32_t)zp << 16);
  // the 16-bit row, not fp32 conversions of it, stays live into the code pass
#pragma unroll
  for (int i = 0; i < MAXC; ++i) asm volatile("" : "+v"(v[i]));
  u32x2* cp = reinterpret_cast<u32x2*>(codes + r * C);
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int64_t c = lane + (int64_t)i * 64;
    u32x2 pk;
    pk[0] = pack_codes16(zp_code_pair16<DT>(v[i][0], mul, zp2), zp_code_pair16<DT>(v[i][1], mul, zp2));
    pk[1] = pack_codes16(zp_code_pair16<DT>(v[i][2], mul, zp2), zp_code_pair16<DT>(v[i][3], mul, zp2));
    if (c < nch) cp[c] = pk;
  }
}

// --------------------------------------------------------- column-wise ----
// Block = 512 threads on an SW-column strip (SW = 32 or 64): PPR = SW / 8
// threads per row, each with 8 columns, rows grp, grp + GROUPS, ... where
// grp = thread / PPR.  Statistics are combined per column with shuffles
// inside each wave, then over the 8 waves in LDS, in a fixed order.
constexpr int VWC_THREADS = 512;

__device__ __forceinline__ float wave_min_stride(float v, int from) {
  for (int off = 32; off >= from; off >>= 1) v = fminf(v, __shfl_xor(v, off, WAVE));
  return v;
}
__device__ __forceinline__ float wave_max_stride(float v, int from) {
  for (int off = 32; off >= from; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, WAVE));
  return v;
}

template <int DT, int ZP, int VEC, int SW, int UR = 4>
__global__ __launch_bounds__(VWC_THREADS) void vw_cols_kernel(const uint16_t* __restrict__ X, int64_t R, int64_t C,
                                                              int8_t* __restrict__ codes, float* __restrict__ scale,
                                                              int32_t* __restrict__ zpo) {
  constexpr int PPR = SW / 8, GROUPS = VWC_THREADS / PPR, NWV = VWC_THREADS / 64;
  static_assert(SW % 8 == 0 && 64 % PPR == 0, "strip width");
  __shared__ float s_lo[NWV][SW];
  __shared__ float s_hi[NWV][SW];
  __shared__ float s_mul[SW];
  __shared__ int s_zp[SW];
  const int t = threadIdx.x, part = t % PPR, grp = t / PPR, lane = t & 63, wv = t >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * SW + 8 * part;  // this thread's first column
  float lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) lo[e] = hi[e] = 0.0f;
  const bool whole = VEC && c0 + 8 <= C;
  // UR: rows whose loads are in flight together
  if (whole) {
    // rows past R load as 0.0, which lies inside every range already
    for (int64_t r0 = grp; r0 < R; r0 += UR * GROUPS) {
      u32x4 v[UR];
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const int64_t r = r0 + (int64_t)u * GROUPS;
        v[u] = r < R ? *reinterpret_cast<const u32x4*>(X + r * C + c0) : (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < UR; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = to_f32<DT>(half_bits(v[u], e));
          lo[e] = fminf(lo[e], x);
          hi[e] = fmaxf(hi[e], x);
        }
    }
  } else {
    for (int64_t r = grp; r < R; r += GROUPS) {
      const uint16_t* p = X + r * C + c0;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c0 + e < C) {
          const float x = to_f32<DT>(p[e]);
          lo[e] = fminf(lo[e], x);
          hi[e] = fmaxf(hi[e], x);
        }
    }
  }
  // lanes part, part + PPR, ... of a wave hold the same columns
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] = wave_min_stride(lo[e], PPR);
    hi[e] = wave_max_stride(hi[e], PPR);
  }
  if (lane < PPR) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s_lo[wv][8 * lane + e] = lo[e];
      s_hi[wv][8 * lane + e] = hi[e];
    }
  }
  __syncthreads();
  if (t < SW) {
    float l = 0.0f, h = 0.0f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      l = fminf(l, s_lo[w][t]);
      h = fmaxf(h, s_hi[w][t]);
    }
    float sc, mul;
    int zp;
    finish_stats<ZP>(l, h, sc, zp, mul);
    s_mul[t] = mul;
    s_zp[t] = zp;
    const int64_t col = (int64_t)blockIdx.x * SW + t;
    if (col < C) {
      scale[col] = sc;
      if (ZP) zpo[col] = zp;
    }
  }
  __syncthreads();
  float mul[8];
  int zp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mul[e] = s_mul[8 * part + e];
    zp[e] = s_zp[8 * part + e];
  }
  if (whole) {
    for (int64_t r0 = grp; r0 < R; r0 += UR * GROUPS) {
      u32x4 v[UR];
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const int64_t r = r0 + (int64_t)u * GROUPS;
        v[u] = r < R ? *reinterpret_cast<const u32x4*>(X + r * C + c0) : (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const int64_t r = r0 + (int64_t)u * GROUPS;
        int k[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) k[e] = code_of<ZP>(to_f32<DT>(half_bits(v[u], e)), mul[e], zp[e]);
        if (r < R)
          *reinterpret_cast<u32x2*>(codes + r * C + c0) =
              (u32x2){pack4(k[0], k[1], k[2], k[3]), pack4(k[4], k[5], k[6], k[7])};
      }
    }
  } else {
    for (int64_t r = grp; r < R; r += GROUPS) {
      const uint16_t* p = X + r * C + c0;
      int8_t* q = codes + r * C + c0;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c0 + e < C) q[e] = (int8_t)code_of<ZP>(to_f32<DT>(p[e]), mul[e], zp[e]);
    }
  }
}

// Columns of at most GROUPS * RPT rows (C % 8 == 0): each thread holds its
// RPT rows of the strip in registers, so the strip is read from memory once,
// with RPT loads in flight per thread, and every code store comes after the
// only wait (the two-pass kernel above reloads rows after storing codes, and
// each reload waits for the stores before it; 4096 x 4096 fp16, absmax,
// 37.2 -> 34.7 us per kernel: half the compute units hold a strip, so the
// strip count, not the waits, bounds it).  A thread whose 8 columns lie
// past C (C % 8 == 0: all of them or none) reads row data of columns 0-7 and
// stores nothing; rows past R re-read row R - 1, which changes no minimum or
// maximum, and store nothing.  Requires R >= 1.
template <int DT, int ZP, int SW, int RPT>
__global__ __launch_bounds__(VWC_THREADS) void vw_cols_reg_kernel(const uint16_t* __restrict__ X, int64_t R,
                                                                  int64_t C, int8_t* __restrict__ codes,
                                                                  float* __restrict__ scale, int32_t* __restrict__ zpo) {
  constexpr int PPR = SW / 8, GROUPS = VWC_THREADS / PPR, NWV = VWC_THREADS / 64;
  static_assert(SW % 8 == 0 && 64 % PPR == 0, "strip width");
  __shared__ float s_lo[NWV][SW];
  __shared__ float s_hi[NWV][SW];
  __shared__ float s_mul[SW];
  __shared__ int s_zp[SW];
  const int t = threadIdx.x, part = t % PPR, grp = t / PPR, lane = t & 63, wv = t >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * SW + 8 * part;  // this thread's first column
  const bool live = c0 < C;
  const uint16_t* base = X + (live ? c0 : 0);
  u32x4 v[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int64_t r = grp + (int64_t)u * GROUPS;
    v[u] = *reinterpret_cast<const u32x4*>(base + (r < R ? r : R - 1) * C);
  }
  float lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) lo[e] = hi[e] = 0.0f;
#pragma unroll
  for (int u = 0; u < RPT; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = to_f32<DT>(half_bits(v[u], e));
      lo[e] = fminf(lo[e], x);
      hi[e] = fmaxf(hi[e], x);
    }
  // lanes part, part + PPR, ... of a wave hold the same columns
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] = wave_min_stride(lo[e], PPR);
    hi[e] = wave_max_stride(hi[e], PPR);
  }
  if (lane < PPR) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s_lo[wv][8 * lane + e] = lo[e];
      s_hi[wv][8 * lane + e] = hi[e];
    }
  }
  __syncthreads();
  if (t < SW) {
    float l = 0.0f, h = 0.0f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      l = fminf(l, s_lo[w][t]);
      h = fmaxf(h, s_hi[w][t]);
    }
    float sc, mul;
    int zp;
    finish_stats<ZP>(l, h, sc, zp, mul);
    s_mul[t] = mul;
    s_zp[t] = zp;
    const int64_t col = (int64_t)blockIdx.x * SW + t;
    if (col < C) {
      scale[col] = sc;
      if (ZP) zpo[col] = zp;
    }
  }
  __syncthreads();
  float mul[8];
  int zp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mul[e] = s_mul[8 * part + e];
    zp[e] = s_zp[8 * part + e];
  }
  // the 16-bit rows, not their fp32 conversions, are what stays live across
  // the barriers (kept as converted values they would take twice the registers)
#pragma unroll
  for (int u = 0; u < RPT; ++u) asm volatile("" : "+v"(v[u]));
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int64_t r = grp + (int64_t)u * GROUPS;
    int k[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) k[e] = code_of<ZP>(to_f32<DT>(half_bits(v[u], e)), mul[e], zp[e]);
    if (live && r < R)
      *reinterpret_cast<u32x2*>(codes + r * C + c0) = (u32x2){pack4(k[0], k[1], k[2], k[3]), pack4(k[4], k[5], k[6], k[7])};
  }
}

// Column-wise launch for one strip width: the register kernel when the rows
// fit (RPT 8, 16 or 32 rows per thread), else the two-pass kernel.
template <int DT, int ZP, int SW>
hipError_t launch_vw_cols(const uint16_t* X, int64_t R, int64_t C, bool vec, int8_t* codes, float* scale,
                          int32_t* zp, hipStream_t s) {
  constexpr int GROUPS = VWC_THREADS / (SW / 8);
  const dim3 grid((unsigned)((C + SW - 1) / SW));
  // the register kernel reads row R - 1 (and columns 0-7) unconditionally:
  // R >= 1, and C >= 8 (the caller launches nothing for C <= 0)
  if (vec && R >= 1 && R <= (int64_t)GROUPS * 8)
    vw_cols_reg_kernel<DT, ZP, SW, 8><<<grid, VWC_THREADS, 0, s>>>(X, R, C, codes, scale, zp);
  else if (vec && R >= 1 && R <= (int64_t)GROUPS * 16)
    vw_cols_reg_kernel<DT, ZP, SW, 16><<<grid, VWC_THREADS, 0, s>>>(X, R, C, codes, scale, zp);
  else if (vec && R >= 1 && R <= (int64_t)GROUPS * 32)
    vw_cols_reg_kernel<DT, ZP, SW, 32><<<grid, VWC_THREADS, 0, s>>>(X, R, C, codes, scale, zp);
  else if (vec)
    vw_cols_kernel<DT, ZP, 1, SW><<<grid, VWC_THREADS, 0, s>>>(X, R, C, codes, scale, zp);
  else
    vw_cols_kernel<DT, ZP, 0, SW><<<grid, VWC_THREADS, 0, s>>>(X, R, C, codes, scale, zp);
  return hipGetLastError();
}

template <int DT, int ZP>
hipError_t launch_vw_t(const uint16_t* X, int64_t R, int64_t C, int axis, int8_t* codes, float* scale,
                       int32_t* zp, hipStream_t s) {
  const bool vec = (C % 8) == 0;
  if (axis == 0) {  // one vector per row
    if (R <= 0) return hipSuccess;
    const dim3 grid((unsigned)((R + 3) / 4));
    // zero-point rows held in registers (absmax per row runs the weight
    // quantiser, above); the kernel reads chunk 0 of every row
    // unconditionally: C >= 8
    if constexpr (ZP) {
      const bool reg = vec && C > 0;
      if (reg && C <= 512 * 2) {
        vw_rows_zp_kernel<DT, 2><<<grid, 256, 0, s>>>(X, R, C, codes, scale, zp);
        return hipGetLastError();
      }
      if (reg && C <= 512 * 8) {
        vw_rows_zp_kernel<DT, 8><<<grid, 256, 0, s>>>(X, R, C, codes, scale, zp);
        return hipGetLastError();
      }
      if (reg && C <= 512 * 24) {
        vw_rows_zp_kernel<DT, 24><<<grid, 256, 0, s>>>(X, R, C, codes, scale, zp);
        return hipGetLastError();
      }
    }
    if (vec)
      vw_rows_kernel<DT, ZP, 1><<<grid, 256, 0, s>>>(X, R, C, codes, scale, zp);
    else
      vw_rows_kernel<DT, ZP, 0><<<grid, 256, 0, s>>>(X, R, C, codes, scale, zp);
  } else {          // one vector per column: 64-column strips (whole 128-byte
                    // lines) when there are enough of them to fill the chip,
                    // else 32-column strips (measured best of 8/16/32/64 at
                    // C = 4096: fewer, fuller lines beat more workgroups)
    if (C <= 0) return hipSuccess;
    return C >= 64 * 256 ? launch_vw_cols<DT, ZP, 64>(X, R, C, vec, codes, scale, zp, s)
                         : launch_vw_cols<DT, ZP, 32>(X, R, C, vec, codes, scale, zp, s);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_vectorwise(int dt, const void* X, int64_t R, int64_t C, int zeropoint, int axis,
                                   int8_t* codes, float* scale, int32_t* zp, hipStream_t s) {
  // Absmax per row is exactly what the forward's weight quantiser computes
  // (the same codes, the absmax as the scale, the same tiny-absmax prescale),
  // and its kernel takes the row maximum on packed 16-bit magnitudes: 4096 x
  // 4096 fp16 in about 10.5 against 14.3 us.  (C = 0, all-zero rows' scales
  // only, stays below.)
  if (!zeropoint && axis == 0 && R > 0 && C > 0) return launch_quant_weight(dt, X, R, C, codes, scale, s);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (dt == DT_F16)
    return zeropoint ? launch_vw_t<DT_F16, 1>(x, R, C, axis, codes, scale, zp, s)
                     : launch_vw_t<DT_F16, 0>(x, R, C, axis, codes, scale, zp, s);
  return zeropoint ? launch_vw_t<DT_BF16, 1>(x, R, C, axis, codes, scale, zp, s)
                   : launch_vw_t<DT_BF16, 0>(x, R, C, axis, codes, scale, zp, s);
}

}  // namespace lli8
