// Vector-wise quantisation of a 16-bit matrix on its own: absmax or
// zero-point, one scale per row or per column ("Hugging Face integrates
// LLM.int8() ...", section "Quantization mechanics": both schemes, either
// way).  Not a step of the forward; the forward's own quantisers live in
// lli8_quant.hip and lli8_decode.hip.
//
//   absmax:     code = clamp(round_half_away(fl32(x * fl32(127 / amax))), +-127),
//               scale = amax (0 for an all-zero vector, codes 0)
//   zero-point: lo = min(min x, 0), hi = max(max x, 0), nd = fl32(254 / fl32(hi - lo)),
//               zp = round_half_away(fl32(-lo * nd)) - 127,
//               code = clamp(round_half_away(fl32(x * nd)) + zp, +-127),
//               scale = nd, zero point = zp (0 and 0 for an all-zero vector)
//
// Both are HBM-bound codecs: read X once from memory, write the codes once.
// Row-wise: one wave per row, a statistics pass, then a code pass over the
// same row (in cache by then).  Column-wise: one workgroup per 32- or
// 64-column strip walking every row twice (statistics, then codes), 8
// columns per thread; one launch, no atomics, no scratch.
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
    const float amax = fmaxf(fabsf(lo), fabsf(hi));
    scale = amax;
    mul = amax > 0.0f ? 127.0f / amax : 0.0f;
    zp = 0;
  }
}

// One code; mul = 0 marks an all-zero vector (code 0).
template <int ZP>
__device__ __forceinline__ int code_of(float x, float mul, int zp) {
  if (mul == 0.0f) return 0;
  const int q = (int)roundf(x * mul) + (ZP ? zp : 0);
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
  if constexpr (VEC) {
    const int64_t nch = C >> 3;
    for (int64_t c = lane; c < nch; c += 64) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * c);
      int q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = code_of<ZP>(to_f32<DT>(half_bits(v, e)), mul, zp);
      *reinterpret_cast<u32x2*>(crow + 8 * c) = (u32x2){pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7])};
    }
  } else {
    for (int64_t c = lane; c < C; c += 64) crow[c] = (int8_t)code_of<ZP>(to_f32<DT>(row[c]), mul, zp);
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

template <int DT, int ZP>
hipError_t launch_vw_t(const uint16_t* X, int64_t R, int64_t C, int axis, int8_t* codes, float* scale,
                       int32_t* zp, hipStream_t s) {
  const bool vec = (C % 8) == 0;
  if (axis == 0) {  // one vector per row
    if (R <= 0) return hipSuccess;
    const dim3 grid((unsigned)((R + 3) / 4));
    if (vec)
      vw_rows_kernel<DT, ZP, 1><<<grid, 256, 0, s>>>(X, R, C, codes, scale, zp);
    else
      vw_rows_kernel<DT, ZP, 0><<<grid, 256, 0, s>>>(X, R, C, codes, scale, zp);
  } else {          // one vector per column: 64-column strips (whole 128-byte
                    // lines) when there are enough of them to fill the chip,
                    // else 32-column strips (measured best of 8/16/32/64 at
                    // C = 4096: fewer, fuller lines beat more workgroups)
    if (C <= 0) return hipSuccess;
    if (C >= 64 * 256) {
      const dim3 grid((unsigned)((C + 63) / 64));
      if (vec)
        vw_cols_kernel<DT, ZP, 1, 64><<<grid, VWC_THREADS, 0, s>>>(X, R, C, codes, scale, zp);
      else
        vw_cols_kernel<DT, ZP, 0, 64><<<grid, VWC_THREADS, 0, s>>>(X, R, C, codes, scale, zp);
    } else {
      const dim3 grid((unsigned)((C + 31) / 32));
      if (vec)
        vw_cols_kernel<DT, ZP, 1, 32><<<grid, VWC_THREADS, 0, s>>>(X, R, C, codes, scale, zp);
      else
        vw_cols_kernel<DT, ZP, 0, 32><<<grid, VWC_THREADS, 0, s>>>(X, R, C, codes, scale, zp);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_vectorwise(int dt, const void* X, int64_t R, int64_t C, int zeropoint, int axis,
                                   int8_t* codes, float* scale, int32_t* zp, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (dt == DT_F16)
    return zeropoint ? launch_vw_t<DT_F16, 1>(x, R, C, axis, codes, scale, zp, s)
                     : launch_vw_t<DT_F16, 0>(x, R, C, axis, codes, scale, zp, s);
  return zeropoint ? launch_vw_t<DT_BF16, 1>(x, R, C, axis, codes, scale, zp, s)
                   : launch_vw_t<DT_BF16, 0>(x, R, C, axis, codes, scale, zp, s);
}

}  // namespace lli8
