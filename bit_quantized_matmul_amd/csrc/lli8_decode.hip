// Fused decode path (T <= 16, K <= 4096): the whole LLM.int8() forward in one
// launch, with no workgroup ever waiting on another.  Eight waves per
// workgroup (two per SIMD, so one wave's dependent arithmetic overlaps the
// other's), each owning two 256-column slices of K.
//
// For a handful of tokens the int8 weight stream (N x K bytes) is the only
// real HBM traffic; separate launches for the outlier scan, the activation
// quantiser and the GEMM each cost more than the stream itself, and so does a
// grid-wide barrier.  So every workgroup derives the activation split on its
// own (X is at most 16 x 4096 values and sits in L2 after the first touch):
//   1. load X in the MFMA operand layout (lane = token row t);
//   2. statistics with packed 16-bit integer max over |x| bit patterns: a
//      column is an outlier when some |x| > threshold ("Core idea of
//      LLM.int8()" step 1); the row absmax over the other columns is SCA
//      ("Quantization mechanics", absmax bullet); then the loads of its 16
//      weight rows (all of K) are issued, so the weight stream overlaps the
//      rest and the X loads never queue behind it;
//   3. codes round(fl32(|x| * fl32(127 / SCA))) with halves away from zero,
//      signed, 0 on outlier columns, written straight into the MFMA A
//      operands;
//   4. v_mfma_i32_16x16x64_i8 over K, the eight waves' int32 tiles summed in
//      a fixed order, then the epilogue: dequantisation, the 16-bit outlier
//      product against (CB * SCB) / 127 ("Integration into transformers"),
//      bias, one rounding.
// Workgroup 0 also writes the side outputs (CA, SCA, bitmap, idx, n_idx).
#include "lli8_device.h"
#include "lli8_internal.h"

namespace lli8 {

constexpr int FD_NW = 8;                      // waves per workgroup: two per SIMD
constexpr int FD_THREADS = FD_NW * 64;
constexpr int FD_SS = 2;                      // 256-column K slices per wave
constexpr int FD_MAXK = FD_NW * FD_SS * 256;  // 4096
constexpr int FD_MAXW = FD_MAXK / 32;
constexpr int FD_OUT_LDS = 64;           // outlier columns staged in LDS; more fall back to global reads

// Codes of the two 16-bit values of x for row factor s = fl32(127 / absmax),
// as two int16 in one dword.  |x| * s <= 127.5, and for such v,
// round-half-away(v) == floor(fl32(v' + 0.5)) with v' = v with mantissa bit 0
// cleared (v' + 0.5 is exact, and clearing bit 0 never moves v across a
// half-integer); v_cvt_rpi_i32_f32 computes floor(v' + 0.5).  The sign of x
// is applied to both magnitudes at once with packed 16-bit arithmetic.
typedef short i16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int cvt_rpi(float v) {
  int r;
  asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

template <int DT>
__device__ __forceinline__ uint32_t code_pair16(uint32_t x, float s) {
  const float vlo = fabsf(to_f32<DT>(x & 0xFFFFu)) * s;
  const float vhi = fabsf(to_f32<DT>(x >> 16)) * s;
  const int mlo = cvt_rpi(__uint_as_float(__float_as_uint(vlo) & 0xFFFFFFFEu));
  const int mhi = cvt_rpi(__uint_as_float(__float_as_uint(vhi) & 0xFFFFFFFEu));
  const i16x2 mag = __builtin_bit_cast(i16x2, (uint32_t)mlo | ((uint32_t)mhi << 16));
  const i16x2 neg = __builtin_bit_cast(i16x2, x) >> 15;  // -1 where x < 0
  return __builtin_bit_cast(uint32_t, (i16x2)((mag ^ neg) - neg));
}

// Low bytes of the four int16 codes in two dwords, packed little-endian.
__device__ __forceinline__ uint32_t pack_codes16(uint32_t p01, uint32_t p23) {
  return __builtin_amdgcn_perm(p23, p01, 0x06040200u);
}

// Column of the first value of 8-value chunk j (0..7) that lane group g (0..3)
// holds in 256-column slice s.  Chunks 2u and 2u+1 form MFMA operand u, which
// covers columns s*256 + 64u + 16g .. +16; the weight operand uses the same
// columns, so the int8 dot products are exact in any order.  The four lanes
// of a row then read one 128-byte line per load instruction.
__device__ __forceinline__ int col_of(int s, int j, int g) { return s * 256 + (j >> 1) * 64 + g * 16 + (j & 1) * 8; }

// 256-column slice behind register slot i of wave w.  Each workgroup starts
// at a different slice (rot), so the workgroups, which all read the same X,
// do not walk the same L2 channels in lockstep; the slot -> slice map stays a
// bijection, and activation and weight operands share it.
__device__ __forceinline__ int slice_of(int w, int i, int rot, int nss) {
  const int s = w + FD_NW * i;
  return s < nss ? (s + rot) % nss : s;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Larger of each 16-bit half (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

// Largest 15-bit magnitude of an 8-value chunk.
__device__ __forceinline__ uint32_t chunk_max(const u32x4& v) {
  const uint32_t m2 = pk_max_u16(pk_max_u16(v[0] & 0x7FFF7FFFu, v[1] & 0x7FFF7FFFu),
                                 pk_max_u16(v[2] & 0x7FFF7FFFu, v[3] & 0x7FFF7FFFu));
  return max(m2 & 0xFFFFu, m2 >> 16);
}

template <int DT>
__global__ __launch_bounds__(FD_THREADS, 1) void decode_fused_kernel(
    const uint16_t* __restrict__ X, int T, int K, int N, float tau, const int8_t* __restrict__ CB,
    const float* __restrict__ SCB, const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
    int8_t* __restrict__ CA, float* __restrict__ SCA, uint32_t* __restrict__ bitmap,
    int32_t* __restrict__ idx, int32_t* __restrict__ n_idx_out, int32_t* __restrict__ acc_out) {
  __shared__ uint32_t s_bm[FD_MAXW];
  __shared__ uint32_t s_pre[FD_MAXW];
  __shared__ int32_t s_idx[FD_MAXK];
  __shared__ uint32_t s_rmax[16];
  __shared__ int s_any;
  __shared__ v4i s_red[FD_NW - 1][64];
  __shared__ float s_ow[FD_OUT_LDS][16];  // recovered weights of the outlier columns, this block
  __shared__ float s_ox[FD_OUT_LDS][16];  // X values of the outlier columns

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nr = lane & 15, g = lane >> 4;
  const int G = gridDim.x, wg = blockIdx.x;
  const int nblk = (N + 15) >> 4;
  const int nss = (K + 255) >> 8;
  const int W = (K + 31) >> 5;
  const int rot = wg % nss;

  // |x| > tau  <=>  (bits & 0x7FFF) > t16, t16 = largest 16-bit magnitude <= tau
  const bool outl = tau > 0.0f && tau <= 3.4028235e38f;
  uint32_t t16 = 0xFFFFu;
  if (outl) {
    uint32_t bb = from_f32<DT>(tau);
    if (to_f32<DT>(bb) > tau) bb -= 1u;
    t16 = bb & 0x7FFFu;
  }

  for (int i = tid; i < W; i += FD_THREADS) s_bm[i] = 0u;
  if (tid < 16) s_rmax[tid] = 0u;
  if (tid == 0) s_any = 0;

  // 1. activations: row nr, chunk j of slot i at column col_of(slice, j, g).
  // Loads are unconditional, at clamped in-range addresses, so the compiler
  // counts them in order.  Validity is applied where values are used: chunks
  // beyond K count as zero; rows beyond T only feed accumulator rows the
  // epilogue never stores, and never flag a column.
  const bool row_ok = nr < T;
  u32x4 xr[FD_SS][8];
  bool kok[FD_SS][8];
  {
    const uint16_t* xrow = X + (int64_t)(row_ok ? nr : 0) * K;
#pragma unroll
    for (int i = 0; i < FD_SS; ++i) {
      const int s = slice_of(w, i, rot, nss);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = col_of(s, j, g);
        kok[i][j] = s < nss && k < K;
        xr[i][j] = *reinterpret_cast<const u32x4*>(xrow + (kok[i][j] ? k : 0));
      }
    }
  }
  const int blk0 = wg;  // the grid never exceeds the number of blocks
  float scb_pre = 0.0f, bias_pre = 0.0f;  // first block's scale and bias, epilogue lanes
  {
    const int64_t col = (int64_t)blk0 * 16 + (lane & 15);
    if (w == 0 && col < N) {
      scb_pre = SCB[col];
      bias_pre = (bias != nullptr) ? to_f32<DT>(bias[col]) : 0.0f;
    }
  }

  // 2. statistics: per-chunk (8 columns) maxima of the 15-bit magnitudes
  uint32_t cmax[FD_SS][8];
  uint32_t lmax = 0u;
  uint32_t hot = 0u;  // bit 8i+j: chunk (i, j) holds a value above the threshold
#pragma unroll
  for (int i = 0; i < FD_SS; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      cmax[i][j] = kok[i][j] ? chunk_max(xr[i][j]) : 0u;
      lmax = max(lmax, cmax[i][j]);
      hot |= (outl && row_ok && cmax[i][j] > t16) ? (1u << (8 * i + j)) : 0u;
    }

  // 3. weight rows of the first block, issued once X has been consumed so the
  //    activation loads never queue behind the weight stream
  u32x4 b[FD_SS][4];
  auto load_cb = [&](int blk) {  // rows beyond N give accumulator columns that are never stored
    const int64_t n = (int64_t)blk * 16 + nr;
    const int8_t* brow = CB + (n < N ? n : 0) * K;
#pragma unroll
    for (int i = 0; i < FD_SS; ++i) {
      const int s = slice_of(w, i, rot, nss);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = col_of(s, 2 * u, g);
        b[i][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(brow + ((s < nss && k < K) ? k : 0)));
      }
    }
  };
  __builtin_amdgcn_sched_barrier(0);
  load_cb(blk0);
  __builtin_amdgcn_sched_barrier(0);

  // 4. outlier columns: OR of the hot-chunk masks over the wave, then only
  //    the hot chunks are examined value by value
  uint32_t hw = hot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) hw |= (uint32_t)__shfl_xor((int)hw, off, WAVE);
  __syncthreads();  // LDS initialised
  if (lane == 0 && hw) s_any = 1;
  __syncthreads();
  const bool any = s_any != 0;
  bool mine = false;  // does this lane's column set hold an outlier column?
  if (any) {
#pragma unroll
    for (int i = 0; i < FD_SS; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((hw >> (8 * i + j)) & 1u) {  // wave-uniform
          uint32_t bits = 0u;
          if ((hot >> (8 * i + j)) & 1u) {
#pragma unroll
            for (int e = 0; e < 8; ++e) bits |= ((half_bits(xr[i][j], e) & 0x7FFFu) > t16 ? 1u : 0u) << e;
          }
          // the 16 lanes of a group hold the same columns for 16 rows
          bits |= __shfl_xor(bits, 1, WAVE);
          bits |= __shfl_xor(bits, 2, WAVE);
          bits |= __shfl_xor(bits, 4, WAVE);
          bits |= __shfl_xor(bits, 8, WAVE);
          const int col = col_of(slice_of(w, i, rot, nss), j, g);
          if (nr == 0 && bits) atomicOr(&s_bm[col >> 5], bits << (col & 31));
        }
    __syncthreads();
    uint32_t fl[FD_SS][4];  // flag bits of the 16 columns behind operand u
#pragma unroll
    for (int i = 0; i < FD_SS; ++i) {
      const int s = slice_of(w, i, rot, nss);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c0 = col_of(s, 2 * u, g);
        fl[i][u] = (s < nss && c0 < K) ? (s_bm[c0 >> 5] >> (c0 & 31)) & 0xFFFFu : 0u;
        mine |= fl[i][u] != 0u;
      }
    }
    if (mine) {  // row maximum without the outlier columns
      lmax = 0u;
#pragma unroll
      for (int i = 0; i < FD_SS; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t f8 = (fl[i][j >> 1] >> (8 * (j & 1))) & 0xFFu;
          uint32_t cm = cmax[i][j];
          if (f8 != 0u) {
            cm = 0u;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              cm = max(cm, ((f8 >> e) & 1u) ? 0u : (half_bits(xr[i][j], e) & 0x7FFFu));
          }
          lmax = max(lmax, cm);
        }
    }
  }
  lmax = max(lmax, (uint32_t)__shfl_xor((int)lmax, 16, WAVE));
  lmax = max(lmax, (uint32_t)__shfl_xor((int)lmax, 32, WAVE));
  if (g == 0) atomicMax(&s_rmax[nr], lmax);
  __syncthreads();
  const float sca = to_f32<DT>(s_rmax[nr]);  // exact row absmax over non-outlier columns
  const float sf = (sca > 0.0f) ? 127.0f / sca : 0.0f;

  // 5. codes, straight into the MFMA A operands: a[i][u] = columns col_of(slice, 2u, g) .. +16
  u32x4 a[FD_SS][4];
#pragma unroll
  for (int i = 0; i < FD_SS; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x4 r;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 v = xr[i][2 * u + h];
        r[2 * h] = pack_codes16(code_pair16<DT>(v[0], sf), code_pair16<DT>(v[1], sf));
        r[2 * h + 1] = pack_codes16(code_pair16<DT>(v[2], sf), code_pair16<DT>(v[3], sf));
      }
      const int c0 = col_of(slice_of(w, i, rot, nss), 2 * u, g);
      const uint32_t bits16 = (mine && c0 < K) ? (s_bm[c0 >> 5] >> (c0 & 31)) & 0xFFFFu : 0u;
      if (bits16) {  // zero the codes of outlier columns
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t nib = (bits16 >> (4 * d)) & 0xFu;
          const uint32_t mask = ((nib & 1u) * 0xFFu) | (((nib >> 1) & 1u) * 0xFF00u) |
                                (((nib >> 2) & 1u) * 0xFF0000u) | (((nib >> 3) & 1u) * 0xFF000000u);
          r[d] &= ~mask;
        }
      }
      a[i][u] = kok[i][2 * u] ? r : (u32x4){0u, 0u, 0u, 0u};  // zero codes beyond K
    }

  // side outputs, workgroup 0
  if (wg == 0) {
    if (row_ok) {
#pragma unroll
      for (int i = 0; i < FD_SS; ++i) {
        const int s = slice_of(w, i, rot, nss);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k = col_of(s, 2 * u, g);
          if (s < nss && k < K) *reinterpret_cast<u32x4*>(CA + (int64_t)nr * K + k) = a[i][u];
        }
      }
    }
    if (w == 0 && g == 0 && row_ok) SCA[nr] = sca;
    for (int i = tid; i < W; i += FD_THREADS) bitmap[i] = s_bm[i];
  }
  int n_out = 0;
  if (any) {
    if (tid < 64) {
      const int seg = (W + 63) / 64;
      const int w0 = lane * seg, w1 = min(W, w0 + seg);
      int cnt = 0;
      for (int i = w0; i < w1; ++i) cnt += __popc(s_bm[i]);
      int run = wave_incl_scan(cnt) - cnt;
      for (int i = w0; i < w1; ++i) {
        s_pre[i] = (uint32_t)run;
        run += __popc(s_bm[i]);
      }
    }
    __syncthreads();
    n_out = (int)(s_pre[W - 1] + __popc(s_bm[W - 1]));
    for (int i = tid; i < W; i += FD_THREADS) {
      uint32_t m = s_bm[i];
      int pos = (int)s_pre[i];
      while (m) {
        const int bit = __builtin_ctz(m);
        s_idx[pos] = i * 32 + bit;
        if (wg == 0) idx[pos] = i * 32 + bit;
        ++pos;
        m &= m - 1u;
      }
    }
    __syncthreads();
  }
  if (wg == 0 && tid == 0) *n_idx_out = n_out;

  // X values of the outlier columns (the same for every block)
  const int n_lds = min(n_out, FD_OUT_LDS);
  for (int q = tid; q < n_lds * 16; q += FD_THREADS) {
    const int p = q >> 4, t = q & 15;
    s_ox[p][t] = (t < T) ? to_f32<DT>(X[(int64_t)t * K + s_idx[p]]) : 0.0f;
  }

  // 6. int8 products and epilogue, 16 output features at a time
  for (int blk = blk0; blk < nblk; blk += G) {
    if (blk != blk0) load_cb(blk);
    // recovered weights dtype(fl32(fl32(CB * SCB) / 127)) of the outlier columns, all loads in parallel
    for (int q = tid; q < n_lds * 16; q += FD_THREADS) {
      const int p = q >> 4;
      const int64_t col = (int64_t)blk * 16 + (q & 15);
      float wv = 0.0f;
      if (col < N) wv = to_f32<DT>(from_f32<DT>(((float)CB[col * K + s_idx[p]] * SCB[col]) / 127.0f));
      s_ow[p][q & 15] = wv;
    }
    v4i acc = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < FD_SS; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, a[i][u]), __builtin_bit_cast(v4i, b[i][u]),
                                                    acc, 0, 0, 0);
    if (w > 0) s_red[w - 1][lane] = acc;
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int q = 0; q < FD_NW - 1; ++q) acc += s_red[q][lane];  // fixed order: deterministic
      // 16x16 layout: lane holds feature lane % 16, tokens 4 * (lane / 16) + r
      const int64_t col = (int64_t)blk * 16 + (lane & 15);
      if (col < N) {
        const float scb = (blk == blk0) ? scb_pre : SCB[col];
        const float bv = (blk == blk0) ? bias_pre : ((bias != nullptr) ? to_f32<DT>(bias[col]) : 0.0f);
        float o[4] = {0.f, 0.f, 0.f, 0.f};
        for (int p = 0; p < n_lds; ++p) {
          const float wv = s_ow[p][lane & 15];
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] += s_ox[p][4 * (lane >> 4) + r] * wv;
        }
        for (int p = n_lds; p < n_out; ++p) {  // beyond the LDS stage: straight from memory
          const int c = s_idx[p];
          const float wv = to_f32<DT>(from_f32<DT>(((float)CB[col * K + c] * scb) / 127.0f));
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 4 * (lane >> 4) + r;
            if (t < T) o[r] += to_f32<DT>(X[(int64_t)t * K + c]) * wv;
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * (lane >> 4) + r;
          if (t >= T) continue;
          if (acc_out != nullptr) acc_out[(int64_t)t * N + col] = acc[r];
          const float sa = to_f32<DT>(s_rmax[t]);
          const float d = (float)acc[r] * (sa * (scb * (1.0f / 16129.0f)));
          out[(int64_t)t * N + col] = from_f32<DT>(d + o[r] + bv);
        }
      }
    }
    __syncthreads();
  }
}

bool decode_fused_supported(int64_t T, int64_t K) { return T >= 1 && T <= 16 && (K % 16) == 0 && K <= FD_MAXK; }

namespace {
int g_cus[64];  // compute units per device, looked up once
}

template <int DT>
static hipError_t launch_fused_t(const FusedArgs& a, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int& cus = g_cus[dev & 63];
  if (cus <= 0) {
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  const int nblk = (int)((a.N + 15) / 16);
  const int G = nblk < cus ? nblk : cus;  // one workgroup per CU; each walks blocks G apart
  decode_fused_kernel<DT><<<dim3(G), dim3(FD_THREADS), 0, s>>>(
      static_cast<const uint16_t*>(a.X), (int)a.T, (int)a.K, (int)a.N, a.tau, a.CB, a.SCB,
      static_cast<const uint16_t*>(a.bias), static_cast<uint16_t*>(a.out), a.CA, a.SCA, a.bitmap, a.idx, a.n_idx,
      a.acc);
  return hipGetLastError();
}

hipError_t launch_decode_fused(const FusedArgs& a, hipStream_t s) {
  return a.dt == DT_F16 ? launch_fused_t<DT_F16>(a, s) : launch_fused_t<DT_BF16>(a, s);
}

}  // namespace lli8
