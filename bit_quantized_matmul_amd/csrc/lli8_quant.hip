// Quantisation kernels of the LLM.int8() linear on gfx950:
//   * outlier-column scan of the activation (bitmap built with atomic OR),
//   * row-wise absmax quantisation of the activation with the outlier columns
//     left out (codes, scales, ascending outlier index list, gathered outlier
//     columns for the 16-bit product),
//   * row-wise absmax quantisation of the weight.
// The method: "Hugging Face integrates LLM.int8() ...", sections "Core idea of
// LLM.int8()" (steps 1-2) and "Quantization mechanics" (absmax bullet).
// All three are HBM-bound streaming kernels: one wave owns a contiguous
// stretch of a row and reads it with 16-byte loads.
#include <algorithm>
#include <type_traits>

#include "lli8_device.h"
#include "lli8_internal.h"

namespace lli8 {

// ---------------------------------------------------------------- fill ----
__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  fill_u32_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p, n, v);
  return hipGetLastError();
}

// --------------------------------------------------------- outlier scan ----
// Column c is an outlier when some row has |X[t, c]| > tau.  A lane owns one
// 16-byte chunk (8 columns) and walks rows keeping packed 16-bit maxima of
// the 15-bit magnitudes (one max per two values per row); the threshold test
// is done once at the end on the raw bits.  Four lanes make one bitmap word.
// K % 8 == 0: the strip kernels below; any K: one thread per column.

// Any K: one thread per column, 64 columns per wave form two bitmap words.
template <int DT>
__global__ __launch_bounds__(256) void scan_outliers_any_kernel(
    const uint16_t* __restrict__ X, int64_t T, int64_t K, float tau,
    uint32_t* __restrict__ bitmap, int rows_per_block) {
  const int lane = threadIdx.x & 63;
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(T, r0 + rows_per_block);
  bool flag = false;
  if (col < K)
    for (int64_t r = r0; r < r1; ++r) flag |= fabsf(to_f32<DT>(X[r * K + col])) > tau;
  const uint64_t m = __ballot(flag);
  const int64_t col0 = col - lane;  // multiple of 64
  if (lane == 0) {
    const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
    if (lo) atomicOr(bitmap + (col0 >> 5), lo);
    if (hi) atomicOr(bitmap + (col0 >> 5) + 1, hi);
  }
}

// Few rows (T <= SCAN_FULL_MAX_T, K % 8 == 0): one 1024-thread workgroup per
// 512-column strip reads every row of it, 16 waves splitting the rows, so
// each bitmap word is final when written (no atomics, no cleared bitmap
// needed, one launch fewer: 0.7-0.9 us per call at T = 17-128, K = N = 4096;
// at T = 256 the strips' reads take longer than the launch they save).
// Lane = 16-byte chunk as above; the waves' packed maxima are combined in
// LDS.
constexpr int64_t SCAN_FULL_MAX_T = 128;

template <int DT>
__global__ __launch_bounds__(1024) void scan_outliers_full_kernel(
    const uint16_t* __restrict__ X, int64_t T, int64_t K, float tau, uint32_t* __restrict__ bitmap) {
  constexpr int RPT = 8;  // rows per batch of loads
  __shared__ uint32_t s_m[16][4][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t nch = K >> 3;
  const int64_t c = (int64_t)blockIdx.x * 64 + lane;
  const u32x4* p = reinterpret_cast<const u32x4*>(X) + (c < nch ? c : nch - 1);
  uint32_t m[4] = {0u, 0u, 0u, 0u};
  for (int64_t r0 = wid; r0 < T; r0 += 16 * RPT) {
    // rows past the end repeat the last row: a repeated row changes no maximum
    u32x4 v[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int64_t r = r0 + 16 * i;
      v[i] = p[(r < T ? r : T - 1) * nch];
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) m[d] = pk_max_u16(m[d], v[i][d] & 0x7FFF7FFFu);
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) s_m[wid][d][lane] = m[d];
  __syncthreads();
  if (wid == 0) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int w = 1; w < 16; ++w) m[d] = pk_max_u16(m[d], s_m[w][d][lane]);
    const uint32_t flags = (c < nch) ? flags8(m, magnitude_threshold<DT>(tau)) : 0u;
    uint32_t word = flags << ((lane & 3) * 8);
    word |= __shfl_xor(word, 1, WAVE);
    word |= __shfl_xor(word, 2, WAVE);
    if ((lane & 3) == 0 && c < nch) bitmap[c >> 2] = word;
  }
}

// Many rows (K % 8 == 0): the 1024-thread strip workgroup above over a range
// of rows, its final words ORed into the bitmap (non-zero ones only).  A grid
// of about two workgroups per compute unit keeps the atomics few (1024
// single-pass workgroups of four waves took 12.4 against 10.0 us at 4096 x
// 4096 fp16), and sixteen waves of four rows per batch keep 128 KiB of loads
// in flight per compute unit: 4096 x 4096 fp16 7.4 us, 4096 x 12288 18.3 us,
// against 7.85 and 18.9 us with eight rows per batch and one workgroup per
// compute unit, and 8.2 and 20.1 us with four waves per workgroup.
constexpr int SCAN_WIDE_RPT = 4;

template <int DT>
__global__ __launch_bounds__(1024) void scan_outliers_wide_kernel(
    const uint16_t* __restrict__ X, int64_t T, int64_t K, float tau, uint32_t* __restrict__ bitmap,
    int rows_per_block) {
  constexpr int RPT = SCAN_WIDE_RPT;  // rows per batch of loads
  __shared__ uint32_t s_m[16][4][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t nch = K >> 3;
  const int64_t c = (int64_t)blockIdx.x * 64 + lane;
  const u32x4* p = reinterpret_cast<const u32x4*>(X) + (c < nch ? c : nch - 1);
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r_end = min(T, r_begin + rows_per_block);
  uint32_t m[4] = {0u, 0u, 0u, 0u};
  for (int64_t r0 = r_begin + wid; r0 < r_end; r0 += 16 * RPT) {
    // rows past the range repeat its last row: a repeated row changes no maximum
    u32x4 v[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int64_t r = r0 + 16 * i;
      v[i] = p[(r < r_end ? r : r_end - 1) * nch];
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) m[d] = pk_max_u16(m[d], v[i][d] & 0x7FFF7FFFu);
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) s_m[wid][d][lane] = m[d];
  __syncthreads();
  if (wid == 0) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int w = 1; w < 16; ++w) m[d] = pk_max_u16(m[d], s_m[w][d][lane]);
    const uint32_t flags = (c < nch) ? flags8(m, magnitude_threshold<DT>(tau)) : 0u;
    uint32_t word = flags << ((lane & 3) * 8);
    word |= __shfl_xor(word, 1, WAVE);
    word |= __shfl_xor(word, 2, WAVE);
    if ((lane & 3) == 0 && c < nch && word != 0u) atomicOr(bitmap + (c >> 2), word);
  }
}

bool scan_writes_all_words(int64_t T, int64_t K) { return T >= 1 && T <= SCAN_FULL_MAX_T && (K & 7) == 0; }

hipError_t launch_scan_outliers(int dt, const void* X, int64_t T, int64_t K, float tau,
                                uint32_t* bitmap, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (scan_writes_all_words(T, K)) {
    const unsigned strips = (unsigned)((K / 8 + 63) / 64);
    if (dt == DT_F16)
      scan_outliers_full_kernel<DT_F16><<<dim3(strips), 1024, 0, s>>>(x, T, K, tau, bitmap);
    else
      scan_outliers_full_kernel<DT_BF16><<<dim3(strips), 1024, 0, s>>>(x, T, K, tau, bitmap);
    return hipGetLastError();
  }
  if ((K & 7) == 0) {
    const int64_t gx = (K / 8 + 63) / 64;
    // rows per workgroup: at least one batch (16 waves x SCAN_WIDE_RPT rows),
    // else as many as make about two workgroups per compute unit
    const int64_t gy_want = std::max<int64_t>(1, 512 / gx);
    const int64_t rows = std::max<int64_t>(16 * SCAN_WIDE_RPT, (T + gy_want - 1) / gy_want);
    const int64_t gy = (T + rows - 1) / rows;
    dim3 grid((unsigned)gx, (unsigned)gy);
    if (dt == DT_F16)
      scan_outliers_wide_kernel<DT_F16><<<grid, 1024, 0, s>>>(x, T, K, tau, bitmap, (int)rows);
    else
      scan_outliers_wide_kernel<DT_BF16><<<grid, 1024, 0, s>>>(x, T, K, tau, bitmap, (int)rows);
  } else {
    const int64_t gx = (K + 255) / 256;
    const int rows = 64;
    dim3 grid((unsigned)gx, (unsigned)((T + rows - 1) / rows));
    if (dt == DT_F16)
      scan_outliers_any_kernel<DT_F16><<<grid, 256, 0, s>>>(x, T, K, tau, bitmap, rows);
    else
      scan_outliers_any_kernel<DT_BF16><<<grid, 256, 0, s>>>(x, T, K, tau, bitmap, rows);
  }
  return hipGetLastError();
}

// ------------------------------------------------------- row quantisers ----
// Shared prologue of the activation quantiser: the bitmap goes to LDS with an
// exclusive prefix count per word, so every column knows its rank among the
// outlier columns.  Block 0 also writes the ascending index list and count.
// LDS: words[W], prefix[W].  Returns the number of outlier columns.
__device__ int load_bitmap_prefix(const uint32_t* __restrict__ bitmap, int64_t W,
                                  uint32_t* words, uint32_t* prefix,
                                  int32_t* __restrict__ idx, int32_t* __restrict__ n_idx) {
  for (int64_t w = threadIdx.x; w < W; w += blockDim.x) words[w] = bitmap[w];
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int64_t seg = (W + 63) / 64;
    const int64_t w0 = lane * seg, w1 = min(W, w0 + seg);
    int cnt = 0;
    for (int64_t w = w0; w < w1; ++w) cnt += __popc(words[w]);
    int run = wave_incl_scan(cnt) - cnt;
    for (int64_t w = w0; w < w1; ++w) {
      prefix[w] = (uint32_t)run;
      run += __popc(words[w]);
    }
  }
  __syncthreads();
  const int total = (W > 0) ? (int)(prefix[W - 1] + __popc(words[W - 1])) : 0;
  if (blockIdx.x == 0) {
    for (int64_t w = threadIdx.x; w < W; w += blockDim.x) {
      uint32_t m = words[w];
      int pos = (int)prefix[w];
      while (m) {
        const int b = __builtin_ctz(m);
        idx[pos++] = (int32_t)(w * 32 + b);
        m &= m - 1u;
      }
    }
    if (threadIdx.x == 0) *n_idx = total;
  }
  return total;
}

// Gathered outlier columns of X: chunk-major [ceil(n/32)][T][32] of 16-bit
// values, zero beyond n, so the 16-bit product can stream 64-byte rows.
__device__ __forceinline__ int64_t xo_offset(int p, int64_t row, int64_t T) {
  return ((int64_t)(p >> 5) * T + row) * 32 + (p & 31);
}

__device__ __forceinline__ void xo_zero_pad(uint16_t* __restrict__ xo, int total, int64_t row,
                                            int64_t T, int lane) {
  const int npad = (total + 31) & ~31;
  for (int p = total + lane; p < npad; p += WAVE) xo[xo_offset(p, row, T)] = 0;
}

// The same prologue with the bitmap words already loaded (thread t holds
// words t and t + 256, W <= 512), and barriers that wait for LDS only: the
// caller's row loads stay in flight through it.
__device__ int bitmap_prefix_regs(const uint32_t (&bw)[2], int64_t W, uint32_t* words, uint32_t* prefix,
                                  int32_t* __restrict__ idx, int32_t* __restrict__ n_idx) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t w = threadIdx.x + 256 * i;
    if (w < W) words[w] = bw[i];
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the words are in LDS
  __builtin_amdgcn_s_barrier();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int64_t seg = (W + 63) / 64;
    const int64_t w0 = lane * seg, w1 = min(W, w0 + seg);
    int cnt = 0;
    for (int64_t w = w0; w < w1; ++w) cnt += __popc(words[w]);
    int run = wave_incl_scan(cnt) - cnt;
    for (int64_t w = w0; w < w1; ++w) {
      prefix[w] = (uint32_t)run;
      run += __popc(words[w]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  const int total = (int)(prefix[W - 1] + __popc(words[W - 1]));
  if (blockIdx.x == 0) {
    for (int64_t w = threadIdx.x; w < W; w += blockDim.x) {
      uint32_t m = words[w];
      int pos = (int)prefix[w];
      while (m) {
        const int b = __builtin_ctz(m);
        idx[pos++] = (int32_t)(w * 32 + b);
        m &= m - 1u;
      }
    }
    if (threadIdx.x == 0) *n_idx = total;
  }
  return total;
}

// One wave per row; the row stays in registers (MAXC 16-byte chunks per lane),
// so HBM sees it once.  Requires K % 8 == 0 and K <= 512 * MAXC.
// EXCL: activation mode (outlier columns excluded, index list, gather).
// Row absmax as a packed 16-bit max of the 15-bit magnitudes (exact: the
// largest bit pattern is the largest value); codes two at a time with
// code_pair16.  Loads are unconditional at in-range addresses (chunks past
// the row end re-read chunk 0 and are masked), so they are counted in order.
template <int DT, bool EXCL, int MAXC>
__global__ __launch_bounds__(256) void quant_rows_reg_kernel(
    const uint16_t* __restrict__ src, int64_t R, int64_t K, int8_t* __restrict__ codes,
    float* __restrict__ scales, const uint32_t* __restrict__ bitmap,
    int32_t* __restrict__ idx, int32_t* __restrict__ n_idx, uint16_t* __restrict__ xo) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t W = (K + 31) >> 5;
  // Activation mode: the bitmap words first, then the row, whose loads stay
  // in flight through the bitmap prologue (R >= 1 here: rows past R re-read
  // the last one and return before using it).
  uint32_t bw[2] = {0u, 0u};
  if constexpr (EXCL) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t w = threadIdx.x + 256 * i;
      bw[i] = bitmap[w < W ? w : W - 1];
    }
  }
  const int64_t row = (int64_t)blockIdx.x * 4 + wid;
  const int64_t nch = K >> 3;
  const u32x4* rp = reinterpret_cast<const u32x4*>(src + (row < R ? row : R - 1) * K);
  u32x4 v[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int64_t c = lane + (int64_t)i * WAVE;
    v[i] = __builtin_nontemporal_load(rp + (c < nch ? c : 0));
  }
  // The bitmap words are taken here, behind the row loads in the count, so
  // the prologue waits for them alone (left to its conditional stores, the
  // compiler sinks the first word's load below the row loads and waits for
  // the whole row before the prologue starts).
  if constexpr (EXCL) asm volatile("" : "+v"(bw[0]), "+v"(bw[1]));
  int total = 0;
  if constexpr (EXCL) total = bitmap_prefix_regs(bw, W, lds, lds + W, idx, n_idx);
  const uint32_t* words = lds;
  const uint32_t* prefix = lds + W;
  if (row >= R) return;
  // The whole row, waited for once: otherwise each chunk's Xo stores below
  // are followed by a wait for every memory operation in flight (loads and
  // stores share one counter), so every further chunk with an outlier column
  // waits for the previous one's stores to land (4096 x 4096 fp16, four
  // outlier columns, back to back: 13.6 -> 13.1 us per launch).
  if constexpr (EXCL) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // Outlier columns (and chunks past the row end) are zeroed in place, so
  // that neither the row maximum nor the codes need a mask per value: a zero
  // value codes to 0.  Only chunk positions where some lane of the wave has
  // such a column take the branch (outlier columns are few), and the outlier
  // values go to Xo first.
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int64_t c = lane + (int64_t)i * WAVE;
    uint32_t f = 0xFFu;
    if (c < nch) f = EXCL ? (words[c >> 2] >> ((c & 3) * 8)) & 0xFFu : 0u;
    if (__ballot(f != 0u) != 0) {
      if constexpr (EXCL) {
        // this chunk's outlier columns into Xo, a loop over the set bits (an
        // unrolled test per column would keep a mask per column live)
        uint32_t g = (c < nch && xo != nullptr) ? f : 0u;
        if (g != 0u) {
          const int64_t cw = c >> 2;
          const uint32_t word = words[cw];
          const int base = (int)prefix[cw];
          while (g) {
            const int e = __builtin_ctz(g);
            g &= g - 1u;
            const int bit = (int)((c & 3) * 8 + e);
            const int p = base + __popc(word & ((1u << bit) - 1u));
            xo[xo_offset(p, row, R)] = (uint16_t)half_bits(v[i], e);
          }
        }
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // 0xFFFF in each half whose value is kept: (1 - flag) per half, times 0xFFFF
        const uint32_t t = (((f >> (2 * d)) & 1u) | (((f >> (2 * d + 1)) & 1u) << 16)) ^ 0x00010001u;
        v[i][d] &= t * 0xFFFFu;
      }
    }
  }
  uint32_t mx = 0u;
#pragma unroll
  for (int i = 0; i < MAXC; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d) mx = pk_max_u16(mx, v[i][d] & 0x7FFF7FFFu);
  mx = max(mx & 0xFFFFu, mx >> 16);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, WAVE));
  const float m = to_f32<DT>(mx);  // exact absmax of the kept values
  const float s = row_factor(m);
  u32x2* cp = reinterpret_cast<u32x2*>(codes + row * K);
  auto put_codes = [&](auto PREc) {
    constexpr bool PRE = decltype(PREc)::value;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int64_t c = lane + (int64_t)i * WAVE;
      u32x2 pk;
      pk[0] = pack_codes16(code_pair16<DT, PRE>(v[i][0], s), code_pair16<DT, PRE>(v[i][1], s));
      pk[1] = pack_codes16(code_pair16<DT, PRE>(v[i][2], s), code_pair16<DT, PRE>(v[i][3], s));
      if (c < nch) cp[c] = pk;
    }
  };
  if (DT == DT_BF16 && tiny_absmax(m)) put_codes(std::integral_constant<bool, DT == DT_BF16>());  // uniform per row
  else put_codes(std::false_type());
  if (lane == 0) scales[row] = m;
  if constexpr (EXCL) {
    if (xo != nullptr) xo_zero_pad(xo, total, row, R, lane);
  }
}

// Any K (and K beyond the register budget): two passes over the row, the
// second served from cache.  One wave per row.
template <int DT, bool EXCL>
__global__ __launch_bounds__(256) void quant_rows_any_kernel(
    const uint16_t* __restrict__ src, int64_t R, int64_t K, int8_t* __restrict__ codes,
    float* __restrict__ scales, const uint32_t* __restrict__ bitmap,
    int32_t* __restrict__ idx, int32_t* __restrict__ n_idx, uint16_t* __restrict__ xo) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t W = (K + 31) >> 5;
  int total = 0;
  if constexpr (EXCL) total = load_bitmap_prefix(bitmap, W, lds, lds + W, idx, n_idx);
  const uint32_t* words = lds;
  const uint32_t* prefix = lds + W;

  const int64_t row = (int64_t)blockIdx.x * 4 + wid;
  if (row >= R) return;
  const uint16_t* rp = src + row * K;
  float m = 0.0f;
  for (int64_t k = lane; k < K; k += WAVE) {
    bool out = false;
    if constexpr (EXCL) out = (words[k >> 5] >> (k & 31)) & 1u;
    if (!out) m = fmaxf(m, fabsf(to_f32<DT>(rp[k])));
  }
  m = wave_max(m);
  const float s = row_factor(m);
  const float pre = tiny_absmax(m) ? PRESCALE : 1.0f;  // (1: the plain product, unchanged)
  int8_t* cp = codes + row * K;
  for (int64_t k = lane; k < K; k += WAVE) {
    const uint32_t h = rp[k];
    bool out = false;
    if constexpr (EXCL) out = (words[k >> 5] >> (k & 31)) & 1u;
    int q = 0;
    if (!out && m > 0.0f) q = quant_code(to_f32<DT>(h) * pre, s);
    cp[k] = (int8_t)q;
    if constexpr (EXCL) {
      if (out && xo != nullptr) {
        const uint32_t word = words[k >> 5];
        const int p = (int)prefix[k >> 5] + __popc(word & ((1u << (k & 31)) - 1u));
        xo[xo_offset(p, row, R)] = (uint16_t)h;
      }
    }
  }
  if (lane == 0) scales[row] = m;
  if constexpr (EXCL) {
    if (xo != nullptr) xo_zero_pad(xo, total, row, R, lane);
  }
}

template <int DT, bool EXCL>
static hipError_t launch_quant_rows_t(const uint16_t* src, int64_t R, int64_t K, int8_t* codes,
                                      float* scales, const uint32_t* bitmap, int32_t* idx,
                                      int32_t* n_idx, uint16_t* xo, hipStream_t s) {
  // Activation mode launches at least one block, so that block 0 writes the
  // index list and count even for T == 0.
  const int64_t nb4 = (R + 3) / 4;
  const int64_t blocks = (EXCL && nb4 < 1) ? 1 : nb4;
  if (blocks == 0) return hipSuccess;
  const size_t lds = EXCL ? (size_t)2 * ((K + 31) / 32) * sizeof(uint32_t) : 0;
  dim3 grid((unsigned)blocks), block(256);
  if (R == 0)  // activation mode, no rows: index list and count only
    quant_rows_any_kernel<DT, EXCL><<<grid, block, lds, s>>>(src, R, K, codes, scales, bitmap, idx, n_idx, xo);
  else if ((K & 7) == 0 && K <= 512 * 2)
    quant_rows_reg_kernel<DT, EXCL, 2><<<grid, block, lds, s>>>(src, R, K, codes, scales, bitmap, idx, n_idx, xo);
  else if ((K & 7) == 0 && K <= 512 * 8)
    quant_rows_reg_kernel<DT, EXCL, 8><<<grid, block, lds, s>>>(src, R, K, codes, scales, bitmap, idx, n_idx, xo);
  else if ((K & 7) == 0 && K <= 512 * 16)
    quant_rows_reg_kernel<DT, EXCL, 16><<<grid, block, lds, s>>>(src, R, K, codes, scales, bitmap, idx, n_idx, xo);
  else if ((K & 7) == 0 && K <= 512 * 24)
    quant_rows_reg_kernel<DT, EXCL, 24><<<grid, block, lds, s>>>(src, R, K, codes, scales, bitmap, idx, n_idx, xo);
  else
    quant_rows_any_kernel<DT, EXCL><<<grid, block, lds, s>>>(src, R, K, codes, scales, bitmap, idx, n_idx, xo);
  return hipGetLastError();
}

hipError_t launch_quant_weight(int dt, const void* W, int64_t N, int64_t K, int8_t* CB, float* SCB,
                               hipStream_t s) {
  const uint16_t* w = static_cast<const uint16_t*>(W);
  if (dt == DT_F16)
    return launch_quant_rows_t<DT_F16, false>(w, N, K, CB, SCB, nullptr, nullptr, nullptr, nullptr, s);
  return launch_quant_rows_t<DT_BF16, false>(w, N, K, CB, SCB, nullptr, nullptr, nullptr, nullptr, s);
}

// ------------------------------------------ few rows: split in one launch ----
// T <= 32, K % 8 == 0, K <= 4096: the outlier scan and the row quantiser in
// one launch, with no workgroup waiting on another.  Workgroup r quantises
// row r, and every workgroup reads all T rows to find the outlier columns
// itself (at most 256 KiB of X, in L2 after the first touch).  Thread c owns
// the 8-column chunk c: its loads of all rows (rows past T repeat row T - 1,
// which changes no maximum) go out at once, then the column maxima give its
// flags; its own row's chunk is one of them.  (Two batches of 32 rows for T
// up to 64 measured no faster than the two launches.)  The rest follows the row
// quantiser: absmax of the kept values (exact packed 16-bit maxima), codes by
// code_pair16, outlier columns gathered into Xo at their rank in the
// ascending index list, and workgroup 0 writes the bitmap, list and count.
constexpr int64_t SPLIT_SMALL_MAX_T = 32;

template <int DT, int ROWS>
__global__ __launch_bounds__(512) void split_small_kernel(
    const uint16_t* __restrict__ X, int64_t T, int64_t K, float tau, int8_t* __restrict__ codes,
    float* __restrict__ scales, uint32_t* __restrict__ bitmap, int32_t* __restrict__ idx,
    int32_t* __restrict__ n_idx, uint16_t* __restrict__ xo) {
  __shared__ uint32_t s_words[128], s_prefix[128], s_max[8];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t row = blockIdx.x;
  const int64_t nch = K >> 3, W = (K + 31) >> 5;
  const int c = tid;
  const bool cok = c < nch;
  const u32x4* p = reinterpret_cast<const u32x4*>(X) + (cok ? c : 0);
  uint32_t m[4] = {0u, 0u, 0u, 0u};
  u32x4 x = (u32x4){0u, 0u, 0u, 0u};  // this row's chunk
  for (int r0 = 0; r0 < T; r0 += ROWS) {  // one batch (T <= ROWS)
    u32x4 v[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) v[i] = p[(r0 + i < T ? r0 + i : T - 1) * nch];
    __builtin_amdgcn_sched_barrier(0);  // the batch's loads all in flight before the first wait
#pragma unroll
    for (int i = 0; i < ROWS; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) m[d] = pk_max_u16(m[d], v[i][d] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 0; i < ROWS; ++i)
      if (r0 + i == row) x = v[i];
  }
  const uint32_t f8 = cok ? flags8(m, magnitude_threshold<DT>(tau)) : 0u;
  uint32_t wv = f8 << ((c & 3) * 8);
  wv |= __shfl_xor(wv, 1, WAVE);
  wv |= __shfl_xor(wv, 2, WAVE);
  if ((c & 3) == 0 && cok) s_words[c >> 2] = wv;

  // chunks past the row end count as all-outlier (excluded)
  const uint32_t ob = cok ? f8 : 0xFFu;
  uint32_t mx = 0u;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t keep = (((ob >> (2 * d)) & 1u) ? 0u : 0x7FFFu) | (((ob >> (2 * d + 1)) & 1u) ? 0u : 0x7FFF0000u);
    mx = pk_max_u16(mx, x[d] & keep);
  }
  mx = max(mx & 0xFFFFu, mx >> 16);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, WAVE));
  if (lane == 0) s_max[wid] = mx;
  __syncthreads();
  if (wid == 0) {  // exclusive prefix count of outlier columns per word (W <= 128: two per lane)
    const uint32_t w0 = (2 * lane < W) ? s_words[2 * lane] : 0u;
    const uint32_t w1 = (2 * lane + 1 < W) ? s_words[2 * lane + 1] : 0u;
    const int cnt = __popc(w0) + __popc(w1);
    const int run = wave_incl_scan(cnt) - cnt;
    if (2 * lane < W) s_prefix[2 * lane] = (uint32_t)run;
    if (2 * lane + 1 < W) s_prefix[2 * lane + 1] = (uint32_t)(run + __popc(w0));
  }
  __syncthreads();
  const int total = (int)(s_prefix[W - 1] + __popc(s_words[W - 1]));
  uint32_t bm = s_max[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) bm = max(bm, s_max[i]);
  const float am = to_f32<DT>(bm);  // exact absmax of the row's kept values
  const float sc = row_factor(am);
  if (cok) {
    u32x2 pk;
    if (DT == DT_BF16 && tiny_absmax(am)) {  // uniform: one row per workgroup
      constexpr bool P = DT == DT_BF16;
      pk[0] = pack_codes16(code_pair16<DT, P>(x[0], sc), code_pair16<DT, P>(x[1], sc)) & ~byte_mask4(ob);
      pk[1] = pack_codes16(code_pair16<DT, P>(x[2], sc), code_pair16<DT, P>(x[3], sc)) & ~byte_mask4(ob >> 4);
    } else {
      pk[0] = pack_codes16(code_pair16<DT>(x[0], sc), code_pair16<DT>(x[1], sc)) & ~byte_mask4(ob);
      pk[1] = pack_codes16(code_pair16<DT>(x[2], sc), code_pair16<DT>(x[3], sc)) & ~byte_mask4(ob >> 4);
    }
    reinterpret_cast<u32x2*>(codes + row * K)[c] = pk;
  }
  if (xo != nullptr) {
    uint32_t f = f8;
    if (f != 0u) {
      const uint32_t word = s_words[c >> 2];
      const int base = (int)s_prefix[c >> 2];
      while (f) {
        const int e = __builtin_ctz(f);
        f &= f - 1u;
        const int bit = (c & 3) * 8 + e;
        const int rank = base + __popc(word & ((1u << bit) - 1u));
        xo[xo_offset(rank, row, T)] = (uint16_t)half_bits(x, e);
      }
    }
    if (wid == 0) xo_zero_pad(xo, total, row, T, lane);
  }
  if (tid == 0) scales[row] = am;
  if (blockIdx.x == 0) {
    for (int64_t w = tid; w < W; w += 512) {
      const uint32_t word = s_words[w];
      bitmap[w] = word;
      uint32_t mm = word;
      int pos = (int)s_prefix[w];
      while (mm) {
        const int b = __builtin_ctz(mm);
        idx[pos++] = (int32_t)(w * 32 + b);
        mm &= mm - 1u;
      }
    }
    if (tid == 0) *n_idx = total;
  }
}

bool split_small_supported(int64_t T, int64_t K) {
  return T >= 1 && T <= SPLIT_SMALL_MAX_T && (K & 7) == 0 && K <= 4096;
}

hipError_t launch_split_small(int dt, const void* X, int64_t T, int64_t K, float tau, int8_t* CA, float* SCA,
                              uint32_t* bitmap, int32_t* idx, int32_t* n_idx, void* xo, hipStream_t s) {
  if (!split_small_supported(T, K)) return hipErrorInvalidValue;
  const uint16_t* x = static_cast<const uint16_t*>(X);
  uint16_t* g = static_cast<uint16_t*>(xo);
  decltype(&split_small_kernel<DT_F16, 8>) k;
  if (dt == DT_F16)
    k = T <= 8 ? split_small_kernel<DT_F16, 8> : T <= 16 ? split_small_kernel<DT_F16, 16>
      : T <= 24 ? split_small_kernel<DT_F16, 24> : split_small_kernel<DT_F16, 32>;
  else
    k = T <= 8 ? split_small_kernel<DT_BF16, 8> : T <= 16 ? split_small_kernel<DT_BF16, 16>
      : T <= 24 ? split_small_kernel<DT_BF16, 24> : split_small_kernel<DT_BF16, 32>;
  k<<<dim3((unsigned)T), dim3(512), 0, s>>>(x, T, K, tau, CA, SCA, bitmap, idx, n_idx, g);
  return hipGetLastError();
}

hipError_t launch_quant_act(int dt, const void* X, int64_t T, int64_t K, const uint32_t* bitmap,
                            int8_t* CA, float* SCA, int32_t* idx, int32_t* n_idx, void* xo,
                            hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  uint16_t* g = static_cast<uint16_t*>(xo);
  if (dt == DT_F16)
    return launch_quant_rows_t<DT_F16, true>(x, T, K, CA, SCA, bitmap, idx, n_idx, g, s);
  return launch_quant_rows_t<DT_BF16, true>(x, T, K, CA, SCA, bitmap, idx, n_idx, g, s);
}

// ------------------------------------------------ recovered outlier weights ----
// dtype(fl32(fl32(CB * SCB) / 127)) ("Integration into transformers") of the
// outlier columns, written once per call chunk-major [chunk][N][32] (zero
// beyond n) so that every GEMM tile reads them as contiguous 64-byte rows
// instead of gathering single bytes of CB.  Thread = one 16-byte piece (8
// values) of one row; the columns come from the index list.  A fixed grid
// walks however many chunks this call's n fills (at most `chunks`).
template <int DT>
__global__ __launch_bounds__(256) void recover_outliers_kernel(
    const int8_t* __restrict__ CB, const float* __restrict__ SCB, int64_t N, int64_t K,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ n_idx_p, uint16_t* __restrict__ wo, int chunks) {
  const int total = *n_idx_p;
  const int used = min((total + 31) >> 5, chunks);
  // Piece q: part q % 4 of row 16 b + (q / 4) % 16 of chunk (q / 64) % used,
  // b = q / (64 used).  A wave writes 16 consecutive 64-byte rows of one
  // chunk (1 KiB, contiguous) and the next wave the same rows' next chunk,
  // whose CB bytes lie in the lines just read.
  const int64_t nblk = (N + 15) >> 4;
  const int64_t pieces = nblk * used * 64;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < pieces; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t g = q >> 6;  // (row block, chunk)
    const int64_t b = g / used;
    const int ch = (int)(g - b * used);
    const int64_t n = b * 16 + ((q >> 2) & 15);
    if (n >= N) continue;
    const int cp = ch * 4 + (int)(q & 3);  // chunk * 4 + part
    const int p0 = cp * 8;
    const float scb = SCB[n];
    const int8_t* cbrow = CB + n * K;
    uint32_t v[4] = {0u, 0u, 0u, 0u};
    const int c0 = (p0 < total) ? idx[p0] : 0;
    if (p0 + 8 <= total && (K & 3) == 0 && idx[p0 + 7] - c0 == 7) {
      // eight consecutive columns (every column an outlier, say): three
      // aligned dwords cover them
      const int a0 = c0 & ~3, sh = c0 & 3;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(cbrow + a0);
      const uint32_t d0 = src[0], d1 = src[1], d2 = (sh != 0) ? src[2] : 0u;
      const uint32_t lo = (uint32_t)(((uint64_t)d1 << 32 | d0) >> (8 * sh));
      const uint32_t hi = (uint32_t)(((uint64_t)d2 << 32 | d1) >> (8 * sh));
      // the division's range test once per piece, not per value (the eight
      // values share the row scale): the conversion and division are most of
      // this kernel's work when every column is an outlier
      if (div127_scale_ok(scb)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int8_t cb = (int8_t)(((e < 4 ? lo : hi) >> (8 * (e & 3))) & 0xFFu);
          v[e >> 1] |= (uint32_t)from_f32<DT>(div127_inrange((float)cb * scb)) << (16 * (e & 1));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int8_t cb = (int8_t)(((e < 4 ? lo : hi) >> (8 * (e & 3))) & 0xFFu);
          v[e >> 1] |= (uint32_t)from_f32<DT>(div127((float)cb * scb)) << (16 * (e & 1));
        }
      }
    } else {
      // scattered columns: the eight indices, then the eight bytes, each set
      // requested at once (index clamped into the list; surplus values are
      // dropped below), rather than a load behind a condition per value,
      // which the compiler waits on one at a time
      int col[8];
      int8_t cbv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) col[e] = idx[p0 + e < total ? p0 + e : total - 1];
#pragma unroll
      for (int e = 0; e < 8; ++e) cbv[e] = cbrow[col[e]];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (p0 + e < total) {
          const uint32_t w = from_f32<DT>(div127((float)cbv[e] * scb));
          v[e >> 1] |= w << (16 * (e & 1));
        }
      }
    }
    *reinterpret_cast<u32x4*>(wo + (((int64_t)(cp >> 2) * N + n) * 32 + (cp & 3) * 8)) = (u32x4){v[0], v[1], v[2], v[3]};
  }
}

hipError_t launch_recover_outliers(int dt, const int8_t* CB, const float* SCB, int64_t N, int64_t K,
                                   const int32_t* idx, const int32_t* n_idx, void* wo, int chunks, hipStream_t s) {
  if (wo == nullptr || chunks <= 0 || N <= 0) return hipSuccess;
  // How many chunks this call fills is known on the device only.  The grid
  // covers up to four (128 outlier columns: one piece per thread); the loop
  // walks any more.  A grid sized for every chunk the scratch can hold would
  // be mostly workgroups with nothing to do.
  const int64_t most = (int64_t)(chunks < 4 ? chunks : 4) * 64 * ((N + 15) / 16);
  const int64_t want = (most + 255) / 256;
  const int64_t blocks = want < 4096 ? want : 4096;
  uint16_t* w = static_cast<uint16_t*>(wo);
  if (dt == DT_F16)
    recover_outliers_kernel<DT_F16><<<dim3((unsigned)blocks), 256, 0, s>>>(CB, SCB, N, K, idx, n_idx, w, chunks);
  else
    recover_outliers_kernel<DT_BF16><<<dim3((unsigned)blocks), 256, 0, s>>>(CB, SCB, N, K, idx, n_idx, w, chunks);
  return hipGetLastError();
}

}  // namespace lli8
