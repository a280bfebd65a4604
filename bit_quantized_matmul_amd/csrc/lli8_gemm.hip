// int8 GEMM with the dequantisation, the 16-bit outlier product and the bias
// fused into its epilogue, on gfx950 MFMA.
//
// The method ("Hugging Face integrates LLM.int8() ...", section "Core idea of
// LLM.int8()"): the non-outlier part is an int8 x int8 product with int32
// accumulation, dequantised with the row scale of the activation and the row
// scale of the weight; the outlier columns are multiplied in 16-bit against
// the weight recovered as (CB * SCB) / 127 (section "Integration into
// transformers") and the two results are summed.
//
// Three kernels:
//   * persistent kernel (T, N, K multiples of 256): the 256 x 256 2-slot
//     tile loop below, one workgroup per compute unit walking its tiles,
//     the next tile's first steps loaded during the current tile's epilogue.
//   * tile kernel: BM x BN output tile per workgroup of WGM x WGN waves.
//     Large problems (T, N >= 512): 256 x 256 on 4 x 2 waves (two per SIMD),
//     K straight from memory into LDS with global_load_lds: 128-byte steps
//     in a 2-slot ring (K % 256 == 0; the step's barrier sits before its last
//     sub-step's MFMAs, and each sub-step's LDS operand reads interleave with
//     the previous sub-step's MFMAs), 64-byte steps in a 4-slot ring (K % 64
//     == 0), else register-staged 64-byte steps.  Smaller problems: 128 x 128
//     or 64 x 64 tiles on 2 x 2 waves, register-staged.  v_mfma_i32_32x32x32_i8
//     throughout.  The epilogue turns the int32 accumulators into fp32 in
//     place (same 32x32 register layout), runs the outlier columns through
//     v_mfma_f32_32x32x16_{f16,bf16} on the same registers, then adds the
//     bias and rounds once to the output dtype.
//   * weight-streaming kernel (up to 64 tokens, K % 16 == 0): each workgroup owns
//     16 output features and reads their int8 weight rows once with 16-byte
//     loads, 8 or 16 waves splitting K, v_mfma_i32_16x16x64_i8 per block of 16
//     tokens.
#include "lli8_device.h"
#include "lli8_internal.h"

namespace lli8 {


// LDS address of 16-byte chunk c of row r in a tile with KB-byte rows.  A
// 16-byte-per-lane LDS access is served 16 lanes (256 bytes, all 64 banks) at
// a time; the XOR gives the 16 consecutive rows that an MFMA-operand read
// touches (same logical chunk) 16 distinct 16-byte bank groups, and keeps the
// row-wise tile writes conflict-free too.
template <int KB>
__device__ __forceinline__ int tile_off(int r, int c) {
  if constexpr (KB == 64) return r * 64 + ((c ^ ((r >> 2) & 3)) << 4);
  else return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}
__device__ __forceinline__ int lds_off(int r, int c) { return tile_off<64>(r, c); }

// Recovered weight value for the 16-bit product: dtype(fl32(fl32(cb*scb)/127)).
template <int DT>
__device__ __forceinline__ uint16_t recover_w(int8_t cb, float scb) {
  const float p = (float)cb * scb;
  return from_f32<DT>(div127(p));
}

// Two fp32 values rounded (to nearest even) to the 16-bit dtype and packed,
// the first in the low half (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 v = {lo, hi};
  if constexpr (DT == DT_F16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
  }
}

template <int DT>
__device__ __forceinline__ v16f mfma16(const u32x4& a, const u32x4& b, const v16f& c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// Tile index -> (tile_m, tile_n).  Workgroups are dispatched round-robin over
// the eight XCDs; give each XCD a contiguous range of tiles, and walk that
// range in groups of GM tile rows so neighbours share A rows and B columns in
// their XCD's L2.
template <int GM>
__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nb = tiles_m * tiles_n;
  const int q = nb >> 3, rmd = nb & 7;
  const int xcd = b & 7, loc = b >> 3;
  const int t = xcd * q + min(xcd, rmd) + loc;
  const int per_group = GM * tiles_n;
  const int g = t / per_group;
  const int first_m = g * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int in = t - g * per_group;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

// s_waitcnt with only the vector-memory count constrained: at most N of this
// wave's vector memory operations still outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16 bytes per lane from global memory straight into LDS: lane l writes
// bytes 16 l .. 16 l + 15 after the wave-uniform LDS address `lds`.
__device__ __forceinline__ void load_lds16(const int8_t* g, int8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Scheduling hint for the region since the last sched_barrier: its MFMAs,
// LDS reads and global loads in round robin, one of each at a time, so that
// the reads and loads issue while earlier MFMAs occupy the matrix core.
template <int NM, int NR, int NL>
__device__ __forceinline__ void interleave_mfma() {
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if constexpr (NR > 0) if (m < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    if constexpr (NL > 0) if (m < NL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
  }
}

// The tile epilogue: int32 tile (copied to acc_out when asked) -> fp32
// dequantised -> plus the 16-bit outlier product -> one rounding -> out.
// ring_a/ring_b are the LDS buffers: with PF = 0 the outlier operands are
// staged there (the ring slots of a direct-load kernel; the first buffer for
// weights gathered from CB).  PF = 1 (whole tiles, every chunk's recovered
// weights in scratch) loads them straight into registers and leaves LDS
// alone, so the caller's loads of its next tile can be in flight; its
// before_store() runs once the last value the epilogue waits for has
// arrived, before the stores.
template <int DT, int BM, int BN, int WGM, int WGN, int DL, int FL, int PF, class F>
__device__ __forceinline__ void tile_epilogue(
    v16i (&acc)[BM / WGM / 32][BN / WGN / 32], int64_t m0, int64_t n0, int T, int N, int K,
    const float* __restrict__ SCA, const float* __restrict__ SCB, const uint16_t* __restrict__ bias,
    const uint16_t* __restrict__ xo, const int32_t* __restrict__ idx, int n_idx, const int8_t* __restrict__ CB,
    const uint16_t* __restrict__ wo, int wo_chunks, uint16_t* __restrict__ out, int32_t* __restrict__ acc_out,
    int8_t* const (&ra)[4], int8_t* const (&rb)[4], F&& before_store) {
  static_assert(!PF || FL, "register-staged outlier operands need whole tiles");
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  // the thread index through an empty asm: nothing derived from it is
  // hoisted out of a caller's tile loop to sit in registers through the
  // K loop
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  int8_t* const ep_a = ra[0];
  int8_t* const ep_b = rb[0];
  // ---- epilogue.  32x32 accumulator layout: lane holds column (lane & 31),
  // register r holds row 8 * (r / 4) + 4 * (lane / 32) + r % 4.
  const int64_t rbase = m0 + wm * WM + 4 * (lane >> 5);
  const int64_t cbase = n0 + wn * WN + (lane & 31);
  if (acc_out != nullptr) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
        if (row >= T) continue;
        int32_t* arow = acc_out + row * N + cbase;
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if (cbase + j * 32 < N) arow[j * 32] = acc[i][j][r];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // Dequantise in place, the fp32 value reusing the int32 accumulator's
  // registers (the f32 and i32 32x32 MFMAs share one register layout).  With
  // whole tiles the bias joins here, fl32(fl32(acc * SCA) * SCB / 127^2 +
  // bias), four consecutive row scales come in one 16-byte load, and the
  // stores below take two outputs each (N even keeps them aligned); otherwise
  // every access is bounds-checked and the bias is added at the end, which
  // keeps the checked path within the register budget.
  float sb[FN], bv[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t col = cbase + j * 32;
    sb[j] = (col < N) ? SCB[col] * (1.0f / 16129.0f) : 0.0f;
    if constexpr (FL) bv[j] = (bias != nullptr) ? to_f32<DT>(bias[col]) : 0.0f;
  }
  if constexpr (FL) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // rows 8 q + 4 (lane / 32) + 0..3 of this 32-row strip
        const v4f sa4 = *reinterpret_cast<const v4f*>(SCA + rbase + i * 32 + 8 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j][4 * q + e] =
                __float_as_int(__builtin_fmaf((float)acc[i][j][4 * q + e] * sa4[e], sb[j], bv[j]));
      }
      __builtin_amdgcn_sched_barrier(0);  // one strip's scales in flight at a time
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
        const float sa = (row < T) ? SCA[row] : 0.0f;
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j][r] = __float_as_int((float)acc[i][j][r] * (sa * sb[j]));
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the per-row loads of one strip at a time
    }
  }

  // 16-bit outlier product, 32 outlier columns per step.
  const int n_chunks = (n_idx + 31) >> 5;
  if constexpr (PF) {
    // operands straight from the chunk-major 64-byte rows of Xo and of the
    // recovered weights: lane (row l % 32) takes the 16-byte piece
    // 2 s + l / 32 for sub-step s, the MFMA operand layout
    for (int ch = 0; ch < n_chunks; ++ch) {
      u32x4 a[2][FM], b[2][FN];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c = 2 * s + (lane >> 5);
#pragma unroll
        for (int i = 0; i < FM; ++i)
          a[s][i] = *reinterpret_cast<const u32x4*>(
              xo + (((int64_t)ch * T + m0 + wm * WM + i * 32 + (lane & 31)) * 32 + c * 8));
#pragma unroll
        for (int j = 0; j < FN; ++j)
          b[s][j] = *reinterpret_cast<const u32x4*>(
              wo + (((int64_t)ch * N + n0 + wn * WN + j * 32 + (lane & 31)) * 32 + c * 8));
      }
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_bit_cast(v16i, mfma16<DT>(a[s][i], b[s][j], __builtin_bit_cast(v16f, acc[i][j])));
    }
  } else {
  int ch_done = 0;
  if constexpr (DL != 0) {
    // With the recovered weights in scratch, both operands are chunk-major
    // 64-byte rows: the chunks stream through the same LDS ring as the int8
    // steps (direct loads, DL slots), into the dequantised fp32 registers.
    if (n_chunks > 0 && n_chunks <= wo_chunks) {
      constexpr int NW = WGM * WGN;
      constexpr int IA = BM / 16 / NW, IB = BN / 16 / NW;  // 1 KiB loads per wave per chunk (16 rows each)
      static_assert(IA * 16 * NW == BM && IB * 16 * NW == BN, "tile rows must split evenly over the waves");
      const int8_t* xa[IA];
      const int8_t* wb[IB];
#pragma unroll
      for (int j = 0; j < IA; ++j) {
        const int r = (wid * IA + j) * 16 + (lane >> 2);
        const int64_t row = m0 + r < T ? m0 + r : (int64_t)T - 1;
        xa[j] = reinterpret_cast<const int8_t*>(xo) + row * 64 + (((lane & 3) ^ ((r >> 2) & 3)) << 4);
      }
#pragma unroll
      for (int j = 0; j < IB; ++j) {
        const int r = (wid * IB + j) * 16 + (lane >> 2);
        const int64_t row = n0 + r < N ? n0 + r : (int64_t)N - 1;
        wb[j] = reinterpret_cast<const int8_t*>(wo) + row * 64 + (((lane & 3) ^ ((r >> 2) & 3)) << 4);
      }
      auto issue16 = [&](int ch, int8_t* a_slot, int8_t* b_slot) {
        const int c = ch < n_chunks ? ch : n_chunks - 1;
        const int64_t oa = (int64_t)c * T * 64, ob = (int64_t)c * N * 64;
#pragma unroll
        for (int j = 0; j < IA; ++j) load_lds16(xa[j] + oa, a_slot + (wid * IA + j) * 1024);
#pragma unroll
        for (int j = 0; j < IB; ++j) load_lds16(wb[j] + ob, b_slot + (wid * IB + j) * 1024);
      };
      __syncthreads();  // everyone is done with the ring's int8 contents
#pragma unroll
      for (int st = 0; st < DL - 1; ++st) issue16(st, ra[st], rb[st]);
      for (int cg = 0; cg < n_chunks; cg += DL) {
#pragma unroll
        for (int i = 0; i < DL; ++i) {
          wait_vmcnt<(DL - 2) * (IA + IB)>();
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
          issue16(cg + i + DL - 1, ra[(i + DL - 1) % DL], rb[(i + DL - 1) % DL]);
          if (cg + i < n_chunks) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              const int c = 2 * s2 + (lane >> 5);
              u32x4 a[FM], b[FN];
#pragma unroll
              for (int ii = 0; ii < FM; ++ii)
                a[ii] = *reinterpret_cast<const u32x4*>(ra[i] + tile_off<64>(wm * WM + ii * 32 + (lane & 31), c));
#pragma unroll
              for (int jj = 0; jj < FN; ++jj)
                b[jj] = *reinterpret_cast<const u32x4*>(rb[i] + tile_off<64>(wn * WN + jj * 32 + (lane & 31), c));
#pragma unroll
              for (int ii = 0; ii < FM; ++ii)
#pragma unroll
                for (int jj = 0; jj < FN; ++jj)
                  acc[ii][jj] = __builtin_bit_cast(v16i, mfma16<DT>(a[ii], b[jj], __builtin_bit_cast(v16f, acc[ii][jj])));
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      wait_vmcnt<0>();
      ch_done = n_chunks;
    }
  }
  int8_t* oA = ep_a;  // [BM][32] 16-bit values, 64-byte rows
  int8_t* oB = ep_b;  // [BN][32]
  for (int ch = ch_done; ch < n_chunks; ++ch) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < BM * 4 / NT; ++i) {
      const int q = tid + NT * i, r = q >> 2, c = q & 3;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m0 + r < T) v = *reinterpret_cast<const u32x4*>(xo + (((int64_t)ch * T + m0 + r) * 32 + c * 8));
      *reinterpret_cast<u32x4*>(oA + lds_off(r, c)) = v;
    }
    if (ch < wo_chunks) {  // recovered weights precomputed once per call: contiguous rows
#pragma unroll
      for (int i = 0; i < BN * 4 / NT; ++i) {
        const int q = tid + NT * i, r = q >> 2, c = q & 3;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (n0 + r < N) v = *reinterpret_cast<const u32x4*>(wo + (((int64_t)ch * N + n0 + r) * 32 + c * 8));
        *reinterpret_cast<u32x4*>(oB + lds_off(r, c)) = v;
      }
    } else {  // gathered here
      const int j = tid & 31;
      const int p = ch * 32 + j;
      const bool valid = p < n_idx;
      const int64_t col = valid ? idx[p] : 0;
      for (int rr = tid >> 5; rr < BN; rr += NT / 32) {
        const int64_t gn = n0 + rr;
        uint16_t w = 0;
        if (valid && gn < N) w = recover_w<DT>(CB[gn * K + col], SCB[gn]);
        *reinterpret_cast<uint16_t*>(oB + lds_off(rr, j >> 3) + (j & 7) * 2) = w;
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 2 * s + (lane >> 5);
      u32x4 a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = *reinterpret_cast<const u32x4*>(oA + lds_off(wm * WM + i * 32 + (lane & 31), c));
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = *reinterpret_cast<const u32x4*>(oB + lds_off(wn * WN + j * 32 + (lane & 31), c));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_bit_cast(v16i, mfma16<DT>(a[i], b[j], __builtin_bit_cast(v16f, acc[i][j])));
    }
  }
  }  // PF

  before_store();

  // One rounding to the output dtype, store.
  if constexpr (FL) {
    // Rows R and R + 1 of a lane's column convert to one packed dword; lanes
    // 2c and 2c + 1 trade halves of it, so the even lane holds row R of
    // columns 2c, 2c + 1 and the odd lane row R + 1 of the same two columns:
    // one 4-byte store per two values.  Row offsets are uniform, so the
    // stores take a scalar base and one per-lane offset.
    const int odd = lane & 1;
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;  // odd: (nb.hi, own.hi), even: (own.lo, nb.lo)
    const uint32_t loff = (uint32_t)(((4 * (lane >> 5) + odd) * N + (lane & 31) - odd) * 2);
    const int swm = __builtin_amdgcn_readfirstlane(wm), swn = __builtin_amdgcn_readfirstlane(wn);
    char* const ubase = reinterpret_cast<char*>(out + (m0 + swm * WM) * N + n0 + swn * WN);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          char* const rowp = ubase + (int64_t)(i * 32 + 8 * q + 2 * p) * N * 2;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const uint32_t pk = pack2<DT>(__int_as_float(acc[i][j][4 * q + 2 * p]),
                                          __int_as_float(acc[i][j][4 * q + 2 * p + 1]));
            const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)pk, 0xB1, 0xF, 0xF, false);  // lane ^ 1
            *reinterpret_cast<uint32_t*>(rowp + j * 64 + loff) = __builtin_amdgcn_perm(nb, pk, sel);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = cbase + j * 32;
      bv[j] = (bias != nullptr && col < N) ? to_f32<DT>(bias[col]) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
        if (row >= T) continue;
        uint16_t* orow = out + row * N + cbase;
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if (cbase + j * 32 < N) orow[j * 32] = from_f32<DT>(__int_as_float(acc[i][j][r]) + bv[j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// DL = 0: global loads staged through registers, LDS double buffered (any K).
// DL = 2 (K a multiple of 2 BK): loads go straight from global memory into two
// LDS slots, two steps in flight, steps run in pairs.
// DL = D >= 3 (K % BK == 0): straight into a D-slot LDS ring, D - 1 steps ahead.
// FL = 1: every tile lies wholly inside the output (T % BM == 0, N % BN ==
// 0, N even), and the epilogue drops its bounds checks.
// KM (register-staged loads): 0 K % BK == 0; 1 K % 16 == 0 (16-byte loads,
// chunks past K zeroed); 3 K % 8 == 0 (8-byte loads); 4 K % 4 == 0 (4-byte
// loads); 2 any K (bytes).
template <int DT, int BM, int BN, int KM, int BK, int WGM, int WGN, int GM, int DL, int FL>
__global__ __launch_bounds__(64 * WGM * WGN) void linear_tile_kernel(
    const int8_t* __restrict__ CA, const int8_t* __restrict__ CB, const float* __restrict__ SCA,
    const float* __restrict__ SCB, const uint16_t* __restrict__ bias, const uint16_t* __restrict__ xo,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ n_idx_p, uint16_t* __restrict__ out,
    int32_t* __restrict__ acc_out, int T, int N, int K, int tiles_m, int tiles_n,
    const uint16_t* __restrict__ wo, int wo_chunks) {
  constexpr int NT = 64 * WGM * WGN;                    // threads: WGM x WGN waves
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int CPR = BK / 16;                          // 16-byte chunks per tile row
  constexpr int SS = BK / 32;                           // MFMA sub-steps per K step
  constexpr int LA = BM * CPR / NT, LB = BN * CPR / NT;  // 16-byte chunks per thread per step
  static_assert(LA * NT == BM * CPR && LB * NT == BN * CPR, "tile rows must split evenly over the threads");
  static_assert((BM * 4) % NT == 0 && (BN * 4) % NT == 0, "outlier staging: 64-byte rows split evenly over the threads");
  static_assert(DL == 0 || (DL >= 2 && DL <= 4 && KM == 0), "direct loads: K a multiple of the step");
  // register-staged loads: one double-buffered array each; direct loads: one
  // LDS object per ring slot (slots beyond DL are never touched)
  constexpr int SZA = DL ? 1 : 2 * BM * BK, SZB = DL ? 1 : 2 * BN * BK;
  constexpr int RA = DL ? BM * BK : 1, RB = DL ? BN * BK : 1;
  __shared__ __attribute__((aligned(16))) int8_t sA_[SZA];
  __shared__ __attribute__((aligned(16))) int8_t sB_[SZB];
  __shared__ __attribute__((aligned(16))) int8_t dA0[RA], dA1[RA], dA2[DL >= 3 ? RA : 1], dA3[DL >= 4 ? RA : 1];
  __shared__ __attribute__((aligned(16))) int8_t dB0[RB], dB1[RB], dB2[DL >= 3 ? RB : 1], dB3[DL >= 4 ? RB : 1];
  int8_t (*sA)[BM * BK] = reinterpret_cast<int8_t (*)[BM * BK]>(sA_);
  int8_t (*sB)[BN * BK] = reinterpret_cast<int8_t (*)[BN * BK]>(sB_);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  int tm, tn;
  tile_coords<GM>(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int n_idx = *n_idx_p;

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (v16i){0};

  // Global loads run two K steps ahead in two register sets; LDS is double
  // buffered.  Step kt: issue the loads of step kt + 2, multiply out of LDS
  // buffer kt & 1, then store step kt + 1 (loaded one step earlier) into the
  // other buffer.  Loads are branch-free so the compiler's wait counts stay
  // exact: rows past T (N) are clamped to the last row and only feed
  // accumulators that are never stored; steps past the end re-read the last
  // one and are never stored; with K % 64 != 0 (KM >= 1) chunks past K are
  // read at column 0 and zeroed before they reach LDS.
  const int nk = (K + BK - 1) / BK;
  const int8_t* pa[LA];
  const int8_t* pb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = (tid + NT * i) / CPR;
    const int64_t row = m0 + r < T ? m0 + r : (int64_t)T - 1;
    pa[i] = CA + row * K;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = (tid + NT * i) / CPR;
    const int64_t row = n0 + r < N ? n0 + r : (int64_t)N - 1;
    pb[i] = CB + row * K;
  }
  const int cq = (tid % CPR) * 16;  // byte offset of this thread's chunk within a step
  u32x4 ra0[LA], rb0[LB], ra1[LA], rb1[LB];
  auto ld = [&](const int8_t* row, int k) -> u32x4 {
    // Narrow loads past K read an in-range address and are zeroed after the
    // load: a load behind the condition would be a branch, and the compiler
    // waits for every load in flight before each one (16x slower at K = 4008).
    if constexpr (KM == 2) {  // K % 4 != 0: byte-wise, zero past K
      uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int bb = 0; bb < 16; ++bb) {
        const int kk = k + bb;
        const uint32_t v = (uint32_t)(uint8_t)row[kk < K ? kk : 0];
        wv[bb >> 2] |= (kk < K ? v : 0u) << (8 * (bb & 3));
      }
      return (u32x4){wv[0], wv[1], wv[2], wv[3]};
    } else if constexpr (KM == 3) {  // K % 8 == 0, K % 16 != 0: two 8-byte halves
      u32x2 h[2];
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int kd = k + 8 * d;
        const u32x2 v = *reinterpret_cast<const u32x2*>(row + (kd < K ? kd : 0));
        h[d] = kd < K ? v : (u32x2){0u, 0u};
      }
      return (u32x4){h[0][0], h[0][1], h[1][0], h[1][1]};
    } else if constexpr (KM == 4) {  // K % 4 == 0, K % 8 != 0: dword-wise
      uint32_t wv[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int kd = k + 4 * d;
        const uint32_t v = *reinterpret_cast<const uint32_t*>(row + (kd < K ? kd : 0));
        wv[d] = kd < K ? v : 0u;
      }
      return (u32x4){wv[0], wv[1], wv[2], wv[3]};
    } else {
      return *reinterpret_cast<const u32x4*>(row + ((KM == 0 || k < K) ? k : 0));
    }
  };
  auto gload = [&](int kt, u32x4 (&ra)[LA], u32x4 (&rb)[LB]) {
    const int k = min(kt, nk - 1) * BK + cq;
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = ld(pa[i], k);
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = ld(pb[i], k);
  };
  auto fix_tail = [&](int kt, u32x4 (&ra)[LA], u32x4 (&rb)[LB]) {
    if constexpr (KM == 1) {
      if (kt * BK + cq >= K) {
#pragma unroll
        for (int i = 0; i < LA; ++i) ra[i] = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < LB; ++i) rb[i] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
  };
  auto lstore = [&](int buf, const u32x4 (&ra)[LA], const u32x4 (&rb)[LB]) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int q = tid + NT * i, r = q / CPR, c = q % CPR;
      *reinterpret_cast<u32x4*>(&sA[buf][tile_off<BK>(r, c)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int q = tid + NT * i, r = q / CPR, c = q % CPR;
      *reinterpret_cast<u32x4*>(&sB[buf][tile_off<BK>(r, c)]) = rb[i];
    }
  };
  // MFMA operands for one 32-deep sub-step s of a step.
  auto read_frags = [&](int buf, int s, v4i (&fa)[FM], v4i (&fb)[FN]) {
    const int c = 2 * s + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[i] = *reinterpret_cast<const v4i*>(&sA[buf][tile_off<BK>(wm * WM + i * 32 + (lane & 31), c)]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[j] = *reinterpret_cast<const v4i*>(&sB[buf][tile_off<BK>(wn * WN + j * 32 + (lane & 31), c)]);
  };
  auto mfmas = [&](const v4i (&fa)[FM], const v4i (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  v4i fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  // One K step out of buffer `cur` (its sub-step 0 operands already in set 0):
  // while sub-step s multiplies, the operands of sub-step s + 1 are read;
  // before the last sub-step, the next step is stored into the other buffer,
  // then one barrier, then the next step's sub-step 0 operands are read while
  // the last sub-step multiplies.  Every MFMA block finds its operands
  // loaded, and one barrier per step suffices (a buffer is rewritten only
  // after the barrier that follows its last read).
  auto step = [&](int cur, int kt, u32x4 (&la)[LA], u32x4 (&lb)[LB], u32x4 (&sa)[LA], u32x4 (&sb)[LB]) {
    gload(kt + 2, la, lb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < SS; ++s) {
      if (s + 1 < SS) {
        if (s % 2 == 0) read_frags(cur, s + 1, fa1, fb1);
        else read_frags(cur, s + 1, fa0, fb0);
      } else {
        fix_tail(kt + 1, sa, sb);
        lstore(cur ^ 1, sa, sb);
        __syncthreads();
        read_frags(cur ^ 1, 0, fa0, fb0);  // SS is even: the last sub-step uses set 1
      }
      __builtin_amdgcn_sched_barrier(0);
      if (s % 2 == 0) mfmas(fa0, fb0);
      else mfmas(fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (n_idx >= K) {
    // every column is an outlier column: CA is all zeros, nothing to multiply
  } else if constexpr (DL == 0) {
    gload(0, ra0, rb0);
    gload(1, ra1, rb1);
    fix_tail(0, ra0, rb0);
    lstore(0, ra0, rb0);
    __syncthreads();
    read_frags(0, 0, fa0, fb0);
    // Two steps per trip, no branch inside: on entry buffer 0 holds step kt
    // (sub-step 0 operands in set 0) and register set 1 holds step kt + 1.
    // Steps loaded or stored past the end are re-reads of the last one and are
    // never multiplied.
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
      step(0, kt, ra0, rb0, ra1, rb1);
      step(1, kt + 1, ra1, rb1, ra0, rb0);
    }
    if (kt < nk) {  // odd step count: the last step sits in buffer 0
#pragma unroll
      for (int s = 0; s < SS; ++s) {
        if (s + 1 < SS) {
          if (s % 2 == 0) read_frags(0, s + 1, fa1, fb1);
          else read_frags(0, s + 1, fa0, fb0);
        }
        if (s % 2 == 0) mfmas(fa0, fb0);
        else mfmas(fa1, fb1);
      }
    }
  } else {
    // Each load instruction moves RPI = 1024 / BK whole tile rows (1 KiB)
    // straight into LDS (global_load_lds), lane l to bytes 16 l .. 16 l + 15
    // of it.  The swizzle is applied on the source side: lane l of the
    // instruction for rows r0 .. r0 + RPI - 1 fetches the logical chunk of row
    // r = r0 + l / CPR that tile_off<BK> stores at physical chunk l % CPR.
    // Rows past T or N re-read the last row (their results are never
    // stored).  The tile's rows span less than 2^32 bytes (256 K-byte rows,
    // K below 2^24), so 32-bit offsets reach them.  No registers, no LDS
    // store instructions;
    // with 128-byte steps every row read is one whole cache line.  Every ring
    // slot is an LDS object of its own and the loop is unrolled over the ring,
    // so the compiler can tell the slot being read from the slots still being
    // filled and waits only for the former.
    constexpr int NW = WGM * WGN;
    constexpr int RPI = 1024 / BK;                          // tile rows per load instruction
    constexpr int IA = BM / RPI / NW, IB = BN / RPI / NW;  // load instructions per wave per step
    static_assert(IA * RPI * NW == BM && IB * RPI * NW == BN, "tile rows must split evenly over the waves");
    // logical chunk stored at physical chunk p of row r (the XOR is an involution)
    auto src_chunk = [](int r, int p) { return BK == 64 ? (p ^ ((r >> 2) & 3)) : (p ^ ((r >> 1) & 7)); };
    // per-lane 32-bit offsets from the tile's first row; the wave-uniform
    // base (this tile's rows, this step) goes in scalar registers
    const int swid = __builtin_amdgcn_readfirstlane(wid);
    uint32_t oa[IA], ob[IB];
#pragma unroll
    for (int j = 0; j < IA; ++j) {
      const int r = (wid * IA + j) * RPI + lane / CPR;
      const int rr = m0 + r < T ? r : (int)(T - 1 - m0);
      oa[j] = (uint32_t)rr * (uint32_t)K + (uint32_t)(src_chunk(r, lane % CPR) << 4);
    }
#pragma unroll
    for (int j = 0; j < IB; ++j) {
      const int r = (wid * IB + j) * RPI + lane / CPR;
      const int rr = n0 + r < N ? r : (int)(N - 1 - n0);
      ob[j] = (uint32_t)rr * (uint32_t)K + (uint32_t)(src_chunk(r, lane % CPR) << 4);
    }
    const int8_t* const ta = CA + m0 * K;
    const int8_t* const tb = CB + n0 * K;
    // step kt into a ring slot; a step past the end (never multiplied)
    // re-reads the last one, still in L2
    auto issue = [&](int kt, int8_t* a_slot, int8_t* b_slot) {
      const int64_t k = (int64_t)(kt < nk ? kt : nk - 1) * BK;
#pragma unroll
      for (int j = 0; j < IA; ++j) load_lds16(ta + k + oa[j], a_slot + (swid * IA + j) * 1024);
#pragma unroll
      for (int j = 0; j < IB; ++j) load_lds16(tb + k + ob[j], b_slot + (swid * IB + j) * 1024);
    };
    auto frags = [&](const int8_t* a_slot, const int8_t* b_slot, int s, v4i (&fa)[FM], v4i (&fb)[FN]) {
      const int c = 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[i] = *reinterpret_cast<const v4i*>(a_slot + tile_off<BK>(wm * WM + i * 32 + (lane & 31), c));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[j] = *reinterpret_cast<const v4i*>(b_slot + tile_off<BK>(wn * WN + j * 32 + (lane & 31), c));
    };
    int8_t* const ra[4] = {dA0, dA1, dA2, dA3};
    int8_t* const rb[4] = {dB0, dB1, dB2, dB3};
    if constexpr (DL == 2) {
      // Two slots, two steps in flight.  Sub-step s + 1's operands are read
      // while sub-step s multiplies, one LDS read between consecutive MFMAs.
      // The step's one barrier sits before its last sub-step's MFMAs: those
      // keep the matrix cores busy across the barrier, the loads of step
      // kt + 2 into the slot just released and the reads of step kt + 1's
      // first operands.  Each wave waits for all its loads and LDS reads
      // before the barrier, so once past it every load of step kt + 1 has
      // landed and nobody reads slot kt any more.  Past the last step the
      // loads are out of range and the reads are of a slot nobody uses.
      constexpr int NFR = FM + FN;  // LDS reads per sub-step
      constexpr int NLD = IA + IB;  // loads per step
      static_assert(SS % 2 == 0, "operand sets alternate over an even number of sub-steps");
      // one step out of slot `cur` (its sub-step 0 operands already in set 0)
      auto kstep = [&](int kt, int8_t* a_cur, int8_t* b_cur, const int8_t* a_nxt, const int8_t* b_nxt) {
#pragma unroll
        for (int s = 0; s + 1 < SS; ++s) {
          if (s % 2 == 0) {
            frags(a_cur, b_cur, s + 1, fa1, fb1);
            mfmas(fa0, fb0);
          } else {
            frags(a_cur, b_cur, s + 1, fa0, fb0);
            mfmas(fa1, fb1);
          }
          interleave_mfma<FM * FN, NFR, 0>();
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0);  // own loads of step kt + 1, own reads of slot kt
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(kt + 2, a_cur, b_cur);
        frags(a_nxt, b_nxt, 0, fa0, fb0);  // the last sub-step uses set 1
        mfmas(fa1, fb1);
        interleave_mfma<FM * FN, NFR, NLD>();
        __builtin_amdgcn_sched_barrier(0);
      };
      issue(0, ra[0], rb[0]);
      issue(1, ra[1], rb[1]);
      wait_vmcnt<NLD>();
      __builtin_amdgcn_s_barrier();
      frags(ra[0], rb[0], 0, fa0, fb0);
      // nk is even on this path: the loop body is one straight block, and at
      // its head (from before the loop or from its end) only loads into
      // slot 1 are in flight while slot 0 is read
      for (int kg = 0; kg < nk; kg += 2) {
        kstep(kg, ra[0], rb[0], ra[1], rb[1]);
        kstep(kg + 1, ra[1], rb[1], ra[0], rb[0]);
      }
    } else {
#pragma unroll
      for (int st = 0; st < DL - 1; ++st) issue(st, ra[st], rb[st]);
      for (int kg = 0; kg < nk; kg += DL) {
#pragma unroll
        for (int i = 0; i < DL; ++i) {
          // all of step kg + i has landed once every wave is past the barrier,
          // and everyone has finished reading slot i - 1 (one step ago)
          wait_vmcnt<(DL - 2) * (IA + IB)>();
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
          issue(kg + i + DL - 1, ra[(i + DL - 1) % DL], rb[(i + DL - 1) % DL]);
          if (kg + i < nk) {
            frags(ra[i], rb[i], 0, fa0, fb0);
#pragma unroll
            for (int s2 = 0; s2 < SS; s2 += 2) {  // read sub-step s2 + 1 while s2 multiplies, and so on
              frags(ra[i], rb[i], s2 + 1, fa1, fb1);
              mfmas(fa0, fb0);
              if (s2 + 2 < SS) frags(ra[i], rb[i], s2 + 2, fa0, fb0);
              mfmas(fa1, fb1);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    wait_vmcnt<0>();  // the ring's last loads land before the epilogue reuses LDS
    __syncthreads();
  }

  int8_t* const ring_a[4] = {DL ? dA0 : sA_, dA1, dA2, dA3};
  int8_t* const ring_b[4] = {DL ? dB0 : sB_, dB1, dB2, dB3};
  tile_epilogue<DT, BM, BN, WGM, WGN, DL, FL, 0>(acc, m0, n0, T, N, K, SCA, SCB, bias, xo, idx, n_idx, CB, wo,
                                                 wo_chunks, out, acc_out, ring_a, ring_b, [] {});
}

// ----------------------------------------------------------- persistent ----
// 256 x 256 tiles, 128-byte steps in the 2-slot direct-load ring, whole tiles
// only (T % 256 == 0, N % 256 == 0, K % 256 == 0).  One workgroup per compute
// unit walks tiles blockIdx.x, blockIdx.x + gridDim.x, ...; with a multiple
// of 8 workgroups each keeps to one XCD, and at any moment an XCD works on
// neighbouring tiles, as a one-tile-per-workgroup grid would.  When at most
// PF_CHUNKS outlier chunks come with recovered weights in scratch, the last
// step of a tile loads the next tile's first step into the free ring slot
// and the epilogue keeps out of LDS (outlier operands straight into
// registers), so the next tile's first step arrives during the epilogue and
// its second while the stores drain.  Otherwise each tile runs on its own,
// its outlier columns staged through LDS.
constexpr int PF_CHUNKS = 4;

template <int DT, int PF>
__device__ __forceinline__ void persist_tiles(
    const int8_t* __restrict__ CA, const int8_t* __restrict__ CB, const float* __restrict__ SCA,
    const float* __restrict__ SCB, const uint16_t* __restrict__ bias, const uint16_t* __restrict__ xo,
    const int32_t* __restrict__ idx, int n_idx, uint16_t* __restrict__ out, int32_t* __restrict__ acc_out,
    int T, int N, int K, int tiles_m, int tiles_n, const uint16_t* __restrict__ wo, int wo_chunks,
    int8_t* dA0, int8_t* dA1, int8_t* dB0, int8_t* dB1) {
  constexpr int BM = 256, BN = 256, BK = 128, WGM = 4, WGN = 2, GM = 4;
  constexpr int NW = WGM * WGN, WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  constexpr int CPR = BK / 16, SS = BK / 32, RPI = 1024 / BK;
  constexpr int IA = BM / RPI / NW, IB = BN / RPI / NW;
  constexpr int NFR = FM + FN, NLD = IA + IB;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  const int swid = __builtin_amdgcn_readfirstlane(wid);
  const int nb = tiles_m * tiles_n, nk = K / BK;
  const bool int8_part = n_idx < K;  // otherwise CA is all zeros: nothing to multiply
  // the tile's rows in the ring's swizzled order; the same for every tile
  uint32_t oa[IA], ob[IB];
#pragma unroll
  for (int j = 0; j < IA; ++j) {
    const int r = (wid * IA + j) * RPI + lane / CPR;
    oa[j] = (uint32_t)r * (uint32_t)K + (uint32_t)(((lane % CPR) ^ ((r >> 1) & 7)) << 4);
  }
#pragma unroll
  for (int j = 0; j < IB; ++j) {
    const int r = (wid * IB + j) * RPI + lane / CPR;
    ob[j] = (uint32_t)r * (uint32_t)K + (uint32_t)(((lane % CPR) ^ ((r >> 1) & 7)) << 4);
  }
  auto issue = [&](const int8_t* ba, const int8_t* bb, int8_t* a_slot, int8_t* b_slot) {
    // the step's base stays a scalar pair (load = scalar base + 32-bit lane
    // offset), rather than being folded into 64-bit per-lane addresses
    asm volatile("" : "+s"(ba), "+s"(bb));
#pragma unroll
    for (int j = 0; j < IA; ++j) load_lds16(ba + oa[j], a_slot + (swid * IA + j) * 1024);
#pragma unroll
    for (int j = 0; j < IB; ++j) load_lds16(bb + ob[j], b_slot + (swid * IB + j) * 1024);
  };
  v4i fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  auto frags = [&](const int8_t* a_slot, const int8_t* b_slot, int s, v4i (&fa)[FM], v4i (&fb)[FN]) {
    const int c = 2 * s + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[i] = *reinterpret_cast<const v4i*>(a_slot + tile_off<BK>(wm * WM + i * 32 + (lane & 31), c));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[j] = *reinterpret_cast<const v4i*>(b_slot + tile_off<BK>(wn * WN + j * 32 + (lane & 31), c));
  };
  v16i acc[FM][FN];
  auto mfmas = [&](const v4i (&fa)[FM], const v4i (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  // Sub-steps 0 .. SS - 2 of the step in slot (a_cur, b_cur), whose sub-step
  // 0 operands are already in set 0; then the step's one barrier (every
  // wave's loads of the next step have landed, nobody reads this slot any
  // more), and the last sub-step's MFMAs behind it.
  auto substeps = [&](const int8_t* a_cur, const int8_t* b_cur) {
#pragma unroll
    for (int s = 0; s + 1 < SS; ++s) {
      if (s % 2 == 0) {
        frags(a_cur, b_cur, s + 1, fa1, fb1);
        mfmas(fa0, fb0);
      } else {
        frags(a_cur, b_cur, s + 1, fa0, fb0);
        mfmas(fa1, fb1);
      }
      interleave_mfma<FM * FN, NFR, 0>();
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Staged outlier chunks (PF = 0) are 64-byte rows, so one chunk's A and B
  // fit in one of the four 32 KiB LDS objects: a 4-slot ring with three
  // chunks in flight, each slot an object of its own (so the compiler can
  // tell the slot being read from those being filled).
  int8_t* const ring_a[4] = {dA0, dA1, dB0, dB1};
  int8_t* const ring_b[4] = {dA0 + BM * 64, dA1 + BM * 64, dB0 + BM * 64, dB1 + BM * 64};
  static_assert(BM * 64 + BN * 64 <= BM * BK && BN == BM, "a chunk's two operands fit one ring object");

  bool first = true;
  for (int v = blockIdx.x; v < nb; v += gridDim.x) {
    const int vn = v + gridDim.x;
    const bool more = vn < nb;
    int tm, tn;
    tile_coords<GM>(v, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int8_t* const ta = CA + m0 * K;
    const int8_t* const tb = CB + n0 * K;
    int tmn = tm, tnn = tn;
    if (more) tile_coords<GM>(vn, tiles_m, tiles_n, tmn, tnn);
    const int8_t* const tan = CA + (int64_t)tmn * BM * K;  // the next tile's rows
    const int8_t* const tbn = CB + (int64_t)tnn * BN * K;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = (v16i){0};
    if (int8_part) {
      if (!PF || first) {
        if (!first) __syncthreads();  // the previous epilogue is done with LDS
        issue(ta, tb, dA0, dB0);
        issue(ta + BK, tb + BK, dA1, dB1);
        wait_vmcnt<NLD>();
        __builtin_amdgcn_s_barrier();
      }
      // (PF, later tiles: step 0 is in slot 0 since the previous tile's last
      // barrier, step 1 on its way since its epilogue)
      frags(dA0, dB0, 0, fa0, fb0);
      for (int kg = 0; kg + 2 < nk; kg += 2) {
        substeps(dA0, dB0);
        issue(ta + (int64_t)(kg + 2) * BK, tb + (int64_t)(kg + 2) * BK, dA0, dB0);
        frags(dA1, dB1, 0, fa0, fb0);
        mfmas(fa1, fb1);
        interleave_mfma<FM * FN, NFR, NLD>();
        __builtin_amdgcn_sched_barrier(0);
        substeps(dA1, dB1);
        issue(ta + (int64_t)(kg + 3) * BK, tb + (int64_t)(kg + 3) * BK, dA1, dB1);
        frags(dA0, dB0, 0, fa0, fb0);
        mfmas(fa1, fb1);
        interleave_mfma<FM * FN, NFR, NLD>();
        __builtin_amdgcn_sched_barrier(0);
      }
      // the last two steps: slot 0 then takes the next tile's first step
      substeps(dA0, dB0);
      if (PF && more) issue(tan, tbn, dA0, dB0);
      frags(dA1, dB1, 0, fa0, fb0);
      mfmas(fa1, fb1);
      interleave_mfma<FM * FN, NFR, 0>();
      __builtin_amdgcn_sched_barrier(0);
      substeps(dA1, dB1);
      mfmas(fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!PF) __syncthreads();  // the epilogue may stage through LDS
    tile_epilogue<DT, BM, BN, WGM, WGN, 4, 1, PF>(
        acc, m0, n0, T, N, K, SCA, SCB, bias, xo, idx, n_idx, CB, wo, wo_chunks, out, acc_out, ring_a, ring_b,
        [&] {
          // the next tile's second step, once every wave is past the last
          // barrier (nobody reads slot 1 any more)
          if (PF && more && int8_part) issue(tan + BK, tbn + BK, dA1, dB1);
        });
    first = false;
  }
  wait_vmcnt<0>();  // no load into LDS outlives the workgroup
}

template <int DT>
__global__ __launch_bounds__(512) void linear_persist_kernel(
    const int8_t* __restrict__ CA, const int8_t* __restrict__ CB, const float* __restrict__ SCA,
    const float* __restrict__ SCB, const uint16_t* __restrict__ bias, const uint16_t* __restrict__ xo,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ n_idx_p, uint16_t* __restrict__ out,
    int32_t* __restrict__ acc_out, int T, int N, int K, int tiles_m, int tiles_n,
    const uint16_t* __restrict__ wo, int wo_chunks) {
  __shared__ __attribute__((aligned(16))) int8_t dA0[256 * 128], dA1[256 * 128];
  __shared__ __attribute__((aligned(16))) int8_t dB0[256 * 128], dB1[256 * 128];
  const int n_idx = *n_idx_p;
  const int n_chunks = (n_idx + 31) >> 5;
  if (n_chunks <= PF_CHUNKS && n_chunks <= wo_chunks)
    persist_tiles<DT, 1>(CA, CB, SCA, SCB, bias, xo, idx, n_idx, out, acc_out, T, N, K, tiles_m, tiles_n, wo,
                         wo_chunks, dA0, dA1, dB0, dB1);
  else
    persist_tiles<DT, 0>(CA, CB, SCA, SCB, bias, xo, idx, n_idx, out, acc_out, T, N, K, tiles_m, tiles_n, wo,
                         wo_chunks, dA0, dA1, dB0, dB1);
}

// ---------------------------------------------------------------- decode ----
// T <= 16 MB (MB <= 4), K % 16 == 0.  Workgroup = 16 output features in NW waves;
// wave w takes the 256-byte K slices w, w + NW, ... and issues all of a
// slice's loads before its first MFMA.  Lane (n, g) = (lane % 16, lane / 16)
// loads bytes 16 g + 64 u .. + 15 (u = 0 .. 3) of the slice of weight row n
// once and, for each block of 16 tokens, the matching activation bytes,
// which feed four 16x16x64 MFMAs per block (A and B use the same K
// permutation, so the dot products are exact).  So each load instruction
// reads one whole 64-byte sector of each of 16 rows; lanes that read 64
// contiguous bytes each touched four sectors per row and instruction and
// streamed at little more than half the rate.  The weight rows are streamed
// once whatever T is; N / 16 workgroups fill the chip.  The waves' int32
// tiles are summed with LDS integer atomics (exact in any order), and wave mb
// runs the epilogue of token block mb, whose operands that do not depend on
// the product it requested behind its first slice's loads.
template <int DT, int MB, int NW>
__global__ __launch_bounds__(NW * 64) void linear_decode_kernel(
    const int8_t* __restrict__ CA, const int8_t* __restrict__ CB, const float* __restrict__ SCA,
    const float* __restrict__ SCB, const uint16_t* __restrict__ bias, const uint16_t* __restrict__ xo,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ n_idx_p, uint16_t* __restrict__ out,
    int32_t* __restrict__ acc_out, int T, int N, int K) {
  static_assert(NW >= MB, "one wave per token block in the epilogue");
  __shared__ int32_t red[MB][4][64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < MB * 256; i += NW * 64) (&red[0][0][0])[i] = 0;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int nr = lane & 15, g = lane >> 4;
  const int nss = (K + 255) >> 8;
  v4i acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = (v4i){0, 0, 0, 0};
  // Buffer loads: a read outside its resource returns zeros, so weight rows
  // past N, token rows past T and columns past K (offset pushed out of range)
  // need no branch.  A per-lane condition around each load became a branch,
  // and the compiler waited for every load in flight before each one: one
  // memory round trip per block of 16 tokens.
  constexpr int OOB = 0x7FFFFFF0;  // beyond any resource here (sizes < 2^31 bytes)
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(CB + n0 * (int64_t)K), 0, (N - (int)n0 < 16 ? N - (int)n0 : 16) * K, 0x00020000);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)CA, 0, T * K, 0x00020000);

  // The epilogue's operands that do not depend on the product are requested
  // right behind the first slice's loads, so they arrive during the stream:
  // the column's scale and bias, the tokens' scales, and the weight bytes and
  // activations of the first eight outlier columns (indices clamped into
  // range; entries past n_idx are read but never used, and with no gathered
  // columns the activation reads are out of their resource and return 0).
  // Wave w < MB requests those of token block w.
  const int mbe = w < MB ? w : MB - 1;
  // (the outlier columns only where the registers allow: 16 waves hold at
  // most 128 each)
  constexpr bool PF_OUT = NW <= 8 || MB <= 2;
  const int64_t col = n0 + nr;
  const int64_t colc = col < N ? col : (int64_t)N - 1;
  const uint16_t* bsrc = (bias != nullptr) ? bias : reinterpret_cast<const uint16_t*>(SCB);
  const uint32_t bmask = (bias != nullptr) ? 0xFFFFu : 0u;
  int tt[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) tt[r] = 16 * mbe + 4 * g + r;
  float scb, sca[4];
  uint32_t braw;
  int8_t cb0[8];
  u32x4 xq0[4];
  auto prefetch_epilogue = [&]() {
    scb = SCB[colc];
    braw = bsrc[colc];
#pragma unroll
    for (int r = 0; r < 4; ++r) sca[r] = SCA[tt[r] < T ? tt[r] : T - 1];
    if constexpr (!PF_OUT) return;
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // idx holds K >= 16 entries
      const int c = idx[j];
      cb0[j] = CB[colc * K + (c < 0 ? 0 : (c >= K ? K - 1 : c))];
    }
    // chunk 0 of the gathered activations: row t, columns 0 .. 7 in 16 bytes
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(xo != nullptr ? xo : reinterpret_cast<const uint16_t*>(CB)), 0, xo != nullptr ? T * 64 : 0,
        0x00020000);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      xq0[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (tt[r] < T ? tt[r] : T - 1) * 64, 0, 0));
  };

  // Slices per pass: two where the registers allow (a second slice past the
  // end reads out of range, i.e. zeros), so that at K = 4096 each wave's
  // loads all go out at once.
  constexpr int SL = (MB == 4 && NW == 8) ? 2 : 1;
  for (int s = w; s < nss; s += SL * NW) {
    u32x4 b[SL][4];
    u32x4 a[SL][MB][4];
#pragma unroll
    for (int l = 0; l < SL; ++l) {
      const int kb = (s + l * NW) * 256 + g * 16;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = kb + 64 * u;
        b[l][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, k < K ? nr * K + k : OOB, 0, 2));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k = kb + 64 * u;
          a[l][mb][u] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, k < K ? (16 * mb + nr) * K + k : OOB, 0, 0));
        }
    }
    if (s == w && w < MB) prefetch_epilogue();
    // every load of the pass in flight before the first MFMA waits for one
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int l = 0; l < SL; ++l)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, a[l][mb][u]),
                                                          __builtin_bit_cast(v4i, b[l][u]), acc[mb], 0, 0, 0);
  }
  if (w >= nss && w < MB) prefetch_epilogue();  // (K < 256 NW: a wave without a slice)
  __syncthreads();  // the zeroed sums are in place
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) atomicAdd(&red[mb][r][lane], acc[mb][r]);
  __syncthreads();
  if (w >= MB) return;
  const int mb = w;  // this wave's block of 16 tokens
  v4i sum;
#pragma unroll
  for (int r = 0; r < 4; ++r) sum[r] = red[mb][r][lane];

  // 16x16 accumulator layout: lane holds column lane % 16, rows 4 * (lane / 16) + r
  // of its block of 16 tokens.
  const int n_idx = *n_idx_p;
  if (col >= N) return;
  // Outlier columns in groups of eight, products added in column order; the
  // first group from the registers filled above, the others with all of a
  // group's loads out before any of its arithmetic (indices clamped into
  // range, surplus products zeroed: loads behind conditions or next to the
  // division's branch are waited on one by one).
  float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (PF_OUT) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float wv = to_f32<DT>(recover_w<DT>(cb0[j], scb));
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (j < n_idx && tt[r] < T) o[r] += to_f32<DT>((xq0[r][j >> 1] >> (16 * (j & 1))) & 0xFFFFu) * wv;
    }
  }
  for (int p0 = PF_OUT ? 8 : 0; p0 < n_idx; p0 += 8) {
    int8_t cb[8];
    uint16_t xb[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + j < n_idx ? p0 + j : n_idx - 1;
      cb[j] = CB[col * K + idx[p]];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        xb[j][r] = xo[((int64_t)(p >> 5) * T + (tt[r] < T ? tt[r] : T - 1)) * 32 + (p & 31)];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool okp = p0 + j < n_idx;
      const float wv = to_f32<DT>(recover_w<DT>(cb[j], scb));
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (okp && tt[r] < T) o[r] += to_f32<DT>(xb[j][r]) * wv;
    }
  }
  const float bv = to_f32<DT>(braw & bmask);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = tt[r];
    if (t >= T) continue;
    if (acc_out != nullptr) acc_out[(int64_t)t * N + col] = sum[r];
    const float d = (float)sum[r] * (sca[r] * (scb * (1.0f / 16129.0f)));
    out[(int64_t)t * N + col] = from_f32<DT>(d + o[r] + bv);
  }
}

template <int DT, int BM, int BN, int BK, int WGM, int WGN, int GM = 8, int DL = 0>
static hipError_t launch_tile(const LinearArgs& a, hipStream_t s) {
  const int tiles_m = (int)((a.T + BM - 1) / BM), tiles_n = (int)((a.N + BN - 1) / BN);
  const int nb = tiles_m * tiles_n;
  // whole tiles only: the epilogue without bounds checks
  const bool full = (a.T % BM) == 0 && (a.N % BN) == 0 && (a.N % 2) == 0;
  decltype(&linear_tile_kernel<DT, BM, BN, 0, BK, WGM, WGN, GM, DL, 0>) k;
  if constexpr (DL != 0) {  // direct-load configurations need K a multiple of the step
    if ((a.K % BK) != 0) return hipErrorInvalidValue;
    if (DL == 2 && (a.K / BK) % 2 != 0) return hipErrorInvalidValue;  // the 2-slot loop runs steps in pairs
    k = full ? linear_tile_kernel<DT, BM, BN, 0, BK, WGM, WGN, GM, DL, 1>
             : linear_tile_kernel<DT, BM, BN, 0, BK, WGM, WGN, GM, DL, 0>;
  } else {
    k = (a.K % BK) == 0 ? (full ? linear_tile_kernel<DT, BM, BN, 0, BK, WGM, WGN, GM, 0, 1>
                                : linear_tile_kernel<DT, BM, BN, 0, BK, WGM, WGN, GM, 0, 0>)
        : (a.K % 16) == 0 ? linear_tile_kernel<DT, BM, BN, 1, BK, WGM, WGN, GM, 0, 0>
        : (a.K % 8) == 0  ? linear_tile_kernel<DT, BM, BN, 3, BK, WGM, WGN, GM, 0, 0>
        : (a.K % 4) == 0  ? linear_tile_kernel<DT, BM, BN, 4, BK, WGM, WGN, GM, 0, 0>
                          : linear_tile_kernel<DT, BM, BN, 2, BK, WGM, WGN, GM, 0, 0>;
  }
  k<<<dim3(nb), dim3(64 * WGM * WGN), 0, s>>>(a.CA, a.CB, a.SCA, a.SCB, static_cast<const uint16_t*>(a.bias),
                                   static_cast<const uint16_t*>(a.xo), a.idx, a.n_idx,
                                   static_cast<uint16_t*>(a.out), a.acc, (int)a.T, (int)a.N, (int)a.K,
                                   tiles_m, tiles_n, static_cast<const uint16_t*>(a.wo), a.wo ? a.wo_chunks : 0);
  return hipGetLastError();
}

namespace {
int g_gemm_cus[64];  // compute units per device, looked up once
}

static hipError_t compute_units(int& cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int& c = g_gemm_cus[dev & 63];
  if (c <= 0) {
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  cus = c;
  return hipSuccess;
}

template <int DT>
static hipError_t launch_linear_t(const LinearArgs& a, hipStream_t s) {
  if (stream_gemm_route(a.T, a.N, a.K)) {
    // weight-streaming kernel: every weight row read once, N / 16 workgroups
    const int nb = (int)((a.N + 15) / 16);
    // 16 waves (one 256-byte slice each at K = 4096) while a wave's
    // fragments and prefetched epilogue operands fit in 128 registers, else 8
    decltype(&linear_decode_kernel<DT, 1, 16>) k = a.T <= 16 ? linear_decode_kernel<DT, 1, 16>
                                                  : a.T <= 32 ? linear_decode_kernel<DT, 2, 16>
                                                              : linear_decode_kernel<DT, 4, 8>;
    k<<<dim3(nb), dim3(a.T <= 32 ? 16 * 64 : 8 * 64), 0, s>>>(
        a.CA, a.CB, a.SCA, a.SCB, static_cast<const uint16_t*>(a.bias), static_cast<const uint16_t*>(a.xo),
        a.idx, a.n_idx, static_cast<uint16_t*>(a.out), a.acc, (int)a.T, (int)a.N, (int)a.K);
    return hipGetLastError();
  }
  // 256 x 256 tiles once there are enough of them to fill half the chip;
  // with fewer, smaller tiles finish sooner (T = 512-1024, N = K = 4096:
  // 46-47 -> 22-30 us; T = 512, N = 11008: 46.8 -> 41.3 us; from 129 tiles of
  // 256 x 256 on, those win)
  int cus = 0;
  {
    const hipError_t e = compute_units(cus);
    if (e != hipSuccess) return e;
  }
  const int64_t t256 = ((a.T + 255) / 256) * ((a.N + 255) / 256);
  if (a.T >= 512 && a.N >= 512 && a.K < (1 << 24) && 2 * t256 >= cus) {
    // whole 256 x 256 tiles: one workgroup per compute unit walks its tiles
    if (a.T % 256 == 0 && a.N % 256 == 0 && a.K % 256 == 0) {
      const int tiles_m = (int)(a.T / 256), tiles_n = (int)(a.N / 256);
      const int nb = tiles_m * tiles_n;
      const int G = nb < cus ? nb : cus;
      linear_persist_kernel<DT><<<dim3(G), dim3(512), 0, s>>>(
          a.CA, a.CB, a.SCA, a.SCB, static_cast<const uint16_t*>(a.bias), static_cast<const uint16_t*>(a.xo), a.idx,
          a.n_idx, static_cast<uint16_t*>(a.out), a.acc, (int)a.T, (int)a.N, (int)a.K, tiles_m, tiles_n,
          static_cast<const uint16_t*>(a.wo), a.wo ? a.wo_chunks : 0);
      return hipGetLastError();
    }
    // direct loads: 128-byte steps in a 2-slot ring (whole cache lines per
    // row), else 64-byte steps in a 4-slot ring, else register staging
    if (a.K % 256 == 0) return launch_tile<DT, 256, 256, 128, 4, 2, 4, 2>(a, s);  // an even step count
    if (a.K % 64 == 0) return launch_tile<DT, 256, 256, 64, 4, 2, 4, 4>(a, s);
    return launch_tile<DT, 256, 256, 64, 4, 2, 4, 0>(a, s);
  }
  // 128 x 128 tiles unless they leave most of the chip idle; then 64 x 64
  const int64_t t128 = ((a.T + 127) / 128) * ((a.N + 127) / 128);
  // (both take K straight into a 4-slot LDS ring when K % 64 == 0: three
  // steps in flight rather than two register sets; 64 x 64 at T = 129-256,
  // K = N = 4096: 40 -> 31-33 us, and with 128-byte steps when K % 128 == 0
  // 27-29 us)
  if (t128 < 256)
    return (a.K % 128) == 0 ? launch_tile<DT, 64, 64, 128, 2, 2, 8, 4>(a, s)
           : (a.K % 64) == 0 ? launch_tile<DT, 64, 64, 64, 2, 2, 8, 4>(a, s)
                             : launch_tile<DT, 64, 64, 64, 2, 2>(a, s);
  return (a.K % 64) == 0 ? launch_tile<DT, 128, 128, 64, 2, 2, 8, 4>(a, s) : launch_tile<DT, 128, 128, 64, 2, 2>(a, s);
}

hipError_t launch_linear_gemm(const LinearArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  return a.dt == DT_F16 ? launch_linear_t<DT_F16>(a, s) : launch_linear_t<DT_BF16>(a, s);
}

}  // namespace lli8
