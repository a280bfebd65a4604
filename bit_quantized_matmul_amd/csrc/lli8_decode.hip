// Fused decode path (T <= 16, K <= 4096): the whole LLM.int8() forward in one
// launch, with no workgroup ever waiting on another.
//
// For a handful of tokens the int8 weight stream (N x K bytes) is the only
// real HBM traffic; separate launches for the outlier scan, the activation
// quantiser and the GEMM each cost more than the stream itself, and so does a
// grid-wide barrier.  So every workgroup derives the activation split on its
// own (X is at most 16 x 4096 values and sits in L2 after the first touch),
// while its weight rows are already on their way:
//   1. thread c loads the 8-column chunk c of all 16 token rows (each wave
//      load is 1 KiB of one row, fully coalesced), then the 16 weight rows of
//      its block in the MFMA operand layout;
//   2. a column is an outlier when some |x| > threshold ("Core idea of
//      LLM.int8()" step 1): the thread holds every row of its columns, so the
//      flags need no exchange; the row absmax over the other columns is SCA
//      ("Quantization mechanics", absmax bullet), reduced across the
//      workgroup with packed 16-bit maxima;
//   3. codes round(fl32(|x| * fl32(127 / SCA))) with halves away from zero,
//      signed, 0 on outlier columns, go to LDS row-major (XOR-swizzled);
//   4. v_mfma_i32_16x16x64_i8 with A read back from LDS, the eight waves'
//      int32 tiles summed in a fixed order, then the epilogue:
//      dequantisation, the 16-bit outlier product against (CB * SCB) / 127
//      ("Integration into transformers"), bias, one rounding.  The outlier
//      columns' X values and recovered weights come from registers.
// Side outputs (CA, SCA, bitmap, idx, n_idx) are written by all workgroups
// together (CA) or by workgroup 0 (the small ones).
#include "lli8_device.h"
#include "lli8_internal.h"

namespace lli8 {

constexpr int FD_CW = 8;                      // activation waves
constexpr int FD_LW = 4;                      // weight waves
constexpr int FD_THREADS = (FD_CW + FD_LW) * 64;  // 768: three waves per SIMD
constexpr int FD_MAXK = FD_CW * 64 * 8;       // 4096: one 8-column chunk per activation thread
constexpr int FD_MAXW = FD_MAXK / 32;         // bitmap words
constexpr int FD_MPL = FD_MAXK / FD_LW / 64;  // MFMAs (64 columns each) per weight wave: 16
constexpr int FD_OUT_LDS = 64;                // outlier columns staged in LDS; more read global memory
// An arrival count in LDS, for a meeting that the weight waves must not
// join: a wave issuing its weight loads can stall at issue for as long as
// the memory pipeline is full, and a workgroup barrier would hold every
// other wave behind it.  LDS operations of one wave are performed in
// order, so the data a wave writes before its count is seen by any wave
// that has read the count; the empty asm statements keep the compiler from
// moving LDS accesses across the count operations.
__device__ __forceinline__ void lds_arrive(uint32_t* cnt, int lane) {
  asm volatile("" ::: "memory");
  if (lane == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void lds_wait_count(uint32_t* cnt, uint32_t n) {
  while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < n) __builtin_amdgcn_s_sleep(1);
  asm volatile("" ::: "memory");
}

// Cross-lane moves without LDS: DPP within a row of 16 lanes, the gfx950
// permlane swaps across rows.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_QUAD_XOR1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int DPP_QUAD_XOR2 = 0x4E;    // quad_perm [2, 3, 0, 1]
constexpr int DPP_ROW_ROR8 = 0x128;    // lane l <- lane l ^ 8 within its row
constexpr int DPP_HALF_MIRROR = 0x141;  // lane l <- lane 7 - l within its 8-lane half row

// Packed 16-bit maxima of eight dwords per lane, reduced over the wave.  The
// result for dword p sits in lanes 8p .. 8p + 7.  Each step halves the data
// each lane carries: dwords p and p + 4 trade halves of the wave (permlane32
// swap), then p and p + 2 trade rows (permlane16 swap), then p and p + 1
// trade half rows, and the last three steps finish within 8 lanes.
__device__ __forceinline__ uint32_t wave_max8_u16x2(const uint32_t (&pr)[8], int lane) {
  uint32_t q4[4], q2[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(pr[i], pr[i + 4], false, false);
    q4[i] = pk_max_u16(r[0], r[1]);  // lanes 0-31: dword i, lanes 32-63: dword i + 4
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(q4[i], q4[i + 2], false, false);
    q2[i] = pk_max_u16(r[0], r[1]);  // even rows: dword of q4[i], odd rows: of q4[i + 2]
  }
  const bool b3 = (lane & 8) != 0;
  const uint32_t send = b3 ? q2[0] : q2[1];
  uint32_t q1 = pk_max_u16(b3 ? q2[1] : q2[0], dpp<DPP_ROW_ROR8>(send));
  q1 = pk_max_u16(q1, dpp<DPP_HALF_MIRROR>(q1));
  q1 = pk_max_u16(q1, dpp<DPP_QUAD_XOR1>(q1));
  q1 = pk_max_u16(q1, dpp<DPP_QUAD_XOR2>(q1));
  return q1;
}

// Packed 16-bit maxima over the lanes that share (lane & 7): lane l ^ 8
// within its row, then across rows and halves of the wave.
__device__ __forceinline__ uint32_t wave_max_by8_u16x2(uint32_t v) {
  v = pk_max_u16(v, dpp<DPP_ROW_ROR8>(v));
  {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = pk_max_u16(r[0], r[1]);
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = pk_max_u16(r[0], r[1]);
  }
  return v;
}

// Exclusive prefix counts of outlier bitmap words 2l and 2l + 1 (W <= 128)
// packed as two 16-bit halves in lane l, and the total count; the two words
// themselves (0 past W) are left in w0, w1.
__device__ __forceinline__ uint32_t bitmap_prefix(const uint32_t* s_bm, int W, int lane, int& total, uint32_t& w0,
                                                  uint32_t& w1) {
  w0 = (2 * lane < W) ? s_bm[2 * lane] : 0u;
  w1 = (2 * lane + 1 < W) ? s_bm[2 * lane + 1] : 0u;
  const int cnt = __popc(w0) + __popc(w1);
  const int incl = wave_incl_scan(cnt);
  total = __builtin_amdgcn_readlane(incl, 63);
  const uint32_t p0 = (uint32_t)(incl - cnt);
  return p0 | ((p0 + (uint32_t)__popc(w0)) << 16);
}

// LDS byte offset of 16-byte code chunk ch (0..255) of token row t.  Rows are
// FD_MAXK bytes; the XOR gives the 16 rows that one MFMA operand read touches
// 16 distinct 16-byte bank groups, and keeps the row-wise writes
// conflict-free.
__device__ __forceinline__ int code_off(int t, int ch) { return t * FD_MAXK + ((ch ^ t) << 4); }

template <int DT>
__global__ __launch_bounds__(FD_THREADS, 1) void decode_fused_kernel(
    const uint16_t* __restrict__ X, int T, int K, int N, float tau, const int8_t* __restrict__ CB,
    const float* __restrict__ SCB, const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
    int8_t* __restrict__ CA, float* __restrict__ SCA, uint32_t* __restrict__ bitmap,
    int32_t* __restrict__ idx, int32_t* __restrict__ n_idx_out, int32_t* __restrict__ acc_out) {
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[16 * FD_MAXK];
  __shared__ uint32_t s_bm[FD_MAXW];
  __shared__ uint32_t s_pre[FD_MAXW];
  __shared__ int32_t s_idx[FD_MAXK];
  __shared__ uint32_t s_wmax[FD_CW][8];  // per activation wave: row maxima, two rows per dword
  __shared__ uint32_t s_wany[FD_CW];
  __shared__ float s_sca[16];
  __shared__ int s_nout;
  __shared__ v4i s_red[FD_LW][64];  // each weight wave's int32 partial tile
  __shared__ uint32_t s_b1;  // activation waves past their statistics
  __shared__ uint32_t s_b2;  // activation waves done with the first block's outlier operands
  __shared__ float s_owv[FD_OUT_LDS][16];  // recovered weights of the outlier columns, this block
  __shared__ u32x4 s_oxc[FD_OUT_LDS][16];  // the 8-column chunk of each outlier column, all 16 rows
  __shared__ int s_oxe[FD_OUT_LDS];        // the outlier column's place in its chunk
  __shared__ float s_osum[16][16];         // first block's 16-bit outlier product, [token][feature]
  __shared__ float s_oxv[FD_OUT_LDS][16];  // outlier columns' X values, [column][token]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = gridDim.x, wg = blockIdx.x;
  const int nblk = (N + 15) >> 4;
  const int W = (K + 31) >> 5;
  const int blk0 = wg;  // the grid never exceeds the number of blocks

  // Both roles pass the same sequence of workgroup barriers: B0 (the
  // arrival count is zero, and the activation waves' X loads are issued,
  // not waited for, so they reach memory ahead of the weight stream), B2
  // (codes, outlier index list, X values and recovered weights of the
  // outlier columns, row scales), then per block B3 (partial tiles) and B4
  // (epilogue done).  B1 (per-wave row maxima, bitmap) is an arrival count
  // of the activation waves alone; the weight waves issue their stream
  // right after B0 and read the count only once it is issued.
  if (tid == 0) {
    s_b1 = 0u;
    s_b2 = 0u;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): zeroed before B0
  }
  if (w < FD_CW) {
    // ------------------------------------------------ activation waves ----
    const uint32_t t16 = magnitude_threshold<DT>(tau);  // |x| > tau  <=>  (bits & 0x7FFF) > t16
    // 1. chunk c = tid, columns 8c .. 8c + 7, all 16 rows.  Loads are
    // unconditional at clamped in-range addresses, so the compiler counts them
    // in order.  Rows beyond T repeat row T - 1 (harmless: they change no
    // column maximum and only feed accumulator rows that are never stored);
    // chunks beyond K are masked where their values are used.
    const int c = tid;
    const bool cok = 8 * c < K;
    u32x4 xr[16];
    {
      const uint16_t* xc = X + (cok ? 8 * c : 0);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int tt = t < T ? t : T - 1;
        xr[t] = *reinterpret_cast<const u32x4*>(xc + (int64_t)tt * K);
      }
    }
    __builtin_amdgcn_s_barrier();  // B0 (no wait for the X loads)

    // 2. statistics: column maxima of the 15-bit magnitudes over the 16 rows
    // (two columns per dword) and, in the same pass, each row's maximum over
    // this chunk.
    uint32_t cm[4] = {0u, 0u, 0u, 0u};
    uint32_t rm[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      uint32_t a[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        a[d] = xr[t][d] & 0x7FFF7FFFu;
        cm[d] = pk_max_u16(cm[d], a[d]);
      }
      rm[t] = pk_max_u16(pk_max_u16(a[0], a[1]), pk_max_u16(a[2], a[3]));
    }
    const uint32_t f8 = cok ? flags8(cm, t16) : 0u;  // bit e: column 8c + e is an outlier column
    // bitmap word c / 4 from the four lanes of a quad, held by all four; no atomics
    uint32_t wword = f8 << (8 * (c & 3));
    wword |= dpp<DPP_QUAD_XOR1>(wword);
    wword |= dpp<DPP_QUAD_XOR2>(wword);
    if ((c & 3) == 0 && cok) s_bm[c >> 2] = wword;
    const uint64_t anyw = __ballot(f8 != 0u);
    if (lane == 0) s_wany[w] = anyw != 0 ? 1u : 0u;
    if (!cok) {
#pragma unroll
      for (int t = 0; t < 16; ++t) rm[t] = 0u;
    }
    if (f8 != 0u) {  // rare: leave this chunk's outlier columns out of the row maxima
      uint32_t km[4];
#pragma unroll
      for (int d = 0; d < 4; ++d)
        km[d] = ((((f8 >> (2 * d)) & 1u) ? 0u : 0x7FFFu) | (((f8 >> (2 * d + 1)) & 1u) ? 0u : 0x7FFF0000u));
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const u32x4& v = xr[t];
        rm[t] = pk_max_u16(pk_max_u16(v[0] & km[0], v[1] & km[1]), pk_max_u16(v[2] & km[2], v[3] & km[3]));
      }
    }
    {  // two rows per dword, then over the wave: lanes 8p .. 8p + 7 get rows 2p, 2p + 1
      uint32_t pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pr[i] = pk_max_u16(__builtin_amdgcn_perm(rm[2 * i + 1], rm[2 * i], 0x05040100u),
                           __builtin_amdgcn_perm(rm[2 * i + 1], rm[2 * i], 0x07060302u));
      const uint32_t q1 = wave_max8_u16x2(pr, lane);
      if ((lane & 7) == 0) s_wmax[w][lane >> 3] = q1;
    }
    lds_arrive(&s_b1, lane);  // B1 among the activation waves
    lds_wait_count(&s_b1, FD_CW);

    // row scales, in every wave: lane l takes rows 2p, 2p + 1 with p = l & 7
    const bool any = __ballot(lane < FD_CW && s_wany[lane & (FD_CW - 1)] != 0u) != 0;
    const uint32_t rmax2 = wave_max_by8_u16x2(s_wmax[lane >> 3][lane & 7]);
    const float sca_lo = to_f32<DT>(rmax2 & 0xFFFFu), sca_hi = to_f32<DT>(rmax2 >> 16);  // exact row absmax
    const float sf_lo = row_factor(sca_lo);
    const float sf_hi = row_factor(sca_hi);
    if (w == 0 && lane < 8) {
      s_sca[2 * lane] = sca_lo;
      s_sca[2 * lane + 1] = sca_hi;
    }

    // 3. codes into LDS
    {
      const uint32_t ok = cok ? 0xFFFFFFFFu : 0u;  // chunks beyond K get zero codes
      const uint32_t z0 = ~byte_mask4(f8) & ok, z1 = ~byte_mask4(f8 >> 4) & ok;  // and outlier columns
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float sf = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
            __builtin_bit_cast(int, (t & 1) ? sf_hi : sf_lo), t >> 1));
        const u32x4& v = xr[t];
        u32x2 cw;
        const float am = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
            __builtin_bit_cast(int, (t & 1) ? sca_hi : sca_lo), t >> 1));
        if (DT == DT_BF16 && tiny_absmax(am)) {  // uniform: row t's absmax
          constexpr bool P = DT == DT_BF16;
          cw[0] = pack_codes16(code_pair16<DT, P>(v[0], sf), code_pair16<DT, P>(v[1], sf)) & z0;
          cw[1] = pack_codes16(code_pair16<DT, P>(v[2], sf), code_pair16<DT, P>(v[3], sf)) & z1;
        } else {
          cw[0] = pack_codes16(code_pair16<DT>(v[0], sf), code_pair16<DT>(v[1], sf)) & z0;
          cw[1] = pack_codes16(code_pair16<DT>(v[2], sf), code_pair16<DT>(v[3], sf)) & z1;
        }
        *reinterpret_cast<u32x2*>(&s_codes[code_off(t, c >> 1) + (c & 1) * 8]) = cw;
      }
    }
    int n_out = 0;
    if (any) {  // this chunk's outlier columns: their index, and the chunk's X rows
      uint32_t bw0, bw1;
      const uint32_t pp = bitmap_prefix(s_bm, W, lane, n_out, bw0, bw1);
      const int word = c >> 2;  // prefix of this chunk's bitmap word, from lane word / 2 of this wave
      const uint32_t pw = (uint32_t)__shfl((int)pp, (word >> 1) & 63, WAVE);
      const uint32_t pre = (word & 1) ? (pw >> 16) : (pw & 0xFFFFu);
      uint32_t f = f8;
      while (f) {
        const int e = __builtin_ctz(f);
        f &= f - 1u;
        const int col = 8 * c + e;
        const int rank = (int)pre + __popc(wword & ((1u << (col & 31)) - 1u));
        s_idx[rank] = col;
        if (rank < FD_OUT_LDS) {  // whole rows of the chunk, no per-row selects; the reader picks value e
          s_oxe[rank] = e;
#pragma unroll
          for (int t = 0; t < 16; ++t) s_oxc[rank][t] = xr[t];
        }
      }
    }
    __syncthreads();  // B2

    // the first block's 16-bit outlier product over the staged columns while
    // the weight waves run the int8 products; weight wave 0 reads it after
    // B3.  First each X value once (not once per output), then, after the
    // activation waves meet, one (token, feature) per thread over the
    // recovered weights the weight waves staged, summed in column order.
    if (any) {
      const int n_lds = min(n_out, FD_OUT_LDS);
      for (int i = tid; i < 16 * n_lds; i += FD_CW * 64) {
        const int p = i >> 4, j = i & 15;
        s_oxv[p][j] = to_f32<DT>(half_bits(s_oxc[p][j], s_oxe[p]));
      }
      lds_arrive(&s_b2, lane);
      lds_wait_count(&s_b2, FD_CW);
      if (tid < 256) {
        const int t = tid >> 4, n = tid & 15;
        float o = 0.0f;
        for (int p0 = 0; p0 < n_lds; p0 += 8) {  // eight columns' operands read together, summed in order
          float xv[8], wv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int p = min(p0 + i, n_lds - 1);
            xv[i] = s_oxv[p][t];
            wv[i] = s_owv[p][n];
          }
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (p0 + i < n_lds) o += xv[i] * wv[i];
        }
        s_osum[t][n] = o;
      }
    }

    // side outputs: CA shared out over the grid (from activation wave 4 on,
    // the waves that sum no outlier product), the small ones by workgroup 0
    {
      const int cpr = K >> 4;  // 16-byte code chunks per row
      const int units = T * cpr;
      const int ts = (tid + 256) & (FD_CW * 64 - 1);
      for (int u = wg + G * ts; u < units; u += G * (FD_CW * 64)) {
        const int t = u / cpr, ch = u - t * cpr;
        *reinterpret_cast<v4i*>(CA + (int64_t)t * K + ch * 16) = *reinterpret_cast<const v4i*>(&s_codes[code_off(t, ch)]);
      }
    }
    if (wg == 0) {
      if (tid < T) SCA[tid] = s_sca[tid];
      for (int i = tid; i < W; i += FD_CW * 64) bitmap[i] = s_bm[i];
      for (int p = tid; p < n_out; p += FD_CW * 64) idx[p] = s_idx[p];
      if (tid == 0) *n_idx_out = n_out;
    }
    for (int blk = blk0; blk < nblk; blk += G) {
      __syncthreads();  // B3
      __syncthreads();  // B4
    }
  } else {
    // ---------------------------------------------------- weight waves ----
    // Their loads may wait for queue space in the memory pipeline for as long
    // as the weight stream takes; no other work waits behind them.
    const int lw = w - FD_CW;
    const int nr = lane & 15, q = lane >> 4;
    // weight rows of a block in the MFMA B layout: lane (n, q) of weight wave
    // lw holds CB[n][k0 .. k0 + 16) for k0 = 1024 lw + 64 m + 16 q, m = 0 ..
    // 15.  Buffer loads over the block's rows: a read past the last row of CB
    // returns zeros, and reads past K within a row only meet zero codes.
    u32x4 b[FD_MPL];
    float scb_n, bias_n;  // scale and bias of feature nr of the block
    const int vo = nr * K + lw * 1024 + q * 16;
    auto load_cb = [&](int blk) {
      const int rows = min(16, N - blk * 16);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(CB + (int64_t)blk * 16 * K), 0, rows * K, 0x00020000);
#pragma unroll
      for (int m = 0; m < FD_MPL; ++m)
        b[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo + m * 64, 0, 2));
      // unconditional loads at in-range addresses (a branch around them would
      // make the compiler wait for every load in flight); with no bias the
      // load reads SCB and is discarded
      const int64_t n = (int64_t)blk * 16 + nr;
      const int64_t cc = n < N ? n : (int64_t)N - 1;
      const uint16_t* bsrc = (bias != nullptr) ? bias : reinterpret_cast<const uint16_t*>(SCB);
      const uint32_t bmask = (bias != nullptr) ? 0xFFFFu : 0u;
      scb_n = SCB[cc];
      bias_n = to_f32<DT>(bsrc[cc] & bmask);
    };
    // Recovered weights dtype(fl32(fl32(CB * SCB) / 127)) of the outlier
    // columns of this block, from registers, placed by rank; the bitmap words
    // come from the prefix pass's registers (lane L holds words 2L and
    // 2L + 1), so no LDS read waits in this chain.
    auto stage_outlier_weights = [&](uint32_t pp, uint32_t bw0, uint32_t bw1) {
#pragma unroll
      for (int m = 0; m < FD_MPL; ++m) {
        const int L = lw * 16 + m;  // the lane with this m's two words (64 columns)
        const uint32_t wa = (uint32_t)__builtin_amdgcn_readlane((int)bw0, L);
        const uint32_t wb = (uint32_t)__builtin_amdgcn_readlane((int)bw1, L);
        if ((wa | wb) == 0u) continue;  // no outlier column among these 64
        const int k0 = lw * 1024 + m * 64 + q * 16;
        const uint32_t wd = (q >> 1) ? wb : wa;  // word k0 / 32 (0 past K)
        uint32_t bits = (wd >> (k0 & 31)) & 0xFFFFu;
        const uint32_t pw = (uint32_t)__builtin_amdgcn_readlane((int)pp, L);
        const uint32_t pre = (q >> 1) ? (pw >> 16) : (pw & 0xFFFFu);
        while (bits) {
          const int e = __builtin_ctz(bits);
          bits &= bits - 1u;
          const int rank = (int)pre + __popc(wd & ((1u << ((k0 & 31) + e)) - 1u));
          if (rank < FD_OUT_LDS) {
            const int8_t cb = (int8_t)((b[m][e >> 2] >> (8 * (e & 3))) & 0xFFu);
            s_owv[rank][nr] = to_f32<DT>(from_f32<DT>(div127((float)cb * scb_n)));
          }
        }
      }
    };
    // The weight loads are issued right after B0, behind the activation
    // waves' X loads; a wave issuing them stalls until queue space frees up,
    // so the weight waves wait for the activation waves (B1) only after that
    // (issuing them later, once some or all activation waves hold their X
    // rows, measured the same).
    __builtin_amdgcn_s_barrier();  // B0
    load_cb(blk0);
    lds_wait_count(&s_b1, FD_CW);  // B1: bitmap and row maxima are in LDS
    const bool any = __ballot(lane < FD_CW && s_wany[lane & (FD_CW - 1)] != 0u) != 0;
    int n_out = 0;
    uint32_t pp = 0u, bw0 = 0u, bw1 = 0u;
    if (any) {
      pp = bitmap_prefix(s_bm, W, lane, n_out, bw0, bw1);
      stage_outlier_weights(pp, bw0, bw1);
    }
    const int n_lds = min(n_out, FD_OUT_LDS);
    __syncthreads();  // B2

    // 4. int8 products and epilogue, 16 output features at a time
    for (int blk = blk0; blk < nblk; blk += G) {
      if (blk != blk0) {
        load_cb(blk);
        if (any) stage_outlier_weights(pp, bw0, bw1);
      }
      // 16x16 layout: lane holds feature nr = lane % 16, tokens 4 q + r
      // (r = 0 .. 3).  After B3 weight wave lw finishes token 4 q + lw of
      // every lane's group: the four waves' int32 partials summed (exact in
      // any order), its 16-bit outlier product, the epilogue.  The
      // activation waves sum the first block's outlier product between B2 and
      // B3; for later blocks each weight wave sums its token's itself over
      // the recovered weights all four staged after B4 (rows beyond T hold
      // row T - 1: they only feed outputs never stored).
      auto outlier_sum = [&](int t) {
        float o = 0.0f;
        for (int p = 0; p < n_lds; ++p)
          o += to_f32<DT>(reinterpret_cast<const uint16_t*>(&s_oxc[p][t])[s_oxe[p]]) * s_owv[p][nr];
        return o;
      };
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < FD_MPL; h += 8) {  // A operands (codes of rows 0-15, the same columns), 8 reads in flight
        v4i am[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) am[m] = *reinterpret_cast<const v4i*>(&s_codes[code_off(nr, lw * 64 + (h + m) * 4 + q)]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 8; ++m)
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(am[m], __builtin_bit_cast(v4i, b[h + m]), acc, 0, 0, 0);
      }
      s_red[lw][lane] = acc;
      __syncthreads();  // B3
      {
        const int t = 4 * q + lw;
        int32_t a = 0;
#pragma unroll
        for (int i = 0; i < FD_LW; ++i) a += s_red[i][lane][lw];
        float o = 0.0f;
        if (blk != blk0)
          o = outlier_sum(t);
        else if (any)
          o = s_osum[t][nr];
        const int64_t col = (int64_t)blk * 16 + nr;
        if (col < N && t < T) {
          for (int p = n_lds; p < n_out; ++p) {  // beyond the LDS stage: straight from memory
            const int cc = s_idx[p];
            const float wv = to_f32<DT>(from_f32<DT>(div127((float)CB[col * K + cc] * scb_n)));
            o += to_f32<DT>(X[(int64_t)t * K + cc]) * wv;
          }
          if (acc_out != nullptr) acc_out[(int64_t)t * N + col] = a;
          const float d = (float)a * (s_sca[t] * (scb_n * (1.0f / 16129.0f)));
          out[(int64_t)t * N + col] = from_f32<DT>(d + o + bias_n);
        }
      }
      __syncthreads();  // B4
    }
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
