// Calibration kernel, not part of the method: how fast the int8 matrix cores
// run on this board when nothing else limits them.  Each wave issues chains
// of v_mfma_i32_32x32x32_i8 on operands held in registers (no memory traffic
// inside the loop), eight independent accumulators per wave and two waves
// per SIMD, so the matrix core always has an instruction ready.  The rate it
// reaches, against 256 compute units x 8192 int8 operations per clock,
// gives the clock the board sustains under int8 matrix load, and the
// achievable int8 peak the GEMM can be compared with beside the nominal one.
//
// The board's clock under matrix load depends on the operand values: with
// every byte 1 the multipliers hardly switch and the loop runs near the
// nominal rate, while bytes that change from one instruction to the next,
// as a GEMM's do, draw more power and the clock drops.  Pattern 1 measures
// that case: four A and four B operands of pseudo-random bytes per thread,
// and the eight chains pair them differently, so consecutive instructions
// never repeat an operand pair.
#include "lli8_device.h"
#include "lli8_internal.h"

namespace lli8 {

constexpr int CAL_THREADS = 512;  // eight waves: two per SIMD

// A 32-bit integer mix (xor-shift / multiply rounds); only its output
// spread matters here, and the host recomputes it to check the sums.
__device__ __forceinline__ uint32_t cal_mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <int PATTERN>
__global__ __launch_bounds__(CAL_THREADS) void mfma_i8_loop_kernel(int64_t iters, int32_t* __restrict__ sink) {
  const uint32_t t = blockIdx.x * CAL_THREADS + threadIdx.x;
  // pattern 0: every operand byte 1, so each instruction adds 32 to every
  // accumulator; pattern 1: dword e of A operand j is cal_mix(32 t + 4 j + e),
  // of B operand j cal_mix(32 t + 16 + 4 j + e)
  v4i a[4], b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[j][e] = PATTERN ? (int)cal_mix(32u * t + 4u * j + e) : 0x01010101;
      b[j][e] = PATTERN ? (int)cal_mix(32u * t + 16u + 4u * j + e) : 0x01010101;
    }
  v16i acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = (v16i){0};
  for (int64_t i = 0; i < iters; ++i) {
    // chain j multiplies A operand j % 4 by B operand j / 2
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j & 3], b[j >> 1], acc[j], 0, 0, 0);
  }
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[t] = s;
}

hipError_t launch_mfma_i8_loop(int64_t iters, int pattern, int blocks, int32_t* sink, hipStream_t s) {
  if (pattern == 0)
    mfma_i8_loop_kernel<0><<<dim3((unsigned)blocks), dim3(CAL_THREADS), 0, s>>>(iters, sink);
  else
    mfma_i8_loop_kernel<1><<<dim3((unsigned)blocks), dim3(CAL_THREADS), 0, s>>>(iters, sink);
  return hipGetLastError();
}

}  // namespace lli8
