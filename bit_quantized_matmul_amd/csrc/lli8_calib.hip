// Calibration kernel, not part of the method: how fast the int8 matrix cores
// run on this board when nothing else limits them.  Each wave issues chains
// of v_mfma_i32_32x32x32_i8 on operands held in registers (no memory traffic
// inside the loop), eight independent accumulators per wave and two waves
// per SIMD, so the matrix core always has an instruction ready.  The rate it
// reaches, against 256 compute units x 8192 int8 operations per clock,
// gives the clock the board sustains under int8 matrix load, and the
// achievable int8 peak the GEMM can be compared with beside the nominal one.
#include "lli8_device.h"
#include "lli8_internal.h"

namespace lli8 {

constexpr int CAL_THREADS = 512;  // eight waves: two per SIMD

__global__ __launch_bounds__(CAL_THREADS) void mfma_i8_loop_kernel(int64_t iters, int32_t* __restrict__ sink) {
  // every operand byte is 1: each instruction adds 32 to every accumulator
  const v4i a = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  v16i acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = (v16i){0};
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, acc[j], 0, 0, 0);
  }
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[(int64_t)blockIdx.x * CAL_THREADS + threadIdx.x] = s;
}

hipError_t launch_mfma_i8_loop(int64_t iters, int blocks, int32_t* sink, hipStream_t s) {
  mfma_i8_loop_kernel<<<dim3((unsigned)blocks), dim3(CAL_THREADS), 0, s>>>(iters, sink);
  return hipGetLastError();
}

}  // namespace lli8
