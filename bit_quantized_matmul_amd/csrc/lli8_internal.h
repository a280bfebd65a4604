// Host-side launchers of the lli8 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lli8.h"

namespace lli8 {

// Validation of lli8_int8_linear's arguments other than the workspace
// (records the message lli8_last_error returns).
lli8_status_t check_linear_args(const void* X, int64_t T, int64_t K, int64_t N, lli8_dtype_t dtype,
                                const int8_t* CB, const float* SCB, const void* bias, float threshold,
                                const void* out);
// Records msg as this thread's lli8_last_error and returns st.
lli8_status_t set_error(lli8_status_t st, const char* msg);

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);

hipError_t launch_quant_weight(int dt, const void* W, int64_t N, int64_t K, int8_t* CB,
                               float* SCB, hipStream_t s);

hipError_t launch_scan_outliers(int dt, const void* X, int64_t T, int64_t K, float tau,
                                uint32_t* bitmap, hipStream_t s);

// True when launch_scan_outliers writes every bitmap word itself (few rows:
// one workgroup per column strip covers all of them), so the bitmap needs no
// clearing beforehand; otherwise it ORs into a zeroed bitmap.
bool scan_writes_all_words(int64_t T, int64_t K);

// Outlier scan and activation quantiser in one launch for a few rows (T <=
// 32, K % 8 == 0, K <= 4096): bitmap, CA, SCA, idx, n_idx and Xo as the two
// launches below write them.
bool split_small_supported(int64_t T, int64_t K);
hipError_t launch_split_small(int dt, const void* X, int64_t T, int64_t K, float tau, int8_t* CA, float* SCA,
                              uint32_t* bitmap, int32_t* idx, int32_t* n_idx, void* xo, hipStream_t s);

hipError_t launch_quant_act(int dt, const void* X, int64_t T, int64_t K, const uint32_t* bitmap,
                            int8_t* CA, float* SCA, int32_t* idx, int32_t* n_idx, void* xo,
                            hipStream_t s);

// Whether the weight-streaming GEMM kernel takes a shape (K % 16 == 0): it
// reads each weight row once but every workgroup reads all of CA, so it
// wins only on layers of at most 4096 outputs, for up to 32 tokens at any
// depth and up to 64 at K <= 4096 (GEMM times: T = 32, K = 12288: 23.5
// against 27.7 us on tiles; T = 48, K = N = 4096: 21 against 26 us).  Wider
// layers go to the tiles (T = 32, N = 11008: 16.4 against 27.8 us; N = 28672:
// 25.7 against 61.1 us), and so do more tokens (T = 65-128: 26-27 against
// 27-32 us for the step).  The tiles read recovered outlier weights from
// scratch past 256 tokens and gather them from CB below that.
inline bool stream_gemm_route(int64_t T, int64_t N, int64_t K) {
  return (K % 16) == 0 && N <= 4096 && (T <= 32 || (T <= 64 && K <= 4096));
}

// Calibration loop of int8 matrix-core instructions (lli8_calib.hip).
hipError_t launch_mfma_i8_loop(int64_t iters, int pattern, int blocks, int32_t* sink, hipStream_t s);

// W = dtype(fl32(fl32(CB * SCB) / 127)) for a whole [N, K] weight.
hipError_t launch_recover_weight(int dt, const int8_t* CB, const float* SCB, int64_t N, int64_t K, void* W,
                                 hipStream_t s);

hipError_t launch_quant_vectorwise(int dt, const void* X, int64_t R, int64_t C, int zeropoint, int axis,
                                   int8_t* codes, float* scale, int32_t* zp, hipStream_t s);
// Recovered weights of the first min(ceil(n/32), chunks) outlier chunks,
// chunk-major [chunk][N][32] 16-bit (n read on the device).
hipError_t launch_recover_outliers(int dt, const int8_t* CB, const float* SCB, int64_t N, int64_t K,
                                   const int32_t* idx, const int32_t* n_idx, void* wo, int chunks, hipStream_t s);

struct LinearArgs {
  int dt;
  const int8_t* CA;
  const int8_t* CB;
  const float* SCA;
  const float* SCB;
  const void* bias;      // may be null
  const void* xo;        // gathered outlier columns, chunk-major [ceil(n/32)][T][32]
  const void* wo;        // recovered weights of the first wo_chunks outlier chunks, [wo_chunks][N][32]
  int wo_chunks;
  const int32_t* idx;
  const int32_t* n_idx;  // device
  void* out;
  int32_t* acc;          // may be null
  int64_t T, N, K;
};

hipError_t launch_linear_gemm(const LinearArgs& a, hipStream_t s);

// Fused single-launch path for T <= 16 (outlier scan, quantisation, GEMM).
struct FusedArgs {
  int dt;
  const void* X;
  int64_t T, K, N;
  float tau;
  const int8_t* CB;
  const float* SCB;
  const void* bias;  // may be null
  void* out;
  int8_t* CA;
  float* SCA;
  uint32_t* bitmap;
  int32_t* idx;
  int32_t* n_idx;
  int32_t* acc;      // may be null
};

bool decode_fused_supported(int64_t T, int64_t K);
hipError_t launch_decode_fused(const FusedArgs& a, hipStream_t s);

}  // namespace lli8
