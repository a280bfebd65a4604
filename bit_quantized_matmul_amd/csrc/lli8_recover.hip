// The 16-bit weight that the int8 codes stand for ("Hugging Face integrates
// LLM.int8() ...", section "Integration into transformers": the weight is
// recovered as (CB * SCB) / 127):
//
//   W[n, k] = dtype(fl32(fl32(CB[n, k] * SCB[n]) / 127))
//
// the page's expression evaluated left to right in fp32, then rounded to the
// 16-bit dtype -- the same values the forward's 16-bit outlier product uses
// for its weights.  Not a step of the forward: a conversion for callers that
// want the dequantised weight back.  HBM-bound (one byte read, two written
// per element); for K % 8 == 0 each thread converts 8 consecutive codes of a
// row (one 8-byte load, one 16-byte store), otherwise one code at a time.
#include "lli8_device.h"
#include "lli8_internal.h"

namespace lli8 {

namespace {

__device__ __forceinline__ float recover_value(int8_t c, float scb, bool inrange) {
  const float p = (float)c * scb;
  return inrange ? div127_inrange(p) : div127(p);
}

template <int DT>
__global__ __launch_bounds__(256) void recover_weight_vec_kernel(const int8_t* __restrict__ CB,
                                                                 const float* __restrict__ SCB, int64_t N,
                                                                 int64_t K, uint16_t* __restrict__ W) {
  const int64_t per_row = K >> 3;  // 8-code pieces per row
  const int64_t total = N * per_row;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total; p += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = p / per_row;
    const int64_t off = p * 8;  // == n * K + 8 * (p - n * per_row)
    const uint64_t codes = *reinterpret_cast<const uint64_t*>(CB + off);
    const float s = SCB[n];
    const bool inrange = div127_scale_ok(s);
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int8_t c0 = (int8_t)(codes >> (16 * d));
      const int8_t c1 = (int8_t)(codes >> (16 * d + 8));
      o[d] = (uint32_t)from_f32<DT>(recover_value(c0, s, inrange)) |
             ((uint32_t)from_f32<DT>(recover_value(c1, s, inrange)) << 16);
    }
    *reinterpret_cast<u32x4*>(W + off) = o;
  }
}

template <int DT>
__global__ __launch_bounds__(256) void recover_weight_any_kernel(const int8_t* __restrict__ CB,
                                                                 const float* __restrict__ SCB, int64_t N,
                                                                 int64_t K, uint16_t* __restrict__ W) {
  const int64_t total = N * K;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const float s = SCB[e / K];
    W[e] = from_f32<DT>(recover_value(CB[e], s, div127_scale_ok(s)));
  }
}

template <int DT>
hipError_t launch_recover_weight_t(const int8_t* CB, const float* SCB, int64_t N, int64_t K, uint16_t* W,
                                   hipStream_t s) {
  const bool vec = (K % 8) == 0;
  const int64_t work = vec ? N * (K / 8) : N * K;
  const int64_t blocks = std::min<int64_t>((work + 255) / 256, 256 * 16);
  if (vec)
    recover_weight_vec_kernel<DT><<<dim3((unsigned)blocks), 256, 0, s>>>(CB, SCB, N, K, W);
  else
    recover_weight_any_kernel<DT><<<dim3((unsigned)blocks), 256, 0, s>>>(CB, SCB, N, K, W);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_recover_weight(int dt, const int8_t* CB, const float* SCB, int64_t N, int64_t K, void* W,
                                 hipStream_t s) {
  uint16_t* w = static_cast<uint16_t*>(W);
  return dt == DT_F16 ? launch_recover_weight_t<DT_F16>(CB, SCB, N, K, w, s)
                      : launch_recover_weight_t<DT_BF16>(CB, SCB, N, K, w, s);
}

}  // namespace lli8
