// C-ABI of the lli8 library: argument validation, then kernel launches on the
// caller's stream.  Every argument is checked before anything is enqueued, so
// a rejected call writes nothing.  No exception crosses the interface.
#include <algorithm>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/lli8.h"
#include "lli8_internal.h"

namespace {

constexpr int64_t kMaxK = 133144;  // K * 127^2 < 2^31: int32 accumulators stay exact

thread_local char g_err[512] = "";

lli8_status_t fail(lli8_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lli8_status_t fail(lli8_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

lli8_status_t hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return LLI8_OK;
  return fail(LLI8_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

lli8_status_t check_dtype(lli8_dtype_t dt) {
  if (dt != LLI8_F16 && dt != LLI8_BF16) return fail(LLI8_ERR_DTYPE, "dtype %d is not F16 (0) or BF16 (1)", (int)dt);
  return LLI8_OK;
}

lli8_status_t check_sizes(int64_t T, int64_t K, int64_t N) {
  if (T < 0 || K < 1 || N < 1) return fail(LLI8_ERR_SHAPE, "bad sizes T=%lld K=%lld N=%lld", (long long)T, (long long)K, (long long)N);
  if (K > kMaxK) return fail(LLI8_ERR_UNSUPPORTED, "K=%lld above %lld (int32 accumulator headroom)", (long long)K, (long long)kMaxK);
  if (T > INT32_MAX || N > INT32_MAX || T * K > ((int64_t)1 << 40) || N * K > ((int64_t)1 << 40))
    return fail(LLI8_ERR_UNSUPPORTED, "sizes too large T=%lld K=%lld N=%lld", (long long)T, (long long)K, (long long)N);
  return LLI8_OK;
}

#define REQUIRE(p, name)                                                       \
  do {                                                                         \
    if ((p) == nullptr) return fail(LLI8_ERR_NULL, "%s is NULL", name);       \
    if (!aligned16(p)) return fail(LLI8_ERR_ALIGN, "%s is not 16-byte aligned", name); \
  } while (0)

#define OPTIONAL(p, name)                                                      \
  do {                                                                         \
    if ((p) != nullptr && !aligned16(p)) return fail(LLI8_ERR_ALIGN, "%s is not 16-byte aligned", name); \
  } while (0)

#define TRY(x)                                                                 \
  do {                                                                         \
    lli8_status_t st_ = (x);                                                   \
    if (st_ != LLI8_OK) return st_;                                            \
  } while (0)

// ---- optional kernel timing (lli8_trace_*) ----
struct Trace {
  bool on = false;
  bool created = false;
  int n = 0;
  const char* name[LLI8_TRACE_MAX];
  hipEvent_t ev[2 * LLI8_TRACE_MAX];
};
Trace g_trace;

lli8_status_t trace_begin(hipStream_t s, const char* name) {
  if (!g_trace.on) return LLI8_OK;
  if (!g_trace.created) {
    for (int i = 0; i < 2 * LLI8_TRACE_MAX; ++i) {
      hipError_t e = hipEventCreate(&g_trace.ev[i]);
      if (e != hipSuccess) return hip_status(e, "trace event create");
    }
    g_trace.created = true;
  }
  if (g_trace.n >= LLI8_TRACE_MAX) return LLI8_OK;
  g_trace.name[g_trace.n] = name;
  return hip_status(hipEventRecord(g_trace.ev[2 * g_trace.n], s), "trace event record");
}

lli8_status_t trace_end(hipStream_t s) {
  if (!g_trace.on || g_trace.n >= LLI8_TRACE_MAX) return LLI8_OK;
  lli8_status_t st = hip_status(hipEventRecord(g_trace.ev[2 * g_trace.n + 1], s), "trace event record");
  g_trace.n++;
  return st;
}

#define TRACED(stream, name, launch)                                           \
  do {                                                                         \
    TRY(trace_begin(stream, name));                                            \
    TRY(hip_status((launch), name));                                           \
    TRY(trace_end(stream));                                                    \
  } while (0)

// The single-launch decode path can be switched off (LLI8_FUSED_DECODE=0) to
// run the general kernels for small T as well.
bool fused_decode_enabled() {
  const char* v = getenv("LLI8_FUSED_DECODE");
  return !(v != nullptr && v[0] == '0');
}

// Outliers are looked for only for a finite positive threshold.
bool outliers_enabled(float tau) { return tau > 0.0f && isfinite(tau); }

lli8_status_t enqueue_activation_split(const void* X, int64_t T, int64_t K, int dt, float tau, int8_t* CA,
                                       float* SCA, uint32_t* bitmap, int32_t* idx, int32_t* n_idx, void* xo,
                                       const int8_t* CB, const float* SCB, int64_t N, void* wo, int wo_chunks,
                                       hipStream_t s) {
  const int64_t W = (K + 31) / 32;
  const bool scan = outliers_enabled(tau);
  if (lli8::split_small_supported(T, K)) {
    // a few rows: scan and quantiser in one launch (a disabled threshold
    // flags no column)
    TRACED(s, "activation_split",
           lli8::launch_split_small(dt, X, T, K, scan ? tau : 0.0f, CA, SCA, bitmap, idx, n_idx, xo, s));
  } else {
    // the scan of a few rows writes every word itself; otherwise it ORs into
    // a cleared bitmap, and with no scan the cleared bitmap is the result
    if (!scan || !lli8::scan_writes_all_words(T, K))
      TRACED(s, "bitmap_clear", lli8::launch_fill_u32(bitmap, W, 0u, s));
    if (scan) TRACED(s, "outlier_scan", lli8::launch_scan_outliers(dt, X, T, K, tau, bitmap, s));
    TRACED(s, "quant_activations", lli8::launch_quant_act(dt, X, T, K, bitmap, CA, SCA, idx, n_idx, xo, s));
  }
  if (wo != nullptr)
    TRACED(s, "recover_outliers", lli8::launch_recover_outliers(dt, CB, SCB, N, K, idx, n_idx, wo, wo_chunks, s));
  return LLI8_OK;
}

// Scratch layout of lli8_int8_linear: gathered outlier columns of X
// [ceil(K/32)][T][32], then, in whatever room is left, recovered outlier
// weights [chunks][N][32] (16-bit each).
size_t xo_bytes(int64_t T, int64_t K) { return (size_t)(T * ((K + 31) / 32 * 32) * 2); }

// One-buffer workspace (lli8_workspace_bytes / lli8_workspace_carve): the
// pieces in this order, each starting on a 256-byte boundary.
size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }

struct Carve {
  size_t ca, sca, bitmap, idx, n_idx, scratch, scratch_bytes, total;
};

Carve carve_layout(int64_t T, int64_t K, int64_t N) {
  Carve c;
  size_t o = 0;
  c.ca = o;
  o += up256((size_t)(T * K));
  c.sca = o;
  o += up256((size_t)(T > 0 ? T : 1) * 4);
  c.bitmap = o;
  o += up256((size_t)((K + 31) / 32) * 4);
  c.idx = o;
  o += up256((size_t)K * 4);
  c.n_idx = o;
  o += 256;
  c.scratch = o;
  const int64_t chunks = std::min<int64_t>((K + 31) / 32, LLI8_WORKSPACE_WO_CHUNKS);
  c.scratch_bytes = (T > 0 ? xo_bytes(T, K) : 0) + (size_t)(N * 64 * chunks);
  o += up256(c.scratch_bytes);
  c.total = o;
  return c;
}

}  // namespace

namespace lli8 {

lli8_status_t check_linear_args(const void* X, int64_t T, int64_t K, int64_t N, lli8_dtype_t dtype,
                                const int8_t* CB, const float* SCB, const void* bias, float threshold,
                                const void* out) {
  TRY(check_dtype(dtype));
  TRY(check_sizes(T, K, N));
  if (isnan(threshold)) return fail(LLI8_ERR_THRESHOLD, "threshold is NaN");
  REQUIRE(CB, "CB");
  REQUIRE(SCB, "SCB");
  OPTIONAL(bias, "bias");
  if (T > 0) {  // with T == 0 nothing of size T is read or written
    REQUIRE(X, "X");
    REQUIRE(out, "out");
  }
  return LLI8_OK;
}

lli8_status_t set_error(lli8_status_t st, const char* msg) { return fail(st, "%s", msg); }

}  // namespace lli8

extern "C" {

const char* lli8_version(void) { return "0.1.0"; }

void lli8_trace_enable(int on) {
  g_trace.on = on != 0;
  if (!g_trace.on && g_trace.created) {  // release the events now, not at process exit
    for (int i = 0; i < 2 * LLI8_TRACE_MAX; ++i) (void)hipEventDestroy(g_trace.ev[i]);
    g_trace.created = false;
    g_trace.n = 0;
  }
}

lli8_status_t lli8_trace_read(lli8_trace_t* out) {
  if (out == nullptr) return fail(LLI8_ERR_NULL, "trace output is NULL");
  out->n = 0;
  for (int i = 0; i < g_trace.n; ++i) {
    TRY(hip_status(hipEventSynchronize(g_trace.ev[2 * i + 1]), "trace event wait"));
    float ms = 0.0f;
    TRY(hip_status(hipEventElapsedTime(&ms, g_trace.ev[2 * i], g_trace.ev[2 * i + 1]), "trace elapsed"));
    out->name[i] = g_trace.name[i];
    out->ms[i] = ms;
    out->n = i + 1;
  }
  g_trace.n = 0;
  return LLI8_OK;
}

const char* lli8_last_error(void) { return g_err; }

const char* lli8_status_string(lli8_status_t s) {
  switch (s) {
    case LLI8_OK: return "ok";
    case LLI8_ERR_NULL: return "required pointer is NULL";
    case LLI8_ERR_SHAPE: return "invalid shape";
    case LLI8_ERR_DTYPE: return "invalid dtype";
    case LLI8_ERR_ALIGN: return "pointer not 16-byte aligned";
    case LLI8_ERR_THRESHOLD: return "threshold is NaN";
    case LLI8_ERR_UNSUPPORTED: return "unsupported size";
    case LLI8_ERR_HIP: return "HIP runtime error";
    case LLI8_ERR_WORKSPACE: return "scratch buffer missing or too small";
  }
  return "unknown status";
}

size_t lli8_scratch_bytes(int64_t T, int64_t K, lli8_dtype_t dtype) {
  (void)dtype;  // both dtypes are 16-bit
  if (T <= 0 || K <= 0) return 0;
  return xo_bytes(T, K);
}

size_t lli8_scratch_bytes_full(int64_t T, int64_t K, int64_t N, lli8_dtype_t dtype) {
  if (T <= 0 || K <= 0 || N <= 0) return lli8_scratch_bytes(T, K, dtype);
  return xo_bytes(T, K) + (size_t)(N * ((K + 31) / 32 * 32) * 2);
}

size_t lli8_workspace_bytes(int64_t T, int64_t K, int64_t N, lli8_dtype_t dtype) {
  (void)dtype;  // both dtypes are 16-bit
  if (T < 0 || K < 1 || N < 1) return 0;
  return carve_layout(T, K, N).total;
}

lli8_status_t lli8_workspace_carve(void* base, size_t bytes, int64_t T, int64_t K, int64_t N, lli8_dtype_t dtype,
                                   lli8_workspace_t* ws) {
  TRY(check_dtype(dtype));
  TRY(check_sizes(T, K, N));
  if (ws == nullptr) return fail(LLI8_ERR_NULL, "workspace struct is NULL");
  REQUIRE(base, "base");
  const Carve c = carve_layout(T, K, N);
  if (bytes < c.total) return fail(LLI8_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", c.total, bytes);
  char* b = static_cast<char*>(base);
  ws->CA = reinterpret_cast<int8_t*>(b + c.ca);
  ws->SCA = reinterpret_cast<float*>(b + c.sca);
  ws->bitmap = reinterpret_cast<uint32_t*>(b + c.bitmap);
  ws->idx = reinterpret_cast<int32_t*>(b + c.idx);
  ws->n_idx = reinterpret_cast<int32_t*>(b + c.n_idx);
  ws->acc = nullptr;
  ws->scratch = b + c.scratch;
  ws->scratch_bytes = c.scratch_bytes;
  return LLI8_OK;
}

// Compute units of the current device (calibration only; not cached).
static int current_device_cus(hipError_t* err) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  *err = e;
  return e == hipSuccess ? cus : 0;
}

size_t lli8_mfma_i8_loop_sink_ints(void) {
  hipError_t e;
  const int cus = current_device_cus(&e);
  return e == hipSuccess ? (size_t)cus * 512 : 0;
}

lli8_status_t lli8_mfma_i8_loop(int64_t iters, int pattern, int32_t* sink, double* ops, void* stream) {
  if (iters < 1) return fail(LLI8_ERR_SHAPE, "iters must be at least 1, got %lld", (long long)iters);
  if (pattern != 0 && pattern != 1) return fail(LLI8_ERR_UNSUPPORTED, "operand pattern must be 0 or 1, got %d", pattern);
  REQUIRE(sink, "sink");
  if (ops == nullptr) return fail(LLI8_ERR_NULL, "ops is NULL");
  hipError_t e;
  const int cus = current_device_cus(&e);
  if (e != hipSuccess) return hip_status(e, "device query");
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(hip_status(lli8::launch_mfma_i8_loop(iters, pattern, cus, sink, s), "mfma loop launch"));
  // 8 waves x 8 instructions x 2 * 32^3 operations per iteration per workgroup
  *ops = (double)cus * 8.0 * 8.0 * 65536.0 * (double)iters;
  return LLI8_OK;
}

lli8_status_t lli8_recover_weight(const int8_t* CB, const float* SCB, int64_t N, int64_t K, lli8_dtype_t dtype,
                                  void* W, void* stream) {
  TRY(check_dtype(dtype));
  if (N < 0 || K < 0) return fail(LLI8_ERR_SHAPE, "bad sizes N=%lld K=%lld", (long long)N, (long long)K);
  if (N == 0 || K == 0) return LLI8_OK;
  if (N * K > ((int64_t)1 << 40)) return fail(LLI8_ERR_UNSUPPORTED, "N*K too large");
  REQUIRE(CB, "CB");
  REQUIRE(SCB, "SCB");
  REQUIRE(W, "W");
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRACED(s, "recover_weight", lli8::launch_recover_weight((int)dtype, CB, SCB, N, K, W, s));
  return LLI8_OK;
}

lli8_status_t lli8_quant_weight_rowwise(const void* W, int64_t N, int64_t K, lli8_dtype_t dtype, int8_t* CB,
                                        float* SCB, void* stream) {
  TRY(check_dtype(dtype));
  if (N < 0 || K < 1) return fail(LLI8_ERR_SHAPE, "bad sizes N=%lld K=%lld", (long long)N, (long long)K);
  if (K > kMaxK) return fail(LLI8_ERR_UNSUPPORTED, "K=%lld above %lld", (long long)K, (long long)kMaxK);
  REQUIRE(W, "W");
  REQUIRE(CB, "CB");
  REQUIRE(SCB, "SCB");
  if (N == 0) return LLI8_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRACED(s, "quant_weight", lli8::launch_quant_weight((int)dtype, W, N, K, CB, SCB, s));
  return LLI8_OK;
}

lli8_status_t lli8_quant_vectorwise(const void* X, int64_t R, int64_t C, lli8_dtype_t dtype,
                                    lli8_scheme_t scheme, lli8_axis_t axis, int8_t* codes,
                                    float* scale, int32_t* zero_point, void* stream) {
  TRY(check_dtype(dtype));
  if (scheme != LLI8_ABSMAX && scheme != LLI8_ZEROPOINT)
    return fail(LLI8_ERR_UNSUPPORTED, "unknown scheme %d", (int)scheme);
  if (axis != LLI8_ROWS && axis != LLI8_COLS) return fail(LLI8_ERR_UNSUPPORTED, "unknown axis %d", (int)axis);
  if (R < 0 || C < 0) return fail(LLI8_ERR_SHAPE, "bad sizes R=%lld C=%lld", (long long)R, (long long)C);
  const int64_t nvec = axis == LLI8_ROWS ? R : C;
  if (nvec == 0) return LLI8_OK;
  if (R > 0 && C > 0) {
    REQUIRE(X, "X");
    REQUIRE(codes, "codes");
  }
  REQUIRE(scale, "scale");
  if (scheme == LLI8_ZEROPOINT) REQUIRE(zero_point, "zero_point");
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRACED(s, scheme == LLI8_ZEROPOINT ? "quant_zeropoint" : "quant_absmax",
         lli8::launch_quant_vectorwise((int)dtype, X, R, C, scheme == LLI8_ZEROPOINT ? 1 : 0,
                                       axis == LLI8_ROWS ? 0 : 1, codes, scale, zero_point, s));
  return LLI8_OK;
}

lli8_status_t lli8_quant_rowwise_outliers(const void* X, int64_t T, int64_t K, lli8_dtype_t dtype, float threshold,
                                          int8_t* CA, float* SCA, uint32_t* bitmap, int32_t* idx, int32_t* n_idx,
                                          void* stream) {
  TRY(check_dtype(dtype));
  TRY(check_sizes(T, K, 1));
  if (isnan(threshold)) return fail(LLI8_ERR_THRESHOLD, "threshold is NaN");
  if (T > 0) {
    REQUIRE(X, "X");
    REQUIRE(CA, "CA");
    REQUIRE(SCA, "SCA");
  }
  REQUIRE(bitmap, "bitmap");
  REQUIRE(idx, "idx");
  REQUIRE(n_idx, "n_idx");
  hipStream_t s = static_cast<hipStream_t>(stream);
  return enqueue_activation_split(X, T, K, (int)dtype, threshold, CA, SCA, bitmap, idx, n_idx, nullptr, nullptr,
                                  nullptr, 0, nullptr, 0, s);
}

lli8_status_t lli8_int8_linear(const void* X, int64_t T, int64_t K, int64_t N, lli8_dtype_t dtype, const int8_t* CB,
                               const float* SCB, const void* bias, float threshold, void* out,
                               const lli8_workspace_t* ws, void* stream) {
  TRY(lli8::check_linear_args(X, T, K, N, dtype, CB, SCB, bias, threshold, out));
  if (ws == nullptr) return fail(LLI8_ERR_NULL, "workspace is NULL");
  if (T > 0) {  // with T == 0 nothing of size T is read or written
    REQUIRE(ws->CA, "ws->CA");
    REQUIRE(ws->SCA, "ws->SCA");
  }
  REQUIRE(ws->bitmap, "ws->bitmap");
  REQUIRE(ws->idx, "ws->idx");
  REQUIRE(ws->n_idx, "ws->n_idx");
  OPTIONAL(ws->acc, "ws->acc");
  const bool outl = outliers_enabled(threshold);
  if (outl && T > 0) {
    const size_t need = lli8_scratch_bytes(T, K, dtype);
    if (ws->scratch == nullptr || ws->scratch_bytes < need)
      return fail(LLI8_ERR_WORKSPACE, "scratch needs %zu bytes, got %zu", need, ws->scratch ? ws->scratch_bytes : (size_t)0);
    if (!aligned16(ws->scratch)) return fail(LLI8_ERR_ALIGN, "ws->scratch is not 16-byte aligned");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T > 0 && lli8::decode_fused_supported(T, K) && fused_decode_enabled()) {
    lli8::FusedArgs f;
    f.dt = (int)dtype;
    f.X = X;
    f.T = T;
    f.K = K;
    f.N = N;
    f.tau = outl ? threshold : 0.0f;
    f.CB = CB;
    f.SCB = SCB;
    f.bias = bias;
    f.out = out;
    f.CA = ws->CA;
    f.SCA = ws->SCA;
    f.bitmap = ws->bitmap;
    f.idx = ws->idx;
    f.n_idx = ws->n_idx;
    f.acc = ws->acc;
    TRACED(s, "decode_fused", lli8::launch_decode_fused(f, s));
    return LLI8_OK;
  }
  // room for recovered outlier weights after the gathered columns (tile path
  // only: the weight-streaming kernel reads CB itself)
  void* wo = nullptr;
  int wo_chunks = 0;
  // (up to 256 tokens the tiles gather CB at the outlier columns themselves:
  // fewer tile rows read each weight row, and the launch saved is worth more,
  // T = 65-256 at N = K = 4096: 26.3-28.4 -> 25.1-26.6 us)
  if (outl && !lli8::stream_gemm_route(T, N, K) && T > 256) {
    const size_t xb = xo_bytes(T, K), per_chunk = (size_t)N * 64;
    const size_t room = ws->scratch_bytes > xb ? ws->scratch_bytes - xb : 0;
    const int64_t c = (int64_t)(room / per_chunk), cmax = (K + 31) / 32;
    wo_chunks = (int)(c < cmax ? c : cmax);
    if (wo_chunks > 0) wo = static_cast<char*>(ws->scratch) + xb;
  }
  TRY(enqueue_activation_split(X, T, K, (int)dtype, threshold, ws->CA, ws->SCA, ws->bitmap, ws->idx, ws->n_idx,
                               outl ? ws->scratch : nullptr, CB, SCB, N, wo, wo_chunks, s));
  lli8::LinearArgs a;
  a.dt = (int)dtype;
  a.CA = ws->CA;
  a.CB = CB;
  a.SCA = ws->SCA;
  a.SCB = SCB;
  a.bias = bias;
  a.xo = outl ? ws->scratch : nullptr;
  a.wo = wo;
  a.wo_chunks = wo_chunks;
  a.idx = ws->idx;
  a.n_idx = ws->n_idx;
  a.out = out;
  a.acc = ws->acc;
  a.T = T;
  a.N = N;
  a.K = K;
  TRACED(s, "int8_gemm", lli8::launch_linear_gemm(a, s));
  return LLI8_OK;
}

}  // extern "C"
