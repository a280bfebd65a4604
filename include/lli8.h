/*
 * lli8 -- the LLM.int8() mixed-precision decomposition linear (forward) on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation, as the pages define it:
 *   - "Hugging Face integrates LLM.int8() 8-bit matrix multiplication into
 *     Transformers and Accelerate", section "Core idea of LLM.int8()":
 *     (1) feature columns of the activation holding a value whose magnitude
 *     exceeds a threshold are split off; (2) they are multiplied in 16-bit,
 *     while the rest is quantised to int8 with vector-wise scales (one per
 *     activation row, one per weight output row) and multiplied in int8;
 *     (3) the int8 result is dequantised and summed with the 16-bit result.
 *   - same page, section "Quantization mechanics": absmax quantisation
 *     scales a vector by 127 / absmax and rounds, giving codes in [-127, 127].
 *   - same page, section "Integration into transformers": the int8 weight CB
 *     and its scale SCB recover the weight as (CB * SCB) / 127.
 *   - "Class Linear8bitLt", __init__ Args: with has_fp16_weights=False the
 *     weight is quantised once when the module is placed on the device; with
 *     True it is quantised in every forward.  The threshold acts on the
 *     activation columns.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer to a caller-owned, contiguous,
 *     row-major buffer.  The library allocates no device memory and keeps no
 *     per-call state; all work is enqueued asynchronously on `stream`
 *     (a hipStream_t passed as void*, so that this header needs no HIP
 *     header; NULL means the default stream).  No call synchronises the
 *     host.  Process-wide, the library remembers only each device's compute
 *     unit count (looked up once, to size persistent grids) and the optional
 *     kernel-timing events of lli8_trace_enable.
 *   - Inputs are finite.  A NaN or infinite activation is outside the
 *     contract: its column may or may not be flagged (the kernels compare
 *     magnitude bit patterns, under which NaN exceeds every threshold).
 *   - X, W, bias and out share one 16-bit dtype (fp16 or bf16).  Codes (CA,
 *     CB) are int8 in [-127, 127]; scales (SCA, SCB) are fp32 and hold the
 *     row absmax itself; the dequantisation factor is SCA * SCB / 127^2.
 *   - Rounding of codes: round(fl32(x * fl32(127 / absmax))), halves away
 *     from zero.  A row whose absmax is 0 gets scale 0 and all-zero codes.
 *     Below an absmax of 2^-100 (bf16 only), where 127 / absmax can
 *     overflow fp32, x and the absmax are scaled by 2^64 first (exact); the
 *     codes are the plain form's wherever that form is finite.
 *   - threshold: column c is an outlier when some |X[t, c]| > threshold
 *     (strict, compared in fp32).  threshold <= 0 or +inf: no outlier
 *     columns (plain vector-wise int8).  NaN: LLI8_ERR_THRESHOLD.
 *   - Arguments are validated before anything is enqueued; on a validation
 *     error nothing is written.  A launch failure returns LLI8_ERR_HIP and
 *     lli8_last_error() gives the runtime's message.  No C++ exception
 *     crosses this interface.  Sizes are int64_t; 0 <= T, 1 <= K, N;
 *     K <= 133144 keeps every int32 accumulator exact.
 *   - Device pointers must be 16-byte aligned (LLI8_ERR_ALIGN otherwise).
 *     With T == 0, the buffers whose size is a multiple of T (X, CA, SCA,
 *     out, acc) may be NULL.
 */
#ifndef LLI8_H
#define LLI8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LLI8_F16 = 0, LLI8_BF16 = 1 } lli8_dtype_t;

typedef enum {
  LLI8_OK = 0,
  LLI8_ERR_NULL = 1,        /* a required pointer is NULL                        */
  LLI8_ERR_SHAPE = 2,       /* T < 0, K < 1 or N < 1                             */
  LLI8_ERR_DTYPE = 3,       /* dtype is not LLI8_F16 / LLI8_BF16                 */
  LLI8_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned           */
  LLI8_ERR_THRESHOLD = 5,   /* threshold is NaN                                  */
  LLI8_ERR_UNSUPPORTED = 6, /* K above 133144 (int32 accumulator headroom)       */
  LLI8_ERR_HIP = 7,         /* the HIP runtime reported an error                 */
  LLI8_ERR_WORKSPACE = 8    /* scratch buffer missing or smaller than required   */
} lli8_status_t;

/*
 * Weight quantisation (per output row), "Core idea of LLM.int8()" step 2 and
 * "Integration into transformers" (CB, SCB, recovery (CB * SCB) / 127).
 *   W   [N, K] fp16/bf16 (read)
 *   CB  [N, K] int8 (written): round(fl32(W * fl32(127 / SCB[n])))
 *   SCB [N] fp32 (written): max_k |W[n, k]|
 * Called once at placement (has_fp16_weights=False) or before every forward
 * (has_fp16_weights=True).
 */
lli8_status_t lli8_quant_weight_rowwise(const void* W, int64_t N, int64_t K,
                                        lli8_dtype_t dtype, int8_t* CB,
                                        float* SCB, void* stream);

/*
 * Activation split and quantisation, "Core idea of LLM.int8()" steps 1-2;
 * record "LLM.int8() / bitsandbytes int8", field "Activation scheme" (the
 * outlier unit is the feature column, found at run time per matmul).
 *   X      [T, K] fp16/bf16 (read)
 *   CA     [T, K] int8 (written): codes of X with outlier columns set to 0
 *   SCA    [T] fp32 (written): max over non-outlier k of |X[t, k]|
 *   bitmap [ceil(K/32)] uint32 (written): bit (c % 32) of word c / 32 is set
 *          when column c is an outlier
 *   idx    [K] int32 (written): the first *n_idx entries are the outlier
 *          columns in ascending order (the module's state.idx); the rest are
 *          left as they were
 *   n_idx  [1] int32 (written, device): number of outlier columns
 */
lli8_status_t lli8_quant_rowwise_outliers(const void* X, int64_t T, int64_t K,
                                          lli8_dtype_t dtype, float threshold,
                                          int8_t* CA, float* SCA,
                                          uint32_t* bitmap, int32_t* idx,
                                          int32_t* n_idx, void* stream);

/*
 * Buffers of one forward call.  The caller owns all of them.  After the call
 * CA, SCA, bitmap, idx and n_idx hold this call's values exactly as
 * lli8_quant_rowwise_outliers defines them.  acc, when not NULL, receives the
 * int32 products acc[t, n] = sum_k CA[t, k] * CB[n, k] ([T, N] row-major).
 * scratch is internal storage of at least lli8_scratch_bytes(T, K, dtype)
 * bytes (the gathered outlier columns of X), required when the threshold
 * enables outlier columns.  Calls sharing one workspace must be ordered on
 * one stream.
 */
typedef struct lli8_workspace {
  int8_t* CA;
  float* SCA;
  uint32_t* bitmap;
  int32_t* idx;
  int32_t* n_idx;
  int32_t* acc;     /* optional */
  void* scratch;
  size_t scratch_bytes;
} lli8_workspace_t;

/* Bytes of one caller buffer that lli8_workspace_carve splits into all the
 * buffers of a forward call for these sizes: CA, SCA, bitmap, idx, n_idx and
 * a scratch with room for the recovered weights of LLI8_WORKSPACE_WO_CHUNKS
 * 32-column outlier chunks (outlier columns beyond them are gathered from CB
 * inside the GEMM tiles), each piece on a 256-byte boundary.  acc is not
 * included.  0 for invalid sizes. */
#define LLI8_WORKSPACE_WO_CHUNKS 8
size_t lli8_workspace_bytes(int64_t T, int64_t K, int64_t N, lli8_dtype_t dtype);

/* Fills *ws with pointers into the caller's device buffer `base` of `bytes`
 * bytes (at least lli8_workspace_bytes(T, K, N, dtype)), acc = NULL.  Writes
 * nothing to device memory.  Errors: LLI8_ERR_NULL (ws or base NULL),
 * _ALIGN (base not 16-byte aligned), _SHAPE, _DTYPE, _UNSUPPORTED as for
 * lli8_int8_linear, LLI8_ERR_WORKSPACE (buffer too small). */
lli8_status_t lli8_workspace_carve(void* base, size_t bytes, int64_t T, int64_t K, int64_t N,
                                   lli8_dtype_t dtype, lli8_workspace_t* ws);

/* Bytes of scratch lli8_int8_linear needs for these sizes (the minimum:
 * the gathered outlier columns of X). */
size_t lli8_scratch_bytes(int64_t T, int64_t K, lli8_dtype_t dtype);

/* Bytes of scratch that also hold the recovered weights (CB * SCB) / 127 of
 * every possible outlier column for an N-row weight: with this much, each
 * call recovers them once instead of in every output tile (the fast path
 * when many columns are outliers).  Any size in between is used as far as it
 * goes, in whole 32-column chunks of N * 64 bytes. */
size_t lli8_scratch_bytes_full(int64_t T, int64_t K, int64_t N, lli8_dtype_t dtype);

/*
 * The whole forward, "Core idea of LLM.int8()" steps 1-3:
 *   out[t, n] = acc[t, n] * SCA[t] * SCB[n] / 127^2
 *             + sum over outlier columns c of X[t, c] * What[n, c]
 *             + bias[n]
 * with What[n, c] = dtype(fl32(fl32(CB[n, c] * SCB[n]) / 127)), the recovery
 * form of "Integration into transformers", accumulated in fp32 and rounded
 * once to the output dtype.
 *   X    [T, K] fp16/bf16 (read)      CB [N, K] int8, SCB [N] fp32 (read)
 *   bias [N] fp16/bf16 or NULL        out [T, N] fp16/bf16 (written)
 * The outlier set is taken from this call's X.
 */
lli8_status_t lli8_int8_linear(const void* X, int64_t T, int64_t K, int64_t N,
                               lli8_dtype_t dtype, const int8_t* CB,
                               const float* SCB, const void* bias,
                               float threshold, void* out,
                               const lli8_workspace_t* ws, void* stream);

/*
 * lli8_int8_linear for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The same forward, the same kernels and the same output as
 * lli8_int8_linear, with every workspace buffer (CA, SCA, bitmap, idx,
 * n_idx and the scratch, laid out as lli8_workspace_carve lays them out) in
 * a fixed device array of LLI8_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on each GPU it runs on until the process ends.  The caller passes
 * inputs and outputs as for lli8_int8_linear; no int32 accumulators are
 * written.  The call allocates nothing and frees nothing (the array's device
 * address is looked up once per device, on the first call there).
 *   - Sizes whose lli8_workspace_bytes(T, K, N, dtype) exceeds the array
 *     (e.g. 4096 tokens at K = 12288) are rejected with LLI8_ERR_UNSUPPORTED
 *     before anything is enqueued; 4096 x 4096 -> 11008 fits.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents: calls that overlap on one GPU (other streams, other
 *     threads) race and must be serialised by the caller.
 *   - Other errors as lli8_int8_linear.
 */
#define LLI8_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
lli8_status_t lli8_int8_linear_noalloc(const void* X, int64_t T, int64_t K, int64_t N,
                                       lli8_dtype_t dtype, const int8_t* CB, const float* SCB,
                                       const void* bias, float threshold, void* out, void* stream);

/* LLI8_NOALLOC_SCRATCH_BYTES, for bindings that cannot read the macro. */
size_t lli8_noalloc_scratch_bytes(void);

/*
 * Weight recovery, "Hugging Face integrates LLM.int8() ...", section
 * "Integration into transformers": the weight the int8 codes stand for is
 * (CB * SCB) / 127.  Evaluated left to right in fp32 and rounded once to the
 * dtype, the values the forward's 16-bit outlier product uses:
 *   W[n, k] = dtype(fl32(fl32(CB[n, k] * SCB[n]) / 127))
 *   CB [N, K] int8, SCB [N] fp32 (read); W [N, K] fp16/bf16 (written).
 * Not a step of lli8_int8_linear.  Errors: LLI8_ERR_NULL, _ALIGN, _SHAPE
 * (N or K negative), _DTYPE, before anything is enqueued; N == 0 or K == 0 is
 * a no-op.
 */
lli8_status_t lli8_recover_weight(const int8_t* CB, const float* SCB, int64_t N, int64_t K,
                                  lli8_dtype_t dtype, void* W, void* stream);

/*
 * Vector-wise quantisation of a 16-bit matrix on its own ("Hugging Face
 * integrates LLM.int8() ...", section "Quantization mechanics": zero-point and
 * absmax, each row-wise or column-wise).  Not a step of lli8_int8_linear.
 *   X      [R, C] fp16/bf16 row-major (read)
 *   codes  [R, C] int8 (written)
 *   scale  [R] (axis LLI8_ROWS) or [C] (axis LLI8_COLS) fp32 (written)
 *   zero_point  same count, int32 (written; zero-point scheme only, may be
 *          NULL for absmax)
 * LLI8_ABSMAX: scale = max |x| of the vector, code = round_half_away(
 *   fl32(x * fl32(127 / scale))) in [-127, 127]; an all-zero vector gets
 *   scale 0 and codes 0.  x is recovered as code * scale / 127.
 * LLI8_ZEROPOINT: the vector's range [min, max] widened to contain 0 is
 *   mapped onto [-127, 127]: scale = nd = fl32(254 / fl32(hi - lo)),
 *   zero_point = round_half_away(fl32(-lo * nd)) - 127 (the code of 0.0),
 *   code = clamp(round_half_away(fl32(x * nd)) + zero_point, -127, 127); an
 *   all-zero vector gets nd 0, zero point 0, codes 0.  x is recovered as
 *   (code - zero_point) / nd.  A range narrower than 254 / FLT_MAX (bf16
 *   only), whose nd would overflow, is outside the contract.
 * Absmax codes of a vector with max |x| below 2^-100 are taken as in the
 * forward (x and the absmax scaled by 2^64 first).
 * Inputs are finite.  Asynchronous on `stream`; pointers 16-byte aligned.
 * Errors: LLI8_ERR_NULL, _SHAPE (R or C negative), _DTYPE, _ALIGN, and
 * LLI8_ERR_UNSUPPORTED for an unknown scheme or axis, before anything is
 * enqueued.
 */
typedef enum { LLI8_ABSMAX = 0, LLI8_ZEROPOINT = 1 } lli8_scheme_t;
typedef enum { LLI8_ROWS = 0, LLI8_COLS = 1 } lli8_axis_t;
lli8_status_t lli8_quant_vectorwise(const void* X, int64_t R, int64_t C, lli8_dtype_t dtype,
                                    lli8_scheme_t scheme, lli8_axis_t axis, int8_t* codes,
                                    float* scale, int32_t* zero_point, void* stream);

/*
 * Calibration, not a step of the method: how fast the int8 matrix cores run
 * on this board with nothing else limiting them, for comparing the GEMM with
 * an achievable peak beside the nominal one.  One 512-thread workgroup per
 * compute unit; each of its eight waves issues 8 * iters
 * v_mfma_i32_32x32x32_i8 on operands held in registers, in eight chains of
 * accumulators; thread t writes the sum of its accumulators (modulo 2^32) to
 * sink[t].
 *   pattern  0: every operand byte 1 (each thread's sum is 4096 * iters);
 *            1: pseudo-random bytes, the clock the board holds when the
 *            operands switch as a GEMM's do.  Dword e (0..3) of thread t's
 *            A operand j (0..3) is mix(32 t + 4 j + e), of its B operand j
 *            mix(32 t + 16 + 4 j + e), where mix(x) is: x ^= x >> 16;
 *            x *= 0x7feb352d; x ^= x >> 15; x *= 0x846ca68b; x ^= x >> 16
 *            (32-bit unsigned arithmetic); chain c (0..7) multiplies A
 *            operand c % 4 by B operand c / 2.
 *   sink     device int32 buffer of lli8_mfma_i8_loop_sink_ints() entries
 *            (512 per compute unit of the current device), 16-byte aligned
 *   ops      host: receives the int8 operations the launch performs
 *            (2 * 32^3 per instruction)
 * Asynchronous on `stream`.  Errors: LLI8_ERR_SHAPE (iters < 1),
 * LLI8_ERR_UNSUPPORTED (pattern not 0 or 1), LLI8_ERR_NULL, LLI8_ERR_ALIGN,
 * LLI8_ERR_HIP.
 */
lli8_status_t lli8_mfma_i8_loop(int64_t iters, int pattern, int32_t* sink, double* ops, void* stream);
size_t lli8_mfma_i8_loop_sink_ints(void);

/*
 * Optional kernel timing, for profiling.  While enabled (process-wide), each
 * kernel the entry points enqueue is bracketed by two HIP events recorded on
 * the call's stream.  lli8_trace_read waits for those events and reports the
 * kernels enqueued since the previous read (at most LLI8_TRACE_MAX; later
 * ones are not recorded), one entry each with its name and elapsed
 * milliseconds, then starts a new record.  Not for concurrent use from
 * several threads.  Disabled by default; the events are created on first use
 * while enabled, and lli8_trace_enable(0) destroys them (call it once the
 * timed work has been read, so that no event outlives the caller's use of
 * the HIP runtime).
 */
#define LLI8_TRACE_MAX 8
typedef struct lli8_trace {
  int n;                             /* kernels since the last read */
  const char* name[LLI8_TRACE_MAX];  /* static strings           */
  float ms[LLI8_TRACE_MAX];
} lli8_trace_t;

void lli8_trace_enable(int on);
lli8_status_t lli8_trace_read(lli8_trace_t* out);

/* Static text for a status code. */
const char* lli8_status_string(lli8_status_t s);

/* Detail of the last LLI8_ERR_HIP or validation error on this thread. */
const char* lli8_last_error(void);

/* Library version, "major.minor.patch". */
const char* lli8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LLI8_H */
