"""ctypes declarations of include/lli8.h and argument marshalling for torch tensors."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "liblli8.so"

LLI8_F16 = 0
LLI8_BF16 = 1
LLI8_ABSMAX, LLI8_ZEROPOINT = 0, 1   # lli8_scheme_t
LLI8_ROWS, LLI8_COLS = 0, 1          # lli8_axis_t

STATUS = {0: "LLI8_OK", 1: "LLI8_ERR_NULL", 2: "LLI8_ERR_SHAPE", 3: "LLI8_ERR_DTYPE",
          4: "LLI8_ERR_ALIGN", 5: "LLI8_ERR_THRESHOLD", 6: "LLI8_ERR_UNSUPPORTED",
          7: "LLI8_ERR_HIP", 8: "LLI8_ERR_WORKSPACE"}


class Lli8Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


class _Workspace(ctypes.Structure):
    _fields_ = [("CA", ctypes.c_void_p), ("SCA", ctypes.c_void_p), ("bitmap", ctypes.c_void_p),
                ("idx", ctypes.c_void_p), ("n_idx", ctypes.c_void_p), ("acc", ctypes.c_void_p),
                ("scratch", ctypes.c_void_p), ("scratch_bytes", ctypes.c_size_t)]


TRACE_MAX = 8


class _Trace(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int), ("name", ctypes.c_char_p * TRACE_MAX),
                ("ms", ctypes.c_float * TRACE_MAX)]


def lli8_trace_enable(on: bool = True):
    lib().lli8_trace_enable(1 if on else 0)


def lli8_trace_read():
    """[(kernel name, ms)] for the kernels enqueued since the previous read (waits for them)."""
    t = _Trace()
    _check(lib().lli8_trace_read(ctypes.byref(t)))
    return [(t.name[i].decode(), float(t.ms[i])) for i in range(t.n)]


def library_path() -> str:
    return os.environ.get("LLI8_LIBRARY", os.path.join(HERE, LIB_NAME))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m bit_quantized_matmul_amd.build`"
                          " (the HIP library is required; there is no CPU fallback)")
    L = ctypes.CDLL(path)
    i64, vp, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    L.lli8_quant_weight_rowwise.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    L.lli8_quant_weight_rowwise.restype = i32
    L.lli8_quant_rowwise_outliers.argtypes = [vp, i64, i64, i32, f32, vp, vp, vp, vp, vp, vp]
    L.lli8_quant_rowwise_outliers.restype = i32
    L.lli8_int8_linear.argtypes = [vp, i64, i64, i64, i32, vp, vp, vp, f32, vp,
                                   ctypes.POINTER(_Workspace), vp]
    L.lli8_int8_linear.restype = i32
    L.lli8_quant_vectorwise.argtypes = [vp, i64, i64, i32, i32, i32, vp, vp, vp, vp]
    L.lli8_quant_vectorwise.restype = i32
    L.lli8_int8_linear_noalloc.argtypes = [vp, i64, i64, i64, i32, vp, vp, vp, f32, vp, vp]
    L.lli8_int8_linear_noalloc.restype = i32
    L.lli8_noalloc_scratch_bytes.argtypes = []
    L.lli8_noalloc_scratch_bytes.restype = ctypes.c_size_t
    L.lli8_recover_weight.argtypes = [vp, vp, i64, i64, i32, vp, vp]
    L.lli8_recover_weight.restype = i32
    L.lli8_workspace_bytes.argtypes = [i64, i64, i64, i32]
    L.lli8_workspace_bytes.restype = ctypes.c_size_t
    L.lli8_workspace_carve.argtypes = [vp, ctypes.c_size_t, i64, i64, i64, i32, ctypes.POINTER(_Workspace)]
    L.lli8_workspace_carve.restype = i32
    L.lli8_scratch_bytes.argtypes = [i64, i64, i32]
    L.lli8_scratch_bytes.restype = ctypes.c_size_t
    L.lli8_scratch_bytes_full.argtypes = [i64, i64, i64, i32]
    L.lli8_scratch_bytes_full.restype = ctypes.c_size_t
    L.lli8_status_string.argtypes = [i32]
    L.lli8_status_string.restype = ctypes.c_char_p
    L.lli8_last_error.argtypes = []
    L.lli8_last_error.restype = ctypes.c_char_p
    L.lli8_version.argtypes = []
    L.lli8_version.restype = ctypes.c_char_p
    L.lli8_mfma_i8_loop.argtypes = [i64, i32, vp, ctypes.POINTER(ctypes.c_double), vp]
    L.lli8_mfma_i8_loop.restype = i32
    L.lli8_mfma_i8_loop_sink_ints.argtypes = []
    L.lli8_mfma_i8_loop_sink_ints.restype = ctypes.c_size_t
    L.lli8_trace_enable.argtypes = [i32]
    L.lli8_trace_enable.restype = None
    L.lli8_trace_read.argtypes = [ctypes.POINTER(_Trace)]
    L.lli8_trace_read.restype = i32
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise Lli8Error(status, lib().lli8_last_error().decode())


def lli8_version() -> str:
    return lib().lli8_version().decode()


def lli8_status_string(status: int) -> str:
    return lib().lli8_status_string(status).decode()


def lli8_scratch_bytes(T: int, K: int, dtype: int = LLI8_F16) -> int:
    return int(lib().lli8_scratch_bytes(T, K, dtype))


def lli8_scratch_bytes_full(T: int, K: int, N: int, dtype: int = LLI8_F16) -> int:
    return int(lib().lli8_scratch_bytes_full(T, K, N, dtype))


# ------------------------------------------------------------ torch glue ----

def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return LLI8_F16
    if t.dtype == torch.bfloat16:
        return LLI8_BF16
    raise TypeError(f"dtype {t.dtype} is not float16 or bfloat16")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to lli8 must be contiguous")
    return t.data_ptr()


def _gpu(t, name: str):
    """t must be a contiguous tensor on a GPU; returns its device."""
    if not t.is_cuda:
        raise ValueError(f"{name} is on {t.device}: lli8 runs on the GPU only (no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.device


def _arg(t, name: str, device, dtype, numel: int, shape=None):
    """A caller buffer: on `device`, of `dtype`, contiguous, holding `numel`
    elements (and of `shape` when given).  Raises before anything is enqueued:
    a host tensor or a short buffer would make a kernel read or write outside
    device memory."""
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


_raw_stream = None


def _stream(device, stream=None) -> int:
    """The HIP stream to enqueue on: `stream`, else torch's current stream of
    `device` (queried through torch's raw-handle accessor when it has one,
    which costs a small fraction of building a Stream object)."""
    global _raw_stream
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    torch = _torch()
    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _raw_stream:
        idx = device.index if device.index is not None else torch.cuda.current_device()
        return _raw_stream(idx)
    return torch.cuda.current_stream(device).cuda_stream


def lli8_quant_weight_rowwise(W, CB=None, SCB=None, stream=None):
    """W [N, K] fp16/bf16 on the GPU -> (CB int8 [N, K], SCB fp32 [N])."""
    torch = _torch()
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N, K]")
    dev = _gpu(W, "W")
    N, K = W.shape
    if CB is None:
        CB = torch.empty((N, K), dtype=torch.int8, device=dev)
    if SCB is None:
        SCB = torch.empty((N,), dtype=torch.float32, device=dev)
    _arg(CB, "CB", dev, torch.int8, N * K, (N, K))
    _arg(SCB, "SCB", dev, torch.float32, N)
    _check(lib().lli8_quant_weight_rowwise(_ptr(W), N, K, _dt(W), _ptr(CB), _ptr(SCB),
                                           _stream(W.device, stream)))
    return CB, SCB


def lli8_quant_rowwise_outliers(X, threshold: float, CA=None, SCA=None, bitmap=None, idx=None,
                                n_idx=None, stream=None):
    """X [T, K] -> (CA, SCA, bitmap, idx, n_idx); idx[:n_idx] are the outlier columns."""
    torch = _torch()
    dev = _gpu(X, "X")
    X2 = X.reshape(-1, X.shape[-1])
    T, K = X2.shape
    CA = torch.empty((T, K), dtype=torch.int8, device=dev) if CA is None else CA
    SCA = torch.empty((T,), dtype=torch.float32, device=dev) if SCA is None else SCA
    bitmap = torch.empty(((K + 31) // 32,), dtype=torch.int32, device=dev) if bitmap is None else bitmap
    idx = torch.empty((K,), dtype=torch.int32, device=dev) if idx is None else idx
    n_idx = torch.empty((1,), dtype=torch.int32, device=dev) if n_idx is None else n_idx
    _arg(CA, "CA", dev, torch.int8, T * K)
    _arg(SCA, "SCA", dev, torch.float32, T)
    _arg(bitmap, "bitmap", dev, torch.int32, (K + 31) // 32)
    _arg(idx, "idx", dev, torch.int32, K)
    _arg(n_idx, "n_idx", dev, torch.int32, 1)
    _check(lib().lli8_quant_rowwise_outliers(_ptr(X2), T, K, _dt(X2), float(threshold), _ptr(CA),
                                             _ptr(SCA), _ptr(bitmap), _ptr(idx), _ptr(n_idx),
                                             _stream(dev, stream)))
    return CA, SCA, bitmap, idx, n_idx


def lli8_recover_weight(CB, SCB, dtype=None, W=None, stream=None):
    """(CB * SCB) / 127 in a 16-bit dtype (float16 by default), the weight the
    int8 codes stand for: W[n, k] = dtype(fl32(fl32(CB[n, k] * SCB[n]) / 127))."""
    torch = _torch()
    if CB.dim() != 2:
        raise ValueError("CB must be 2-D [N, K]")
    dev = _gpu(CB, "CB")
    N, K = CB.shape
    _arg(CB, "CB", dev, torch.int8, N * K)
    _arg(SCB, "SCB", dev, torch.float32, N)
    dtype = (W.dtype if W is not None else torch.float16) if dtype is None else dtype
    if W is None:
        W = torch.empty((N, K), dtype=dtype, device=dev)
    _arg(W, "W", dev, dtype, N * K)
    _check(lib().lli8_recover_weight(_ptr(CB), _ptr(SCB), N, K, _dt(W), _ptr(W), _stream(dev, stream)))
    return W


def lli8_mfma_i8_loop(iters: int, sink=None, device=None, stream=None, pattern: int = 0):
    """Calibration (not a step of the method): a loop of int8 matrix-core
    instructions on register operands, one workgroup per compute unit.
    pattern 0: every operand byte 1; pattern 1: pseudo-random operand bytes
    (their definition is in the C header).  Returns (sink, ops): sink int32
    [lli8_mfma_i8_loop_sink_ints()], thread t's accumulator sum once the
    launch is done ((4096 * iters) mod 2^32 for pattern 0); ops the int8
    operations the launch performs."""
    torch = _torch()
    n = int(lib().lli8_mfma_i8_loop_sink_ints())
    dev = _gpu(sink, "sink") if sink is not None else torch.device("cuda", torch.cuda.current_device()
                                                                       if device is None else device)
    if sink is None:
        sink = torch.empty((n,), dtype=torch.int32, device=dev)
    _arg(sink, "sink", dev, torch.int32, n)
    ops = ctypes.c_double(0.0)
    _check(lib().lli8_mfma_i8_loop(int(iters), int(pattern), _ptr(sink), ctypes.byref(ops),
                                   _stream(dev, stream)))
    return sink, ops.value


def lli8_mfma_i8_loop_sink_ints() -> int:
    return int(lib().lli8_mfma_i8_loop_sink_ints())


def lli8_workspace_bytes(T: int, K: int, N: int, dtype: int = LLI8_F16) -> int:
    return int(lib().lli8_workspace_bytes(T, K, N, dtype))


def lli8_quant_vectorwise(X, scheme: str = "absmax", axis: str = "rows", codes=None, scale=None,
                          zero_point=None, stream=None):
    """X [R, C] fp16/bf16 -> (codes int8 [R, C], scale fp32, zero_point int32 or None),
    one scale per row (axis="rows") or per column (axis="cols"); scheme
    "absmax" (scale = max |x|) or "zeropoint" (scale = 254 / width of the
    range widened to contain 0, zero_point = the code of 0.0)."""
    torch = _torch()
    if scheme not in ("absmax", "zeropoint") or axis not in ("rows", "cols"):
        raise ValueError(f"scheme {scheme!r} / axis {axis!r}")
    if X.dim() != 2:
        raise ValueError("X must be 2-D [R, C]")
    R, C = X.shape
    nvec = R if axis == "rows" else C
    dev = _gpu(X, "X")
    codes = torch.empty((R, C), dtype=torch.int8, device=dev) if codes is None else codes
    scale = torch.empty((nvec,), dtype=torch.float32, device=dev) if scale is None else scale
    _arg(codes, "codes", dev, torch.int8, R * C)
    _arg(scale, "scale", dev, torch.float32, nvec)
    zp = None
    if scheme == "zeropoint":
        zp = torch.empty((nvec,), dtype=torch.int32, device=dev) if zero_point is None else zero_point
        _arg(zp, "zero_point", dev, torch.int32, nvec)
    _check(lib().lli8_quant_vectorwise(_ptr(X), R, C, _dt(X),
                                       LLI8_ZEROPOINT if scheme == "zeropoint" else LLI8_ABSMAX,
                                       LLI8_ROWS if axis == "rows" else LLI8_COLS,
                                       _ptr(codes), _ptr(scale), _ptr(zp), _stream(dev, stream)))
    return codes, scale, zp


class Workspace:
    """Caller-owned buffers of one forward call (torch tensors on one device).

    By default one device buffer of lli8_workspace_bytes(T, K, N) bytes,
    split by lli8_workspace_carve: CA, SCA, bitmap, idx, n_idx and a scratch
    with room for the recovered weights of 8 outlier chunks (256 columns).
    scratch_bytes="full" gives room for every possible outlier column
    (lli8_scratch_bytes_full: N * K * 2 bytes more, the fast path when most
    columns are outliers); an integer gives exactly that much scratch (at
    least lli8_scratch_bytes)."""

    def __init__(self, T: int, K: int, N: int, dtype, device, want_acc: bool = False,
                 scratch_bytes=None):
        torch = _torch()
        self.T, self.K, self.N = T, K, N
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.acc = torch.empty((T, N), dtype=torch.int32, device=device) if want_acc else None
        if scratch_bytes is None:
            nbytes = int(lib().lli8_workspace_bytes(T, K, N, LLI8_F16))
            if nbytes == 0:
                raise ValueError(f"invalid workspace sizes T={T} K={K} N={N}")
            self.buffer = torch.empty((nbytes,), dtype=torch.uint8, device=device)
            st = _Workspace()
            _check(lib().lli8_workspace_carve(self.buffer.data_ptr(), nbytes, T, K, N, LLI8_F16,
                                              ctypes.byref(st)))
            base = self.buffer.data_ptr()

            def view(ptr, count, dtype, shape):
                o = ptr - base
                return self.buffer[o:o + count * dtype.itemsize].view(dtype).view(shape)
            self.CA = view(st.CA, T * K, torch.int8, (T, K))
            self.SCA = view(st.SCA, max(T, 1), torch.float32, (max(T, 1),))
            self.bitmap = view(st.bitmap, (K + 31) // 32, torch.int32, ((K + 31) // 32,))
            self.idx = view(st.idx, K, torch.int32, (K,))
            self.n_idx = view(st.n_idx, 1, torch.int32, (1,))
            self.n_idx.zero_()
            self.scratch = view(st.scratch, max(st.scratch_bytes, 16), torch.uint8, (max(st.scratch_bytes, 16),))
            nbytes = st.scratch_bytes
        else:
            self.CA = torch.empty((T, K), dtype=torch.int8, device=device)
            self.SCA = torch.empty((max(T, 1),), dtype=torch.float32, device=device)
            self.bitmap = torch.empty(((K + 31) // 32,), dtype=torch.int32, device=device)
            self.idx = torch.empty((K,), dtype=torch.int32, device=device)
            self.n_idx = torch.zeros((1,), dtype=torch.int32, device=device)
            nbytes = (lli8_scratch_bytes_full(T, K, N, LLI8_F16) if scratch_bytes == "full"
                      else int(scratch_bytes))
            self.scratch = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=device)
        self._struct = _Workspace(self.CA.data_ptr(), self.SCA.data_ptr(), self.bitmap.data_ptr(),
                                  self.idx.data_ptr(), self.n_idx.data_ptr(),
                                  self.acc.data_ptr() if self.acc is not None else None,
                                  self.scratch.data_ptr(), nbytes)

    def fits(self, T, K, N, want_acc) -> bool:
        return (T, K, N) == (self.T, self.K, self.N) and (self.acc is not None or not want_acc)

    def outlier_columns(self):
        """The ascending outlier columns of the last call (copies to the host)."""
        n = int(self.n_idx.item())
        return self.idx[:n].cpu()


def lli8_int8_linear(X, CB, SCB, bias=None, threshold: float = 6.0, out=None,
                     ws: Optional[Workspace] = None, want_acc: bool = False, stream=None):
    """out = LLM.int8() forward of X [..., K] with the int8 weight (CB, SCB).

    Returns (out, ws); ws holds CA, SCA, bitmap, idx, n_idx (and acc when
    want_acc) of this call.
    """
    torch = _torch()
    dev = _gpu(X, "X")
    X2 = X if X.dim() == 2 else X.reshape(-1, X.shape[-1])
    T, K = X2.shape
    if CB.dim() != 2 or CB.shape[1] != K:
        raise ValueError(f"CB has shape {tuple(CB.shape)}, X has K={K}")
    N = CB.shape[0]
    _arg(CB, "CB", dev, torch.int8, N * K)
    _arg(SCB, "SCB", dev, torch.float32, N)
    if bias is not None:
        _arg(bias, "bias", dev, X.dtype, N)
    if ws is None:
        ws = Workspace(T, K, N, X.dtype, dev, want_acc)
    elif not ws.fits(T, K, N, want_acc) or ws.device != dev:
        raise ValueError(f"workspace for T={ws.T} K={ws.K} N={ws.N} on {ws.device}"
                         f"{' without acc' if ws.acc is None else ''} does not fit T={T} K={K} N={N} on {dev}")
    if out is None:
        out = torch.empty((T, N), dtype=X.dtype, device=dev)
    else:
        _arg(out, "out", dev, X.dtype, T * N)
    _check(lib().lli8_int8_linear(_ptr(X2), T, K, N, _dt(X2), _ptr(CB), _ptr(SCB), _ptr(bias),
                                  float(threshold), _ptr(out), ctypes.byref(ws._struct),
                                  _stream(X.device, stream)))
    return (out if X.dim() == 2 else out.reshape(*X.shape[:-1], N)), ws


def lli8_int8_linear_noalloc(X, CB, SCB, bias=None, threshold: float = 6.0, out=None, stream=None):
    """The forward of lli8_int8_linear with the workspace in the library's
    fixed per-GPU array (lli8_int8_linear_noalloc): the C call allocates
    nothing.  Pass `out` to keep this binding from allocating it.  Calls that
    overlap on one GPU race on the shared array."""
    torch = _torch()
    dev = _gpu(X, "X")
    X2 = X if X.dim() == 2 else X.reshape(-1, X.shape[-1])
    T, K = X2.shape
    if CB.dim() != 2 or CB.shape[1] != K:
        raise ValueError(f"CB has shape {tuple(CB.shape)}, X has K={K}")
    N = CB.shape[0]
    _arg(CB, "CB", dev, torch.int8, N * K)
    _arg(SCB, "SCB", dev, torch.float32, N)
    if bias is not None:
        _arg(bias, "bias", dev, X.dtype, N)
    if out is None:
        out = torch.empty((T, N), dtype=X.dtype, device=dev)
    else:
        _arg(out, "out", dev, X.dtype, T * N)
    _check(lib().lli8_int8_linear_noalloc(_ptr(X2), T, K, N, _dt(X2), _ptr(CB), _ptr(SCB), _ptr(bias),
                                          float(threshold), _ptr(out), _stream(dev, stream)))
    return out if X.dim() == 2 else out.reshape(*X.shape[:-1], N)


def lli8_noalloc_scratch_bytes() -> int:
    return int(lib().lli8_noalloc_scratch_bytes())
