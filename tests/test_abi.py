"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments before touching the GPU (these calls enqueue nothing, so
they run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lli8.h")


def _lib():
    from bit_quantized_matmul_amd import _lib as L
    if not os.path.exists(L.library_path()):
        pytest.skip("liblli8.so not built (run `python -m bit_quantized_matmul_amd.build`)")
    return L


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lli8_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("lli8_quant_weight_rowwise", "lli8_quant_rowwise_outliers", "lli8_int8_linear",
              "lli8_recover_weight", "lli8_workspace_bytes", "lli8_workspace_carve"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    raw = ctypes.CDLL(L.library_path())
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} declared in lli8.h but not exported"


def test_version_and_status_strings():
    L = _lib()
    assert re.match(r"^\d+\.\d+\.\d+$", L.lli8_version())
    for code in range(0, 9):
        assert L.lli8_status_string(code) and L.lli8_status_string(code) != "unknown status"
    assert L.lli8_status_string(99) == "unknown status"


def test_scratch_bytes():
    L = _lib()
    assert L.lli8_scratch_bytes(0, 64) == 0
    assert L.lli8_scratch_bytes(8, 64) == 8 * 64 * 2
    assert L.lli8_scratch_bytes(8, 65) == 8 * 96 * 2
    assert L.lli8_scratch_bytes(4096, 12288, L.LLI8_BF16) == 4096 * 12288 * 2
    assert L.lli8_scratch_bytes_full(8, 65, 10) == 8 * 96 * 2 + 10 * 96 * 2
    assert L.lli8_scratch_bytes_full(0, 64, 10) == 0


FAKE = 0x100000  # a 16-byte aligned non-null address; never dereferenced


def _ws(L, **over):
    vals = dict(CA=FAKE, SCA=FAKE, bitmap=FAKE, idx=FAKE, n_idx=FAKE, acc=None,
                scratch=FAKE, scratch_bytes=1 << 40)
    vals.update(over)
    return L._Workspace(**vals)


def test_validation_weight_quant():
    L = _lib().lib()
    f = L.lli8_quant_weight_rowwise
    assert f(FAKE, 4, 8, 7, FAKE, FAKE, None) == 3          # dtype
    assert f(FAKE, -1, 8, 0, FAKE, FAKE, None) == 2         # N < 0
    assert f(FAKE, 4, 0, 0, FAKE, FAKE, None) == 2          # K < 1
    assert f(FAKE, 4, 133145, 0, FAKE, FAKE, None) == 6     # K too large
    assert f(None, 4, 8, 0, FAKE, FAKE, None) == 1          # W NULL
    assert f(FAKE, 4, 8, 0, None, FAKE, None) == 1          # CB NULL
    assert f(FAKE + 2, 4, 8, 0, FAKE, FAKE, None) == 4      # misaligned
    assert f(FAKE, 0, 8, 0, FAKE, FAKE, None) == 0          # empty: a no-op
    assert b"CB is NULL" in L.lli8_last_error() or True


def test_validation_activation_split():
    L = _lib().lib()
    f = L.lli8_quant_rowwise_outliers
    args = [FAKE, 4, 8, 0, 6.0, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    bad = list(args); bad[4] = float("nan")
    assert f(*bad) == 5
    bad = list(args); bad[3] = 2
    assert f(*bad) == 3
    bad = list(args); bad[1] = -1
    assert f(*bad) == 2
    for pos in (0, 5, 6, 7, 8, 9):
        bad = list(args); bad[pos] = None
        assert f(*bad) == 1
        bad = list(args); bad[pos] = FAKE + 4
        assert f(*bad) == 4


def test_validation_vectorwise():
    L = _lib().lib()
    f = L.lli8_quant_vectorwise
    args = [FAKE, 4, 8, 0, 1, 0, FAKE, FAKE, FAKE, None]
    assert f(*args[:3], 5, *args[4:]) == 3                      # dtype
    assert f(*args[:4], 2, *args[5:]) == 6                      # scheme
    assert f(*args[:5], 3, *args[6:]) == 6                      # axis
    assert f(FAKE, -1, 8, 0, 1, 0, FAKE, FAKE, FAKE, None) == 2  # R < 0
    assert f(FAKE, 4, -8, 0, 1, 0, FAKE, FAKE, FAKE, None) == 2  # C < 0
    for pos in (0, 6, 7, 8):
        bad = list(args); bad[pos] = None
        assert f(*bad) == 1
        bad = list(args); bad[pos] = FAKE + 8
        assert f(*bad) == 4
    absmax = list(args); absmax[4] = 0; absmax[8] = None          # no zero point for absmax: allowed
    absmax[0] = None                                              # ... but X is still required
    assert f(*absmax) == 1
    assert f(FAKE, 0, 8, 0, 1, 0, FAKE, FAKE, FAKE, None) == 0    # no rows: a no-op
    assert f(FAKE, 4, 0, 0, 1, 1, FAKE, FAKE, FAKE, None) == 0    # no columns, column-wise: a no-op


def test_validation_linear():
    Lm = _lib()
    L = Lm.lib()
    f = L.lli8_int8_linear

    def call(ws=None, **kw):
        a = dict(X=FAKE, T=4, K=8, N=3, dt=0, CB=FAKE, SCB=FAKE, bias=None, tau=6.0, out=FAKE)
        a.update(kw)
        w = _ws(Lm) if ws is None else ws
        return f(a["X"], a["T"], a["K"], a["N"], a["dt"], a["CB"], a["SCB"], a["bias"], a["tau"],
                 a["out"], ctypes.byref(w), None)

    assert call(tau=float("nan")) == 5
    assert call(dt=5) == 3
    assert call(T=-1) == 2 and call(N=0) == 2 and call(K=0) == 2
    assert call(K=200000) == 6
    assert call(X=None) == 1 and call(CB=None) == 1 and call(SCB=None) == 1 and call(out=None) == 1
    assert call(T=0, X=None, out=None, K=200000) == 6  # size checks still apply
    assert call(bias=FAKE + 8) == 4
    assert call(ws=_ws(Lm, CA=None)) == 1
    assert call(ws=_ws(Lm, n_idx=FAKE + 4)) == 4
    assert call(ws=_ws(Lm, scratch=None)) == 8
    assert call(ws=_ws(Lm, scratch_bytes=10)) == 8
    assert f(FAKE, 4, 8, 3, 0, FAKE, FAKE, None, 6.0, FAKE, None, None) == 1  # workspace NULL
    assert b"scratch" in L.lli8_last_error() or b"workspace" in L.lli8_last_error()


def test_validation_recover_weight():
    L = _lib().lib()
    f = L.lli8_recover_weight
    assert f(FAKE, FAKE, 4, 8, 3, FAKE, None) == 3                # dtype
    assert f(FAKE, FAKE, -1, 8, 0, FAKE, None) == 2               # N < 0
    assert f(FAKE, FAKE, 4, -8, 0, FAKE, None) == 2               # K < 0
    for pos in (0, 1, 5):
        args = [FAKE, FAKE, 4, 8, 0, FAKE, None]
        args[pos] = None
        assert f(*args) == 1
        args[pos] = FAKE + 4
        assert f(*args) == 4
    assert f(None, None, 0, 8, 0, None, None) == 0                # nothing to do


def test_validation_mfma_loop():
    """The calibration loop refuses bad arguments before touching a device."""
    import ctypes
    L = _lib().lib()
    ops = ctypes.c_double(0.0)
    f = L.lli8_mfma_i8_loop
    assert f(0, 0, FAKE, ctypes.byref(ops), None) == 2           # iters < 1
    assert f(8, 2, FAKE, ctypes.byref(ops), None) == 6           # unknown operand pattern
    assert f(8, -1, FAKE, ctypes.byref(ops), None) == 6
    assert f(8, 0, None, ctypes.byref(ops), None) == 1           # sink NULL
    assert f(8, 1, FAKE + 4, ctypes.byref(ops), None) == 4       # sink misaligned
    assert f(8, 0, FAKE, None, None) == 1                        # ops NULL


def test_workspace_bytes_and_carve():
    """One buffer split into the forward's buffers: every piece 256-byte
    aligned, in bounds, not overlapping, with room for 8 recovered-weight
    chunks in the scratch; nothing is written to the (fake) device address."""
    Lm = _lib()
    L = Lm.lib()
    for T, K, N in [(0, 64, 8), (1, 1, 1), (16, 4096, 4096), (4096, 12288, 49152), (37, 100, 3)]:
        nb = Lm.lli8_workspace_bytes(T, K, N)
        ws = Lm._Workspace()
        base = 0x10000000
        assert L.lli8_workspace_carve(base, nb, T, K, N, 0, ctypes.byref(ws)) == 0
        pieces = [(ws.CA, T * K), (ws.SCA, 4 * max(T, 1)), (ws.bitmap, 4 * ((K + 31) // 32)),
                  (ws.idx, 4 * K), (ws.n_idx, 4), (ws.scratch, ws.scratch_bytes)]
        ends = []
        for ptr, size in pieces:
            ptr = ptr or base  # ctypes gives None for address 0 offsets; base is never 0 here
            assert (ptr - base) % 256 == 0 and base <= ptr and ptr + size <= base + nb
            ends.append((ptr, ptr + size))
        ends.sort()
        assert all(a[1] <= b[0] for a, b in zip(ends, ends[1:]))
        assert ws.acc is None
        assert ws.scratch_bytes >= Lm.lli8_scratch_bytes(T, K) + N * 64 * min((K + 31) // 32, 8)
        assert L.lli8_workspace_carve(base, nb - 1, T, K, N, 0, ctypes.byref(ws)) == 8
    assert L.lli8_workspace_carve(0x10000008, 1 << 30, 4, 8, 3, 0, ctypes.byref(ws)) == 4
    assert L.lli8_workspace_carve(None, 1 << 30, 4, 8, 3, 0, ctypes.byref(ws)) == 1
    assert L.lli8_workspace_carve(0x10000000, 1 << 30, 4, 8, 3, 0, None) == 1
    assert L.lli8_workspace_carve(0x10000000, 1 << 30, 4, 0, 3, 0, ctypes.byref(ws)) == 2
    assert Lm.lli8_workspace_bytes(4, 0, 3) == 0


def test_binding_rejects_host_and_mismatched_tensors():
    """The binding raises before any launch for tensors a kernel would read
    or write out of bounds: host tensors, wrong dtypes, short buffers, a
    workspace of other sizes (no GPU is touched: every check fails first)."""
    import torch
    Lm = _lib()
    X = torch.zeros((4, 8), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU only"):
        Lm.lli8_int8_linear(X, torch.zeros((3, 8), dtype=torch.int8), torch.zeros(3))
    with pytest.raises(ValueError, match="GPU only"):
        Lm.lli8_quant_weight_rowwise(torch.zeros((3, 8), dtype=torch.float16))
    with pytest.raises(ValueError, match="GPU only"):
        Lm.lli8_quant_rowwise_outliers(X, 6.0)
    with pytest.raises(ValueError, match="GPU only"):
        Lm.lli8_quant_vectorwise(X)
    with pytest.raises(ValueError, match="GPU only"):
        Lm.lli8_recover_weight(torch.zeros((3, 8), dtype=torch.int8), torch.zeros(3))
    # the per-operand checks, on tensors standing in for device tensors
    dev = torch.device("cpu")
    good = torch.zeros(6, dtype=torch.float32)
    Lm._arg(good, "SCB", dev, torch.float32, 6)
    with pytest.raises(TypeError, match="dtype"):
        Lm._arg(good, "SCB", dev, torch.float16, 6)
    with pytest.raises(ValueError, match="elements"):
        Lm._arg(good, "SCB", dev, torch.float32, 7)
    with pytest.raises(ValueError, match="shape"):
        Lm._arg(good.view(2, 3), "CB", dev, torch.float32, 6, (3, 2))
    with pytest.raises(ValueError, match="contiguous"):
        Lm._arg(torch.zeros((3, 2)).t(), "CB", dev, torch.float32, 6)
    with pytest.raises(ValueError, match="on meta"):
        Lm._arg(torch.zeros(6, device="meta"), "bias", dev, torch.float32, 6)


def test_package_exports_every_binding_function():
    import bit_quantized_matmul_amd as B
    from bit_quantized_matmul_amd import _lib as L
    public = [n for n in dir(L) if n.startswith("lli8_") and callable(getattr(L, n))]
    assert public
    for n in public:
        assert getattr(B, n, None) is getattr(L, n), f"{n} is not exported by the package"
        assert n in B.__all__


def test_product_path_has_no_cpu_fallback():
    """The package's compute entry points go only through the HIP library."""
    pkg = os.path.join(ROOT, "bit_quantized_matmul_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "import oracle" not in src and "from oracle" not in src
            assert "workloads" not in src
