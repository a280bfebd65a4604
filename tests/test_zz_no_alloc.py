"""lli8_int8_linear_noalloc (workspace in the library's fixed per-GPU array)
gives the output of lli8_int8_linear (caller workspace) bit for bit, on two
calls in a row, the second with a smaller input, each also within the
oracle's output bound; sizes beyond the array are refused before anything
is enqueued."""
import ctypes

import numpy as np
import pytest

import oracle as O
from tests.gpu_helpers import assert_out, bits_of, to_dev
from workloads import random_case

pytestmark = pytest.mark.gpu


def _raw_noalloc(B, X, CB, SCB, bias, tau, out):
    """The C entry point itself, through ctypes (no binding logic)."""
    import torch
    T, K = X.shape
    N = CB.shape[0]
    dt = 0 if X.dtype == torch.float16 else 1
    stream = torch.cuda.current_stream().cuda_stream
    return B.lib().lli8_int8_linear_noalloc(X.data_ptr(), T, K, N, dt, CB.data_ptr(), SCB.data_ptr(),
                                            bias.data_ptr() if bias is not None else None, ctypes.c_float(tau),
                                            out.data_ptr(), ctypes.c_void_p(stream))


@pytest.mark.parametrize("first,second", [
    ((600, 768, 520, "f16"), (16, 512, 300, "f16")),    # 128 x 128 tiles, then the one-launch decode
    ((2048, 1024, 4096, "bf16"), (48, 2048, 1000, "bf16")),  # persistent tiles, then weight streaming
])
def test_noalloc_matches_workspace_entry_point(first, second):
    import torch
    import bit_quantized_matmul_amd as B
    for T, K, N, dt in (first, second):
        case = random_case(T, K, N, dtype=dt, seed=T + K + N, n_out=5)
        print(f"[no-alloc] T={T} K={K} N={N} {dt}", flush=True)
        X, W, bias = to_dev(case.X, dt), to_dev(case.W, dt), to_dev(case.bias, dt)
        CB, SCB = B.lli8_quant_weight_rowwise(W)
        ref, _ = B.lli8_int8_linear(X, CB, SCB, bias, case.threshold)
        out = torch.full((T, N), float("nan"), dtype=X.dtype, device=X.device)
        st = _raw_noalloc(B, X, CB, SCB, bias, case.threshold, out)
        torch.cuda.synchronize()
        assert st == 0, B.lib().lli8_last_error()
        assert torch.equal(out, ref)
        rCB, rSCB = O.quantize_weight_bits(case.W, dt)
        r = O.linear_forward(case.X, dt, rCB, rSCB, case.bias, case.threshold)
        assert_out(bits_of(out), r, dt)
        got = B.lli8_int8_linear_noalloc(X, CB, SCB, bias, case.threshold)  # through the binding too
        torch.cuda.synchronize()
        assert torch.equal(got, ref)


def test_noalloc_refuses_sizes_beyond_the_array():
    import torch
    import bit_quantized_matmul_amd as B
    T, K, N = 4096, 12288, 64
    assert B.lli8_workspace_bytes(T, K, N) > B.lli8_noalloc_scratch_bytes()
    X = torch.zeros((T, K), dtype=torch.float16, device="cuda")
    CB = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    SCB = torch.zeros(N, dtype=torch.float32, device="cuda")
    out = torch.zeros((T, N), dtype=torch.float16, device="cuda")
    assert _raw_noalloc(B, X, CB, SCB, None, 6.0, out) == 6  # LLI8_ERR_UNSUPPORTED
    assert b"no-allocation" in B.lib().lli8_last_error()
    torch.cuda.synchronize()
    assert not out.any()  # nothing was enqueued
