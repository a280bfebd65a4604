"""Forward calls in flight together on separate streams, each with buffers of
its own: every result equals the same call run alone.  The library keeps no
per-call state outside the caller's workspace (the kernels read their sizes
from the arguments and their outlier list from the workspace), so calls that
share no buffers do not interact, whatever route each takes."""
import pytest

from tests.gpu_helpers import to_dev
from workloads import random_case

pytestmark = pytest.mark.gpu

# one shape per route: the persistent 256 x 256 walk, the ragged tile
# kernel, the weight-streaming kernel (17-64 tokens) and the fused decode
SHAPES = [(1024, 512, 8192), (600, 768, 520), (40, 512, 1024), (8, 1024, 2048)]


def _inputs(i, T, K, N, dtype):
    import torch
    import bit_quantized_matmul_amd as B
    case = random_case(T, K, N, seed=300 + i, n_out=1 + 2 * i)
    X = to_dev(case.X, dtype)
    W = to_dev(case.W, dtype)
    bias = to_dev(case.bias, dtype)
    CB, SCB = B.lli8_quant_weight_rowwise(W)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    return X, CB, SCB, bias, tdt


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_calls_on_separate_streams_match_serial(dtype):
    import torch
    import bit_quantized_matmul_amd as B
    ins = [_inputs(i, *s, dtype) for i, s in enumerate(SHAPES)]
    # each call alone, one after another on the current stream
    refs = []
    for X, CB, SCB, bias, _ in ins:
        out, ws = B.lli8_int8_linear(X, CB, SCB, bias, 6.0)
        torch.cuda.synchronize()
        n = int(ws.n_idx.item())
        refs.append((out.clone(), ws.CA.clone(), ws.SCA.clone(), ws.idx[:n].clone(), n))
    # all of them in flight together, three rounds each, one stream per call
    streams = [torch.cuda.Stream() for _ in SHAPES]
    outs, wss = [], []
    for (T, K, N), (X, CB, SCB, bias, tdt) in zip(SHAPES, ins):
        outs.append(torch.full((T, N), float("nan"), dtype=tdt, device="cuda"))
        wss.append(B.Workspace(T, K, N, tdt, "cuda"))
    torch.cuda.synchronize()
    for _ in range(3):
        for s, (X, CB, SCB, bias, _), out, ws in zip(streams, ins, outs, wss):
            with torch.cuda.stream(s):
                B.lli8_int8_linear(X, CB, SCB, bias, 6.0, out=out, ws=ws)
    torch.cuda.synchronize()
    for (T, K, N), ref, out, ws in zip(SHAPES, refs, outs, wss):
        r_out, r_CA, r_SCA, r_idx, n = ref
        assert int(ws.n_idx.item()) == n, (T, K, N)
        assert torch.equal(ws.idx[:n], r_idx), (T, K, N)
        assert torch.equal(ws.CA, r_CA), (T, K, N)
        assert torch.equal(ws.SCA[:T], r_SCA[:T]), (T, K, N)
        assert torch.equal(out.view(torch.int16), r_out.view(torch.int16)), (T, K, N)


def test_shared_weights_on_two_streams():
    """Two calls reading the same CB / SCB (one quantised weight), each with
    its own activation, output and workspace, in flight together."""
    import torch
    import bit_quantized_matmul_amd as B
    T, K, N = 1024, 512, 8192
    ca, cb = random_case(T, K, N, seed=311, n_out=2), random_case(T, K, N, seed=312, n_out=6)
    W = to_dev(ca.W, "f16")
    bias = to_dev(ca.bias, "f16")
    CB, SCB = B.lli8_quant_weight_rowwise(W)
    Xs = [to_dev(ca.X, "f16"), to_dev(cb.X, "f16")]
    refs = []
    for X in Xs:
        out, _ = B.lli8_int8_linear(X, CB, SCB, bias, 6.0)
        torch.cuda.synchronize()
        refs.append(out.clone())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty((T, N), dtype=torch.float16, device="cuda") for _ in Xs]
    wss = [B.Workspace(T, K, N, torch.float16, "cuda") for _ in Xs]
    torch.cuda.synchronize()
    for _ in range(3):
        for s, X, out, ws in zip(streams, Xs, outs, wss):
            with torch.cuda.stream(s):
                B.lli8_int8_linear(X, CB, SCB, bias, 6.0, out=out, ws=ws)
    torch.cuda.synchronize()
    for ref, out in zip(refs, outs):
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
