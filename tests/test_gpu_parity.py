"""Parity of the HIP path (through the C-ABI) with the CPU oracle.

Bit-exact: CB, SCB, CA, SCA, the outlier bitmap, idx, n_idx and the int32
accumulators.  Output: normwise max-abs-rel <= 1e-2 (fp32 accumulation order
and the single final rounding differ from the oracle's float64 sum).
"""
import numpy as np
import pytest

import oracle as O
from tests import parity_cases as PC
from tests.gpu_helpers import assert_out, bits_of, to_dev
from workloads import config_case, random_case

pytestmark = pytest.mark.gpu


def _lib():
    import bit_quantized_matmul_amd as B
    return B


def _run(case, threshold=None, want_acc=True):
    """Quantise W on the GPU (placement step), run the forward; return everything."""
    B = _lib()
    import torch
    tau = case.threshold if threshold is None else threshold
    X = to_dev(case.X, case.dtype)
    W = to_dev(case.W, case.dtype)
    bias = to_dev(case.bias, case.dtype) if case.bias is not None else None
    CB, SCB = B.lli8_quant_weight_rowwise(W)
    out, ws = B.lli8_int8_linear(X, CB, SCB, bias, tau, want_acc=want_acc)
    torch.cuda.synchronize()
    n = int(ws.n_idx.item())
    return dict(CB=CB.cpu().numpy(), SCB=SCB.cpu().numpy(), CA=ws.CA.cpu().numpy(),
                SCA=ws.SCA[:case.T].cpu().numpy(), bitmap=ws.bitmap.cpu().numpy().view(np.uint32),
                idx=ws.idx[:n].cpu().numpy(), n=n,
                acc=ws.acc.cpu().numpy() if want_acc else None, out=bits_of(out))


def _check_full(case, threshold=None):
    tau = case.threshold if threshold is None else threshold
    g = _run(case, tau)
    CB, SCB = O.quantize_weight_bits(case.W, case.dtype)
    assert np.array_equal(g["SCB"], SCB), "SCB"
    assert np.array_equal(g["CB"], CB), "CB"
    r = O.linear_forward(case.X, case.dtype, CB, SCB, case.bias, tau)
    assert g["n"] == r["idx"].size, "n_idx"
    assert np.array_equal(g["idx"], r["idx"]), "idx"
    assert np.array_equal(g["bitmap"], O.outlier_bitmap(r["idx"], case.K)), "bitmap"
    assert np.array_equal(g["SCA"], r["SCA"]), "SCA"
    assert np.array_equal(g["CA"], r["CA"]), "CA"
    assert np.array_equal(g["acc"], r["acc"]), "acc"
    assert_out(g["out"], r, case.dtype)
    return g, r


def test_tiny_config():
    case = config_case("tiny")
    g, r = _check_full(case)
    assert g["idx"].tolist() == [3, 17]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,K,N", PC.SHAPES)
def test_random_shapes(T, K, N, dtype):
    _check_full(PC.shape_case(T, K, N, dtype))


@pytest.mark.parametrize("tau", PC.THRESHOLDS)
def test_thresholds(tau):
    case = PC.threshold_case()
    g, r = _check_full(case, tau)
    if tau <= 0 or tau == float("inf"):
        assert g["n"] == 0
    if tau == 0.1:
        assert g["n"] == case.K  # every column flagged, as in the issue's repro


def test_issue_repro_shape_all_columns():
    """x[2, 8] with threshold 0.1 flags all 8 columns (state.idx = [0..7])."""
    case = PC.issue_case()
    g, r = _check_full(case)
    assert g["idx"].tolist() == list(range(8))
    assert not g["CA"].any() and not g["SCA"].any() and not g["acc"].any()


def test_threshold_edge_exact_value():
    """A column whose largest magnitude is exactly the threshold is not flagged."""
    case = PC.threshold_edge_case()
    g, r = _check_full(case, 6.0)
    assert g["idx"].tolist() == [9]


def test_zero_rows_and_columns():
    case = PC.zero_rows_case()
    g, r = _check_full(case)
    assert g["SCA"][4] == 0 and not g["CA"][4].any()
    assert g["SCB"][3] == 0


def test_empty_T():
    B = _lib()
    import torch
    X = torch.zeros((0, 64), dtype=torch.float16, device="cuda")
    W = torch.randn((32, 64), dtype=torch.float16, device="cuda")
    CB, SCB = B.lli8_quant_weight_rowwise(W)
    out, ws = B.lli8_int8_linear(X, CB, SCB, None, 6.0)
    torch.cuda.synchronize()
    assert out.shape == (0, 32)
    assert int(ws.n_idx.item()) == 0
    assert not ws.bitmap.any()


def test_activation_split_entry_point():
    """lli8_quant_rowwise_outliers alone gives the same CA/SCA/idx as the oracle."""
    B = _lib()
    case = random_case(50, 320, 8, seed=21, n_out=5)
    CA, SCA, bitmap, idx, n_idx = B.lli8_quant_rowwise_outliers(to_dev(case.X, "f16"), 6.0)
    X = O.decode_bits(case.X, "f16")
    ridx, rCA, rSCA = O.quantize_activations(X, 6.0)
    n = int(n_idx.item())
    assert np.array_equal(idx[:n].cpu().numpy(), ridx)
    assert np.array_equal(CA.cpu().numpy(), rCA)
    assert np.array_equal(SCA.cpu().numpy(), rSCA)
    assert np.array_equal(bitmap.cpu().numpy().view(np.uint32), O.outlier_bitmap(ridx, case.K))


@pytest.mark.parametrize("T,K,N", PC.SCATTERED)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_scattered_outlier_flags_merge_across_the_chip(T, K, N, dtype):
    """Each outlier value in a single row, so that the bits of one bitmap
    word are set by workgroups on every compute die (the column scan ORs them
    into the bitmap with atomics): the bitmap, list, codes and output are the
    oracle's."""
    g, r = _check_full(PC.scattered_flags_case(T, K, N, dtype))
    assert g["n"] == min(K, 32) + len([j for j in range(32) if 64 + 3 * j < K])


@pytest.mark.parametrize("T,K,N", PC.WIDE_RATIO)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_outlier_far_beyond_16_bits_leaves_its_neighbour(T, K, N, dtype):
    """An outlier value up to 4e6 times its row's scale (a row of tiny kept
    values) beside a kept column, on every activation route: the kept
    neighbour's code, and everything else, as the oracle's."""
    g, r = _check_full(PC.wide_ratio_case(T, K, N, dtype))
    assert g["n"] == 3


def test_rounding_halves_on_gpu():
    """Row [127, 2.5, -2.5, 0.5, 1.5, -0.5] codes to [127, 3, -3, 1, 2, -1]."""
    B = _lib()
    import torch
    x = torch.tensor([[127, 2.5, -2.5, 0.5, 1.5, -0.5, 0, 0]], dtype=torch.float16, device="cuda")
    CA, SCA, _, _, n = B.lli8_quant_rowwise_outliers(x, 0.0)
    assert CA.cpu().tolist()[0][:6] == [127, 3, -3, 1, 2, -1]
    CB, SCB = B.lli8_quant_weight_rowwise(x)
    assert CB.cpu().tolist()[0][:6] == [127, 3, -3, 1, 2, -1]


def test_deterministic_repeat():
    case = random_case(300, 512, 260, seed=3, n_out=6)
    a = _run(case)
    b = _run(case)
    for k in ("CA", "SCA", "idx", "acc", "out"):
        assert np.array_equal(a[k], b[k]), k


def test_leading_dims_flatten():
    """nn.Linear semantics: leading dims flatten into T."""
    B = _lib()
    import torch
    case = random_case(2 * 3 * 5, 64, 24, seed=9, n_out=2)
    X = to_dev(case.X, "f16")
    W = to_dev(case.W, "f16")
    CB, SCB = B.lli8_quant_weight_rowwise(W)
    out2, _ = B.lli8_int8_linear(X, CB, SCB, None, 6.0)
    out3, _ = B.lli8_int8_linear(X.view(2, 3, 5, 64), CB, SCB, None, 6.0)
    torch.cuda.synchronize()
    assert out3.shape == (2, 3, 5, 24)
    assert torch.equal(out3.reshape(30, 24), out2)


@pytest.mark.parametrize("fused", ["1", "0"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,K,N", PC.SMALL_T)
def test_small_T_both_decode_paths(T, K, N, dtype, fused, monkeypatch):
    """T <= 16 runs the single-launch path by default; LLI8_FUSED_DECODE=0 selects the
    multi-kernel path.  Both must match the oracle."""
    monkeypatch.setenv("LLI8_FUSED_DECODE", fused)
    _check_full(PC.small_t_case(T, K, N, dtype))


@pytest.mark.parametrize("tau", PC.FUSED_THRESHOLDS)
def test_fused_decode_thresholds(tau):
    """Degenerate and dense thresholds on the single-launch path (T <= 16)."""
    _check_full(PC.fused_threshold_case(), tau)


def test_fused_decode_many_blocks_per_workgroup():
    """N well beyond one 16-feature block per CU: each workgroup walks several blocks."""
    _check_full(PC.fused_many_blocks_case())


@pytest.mark.parametrize("tau", [3.0, 2.0, 0.1])
def test_fused_decode_many_blocks_dense_outliers(tau):
    """Several blocks per workgroup with many outlier columns (42 at tau 3; 510 and all
    1024 at tau 2 and 0.1, beyond the 64 staged in LDS), so every block after the first
    sums its 16-bit product itself."""
    _check_full(PC.fused_many_blocks_dense_case(), tau)


@pytest.mark.parametrize("room_chunks", ["full", 0, 1])
def test_recovered_outlier_weights_scratch_sizes(room_chunks):
    """The recovered outlier weights come from scratch for as many 32-column
    chunks as fit and are gathered in the tiles for the rest; every split
    gives the oracle's results (here 70 outlier columns: three chunks)."""
    B = _lib()
    import torch
    case = PC.scratch_sizes_case()
    X = to_dev(case.X, case.dtype)
    W = to_dev(case.W, case.dtype)
    CB, SCB = B.lli8_quant_weight_rowwise(W)
    if room_chunks == "full":
        nbytes = "full"
    else:
        nbytes = B.lli8_scratch_bytes(case.T, case.K) + room_chunks * case.N * 64
    ws = B.Workspace(case.T, case.K, case.N, X.dtype, X.device, want_acc=True, scratch_bytes=nbytes)
    out, ws = B.lli8_int8_linear(X, CB, SCB, None, case.threshold, ws=ws, want_acc=True)
    torch.cuda.synchronize()
    rCB, rSCB = O.quantize_weight_bits(case.W, case.dtype)
    r = O.linear_forward(case.X, case.dtype, rCB, rSCB, None, case.threshold)
    assert int(ws.n_idx.item()) == r["idx"].size == 70
    assert np.array_equal(ws.acc.cpu().numpy(), r["acc"])
    assert_out(bits_of(out), r, case.dtype)


def test_every_column_an_outlier_skips_nothing_it_needs():
    """All K columns flagged (tiny threshold): the int8 product is skipped and
    the output is the 16-bit product alone."""
    case = PC.every_column_case()
    g, r = _check_full(case, 0.01)
    assert g["n"] == case.K
    assert not g["acc"].any()


@pytest.mark.parametrize("T,K,N", [(16, 4096, 512), (600, 768, 520)])
def test_graph_replays_match_eager(T, K, N):
    """The whole call captured in a HIP graph (torch.cuda.graph on a side
    stream) and replayed several times, with eager calls on other inputs in
    between: every replay equals the eager result on its own input."""
    import torch
    B = _lib()
    ca, cb = random_case(T, K, N, seed=71, n_out=3), random_case(T, K, N, seed=72, n_out=5)
    Xa, Xb = to_dev(ca.X, "f16"), to_dev(cb.X, "f16")
    W = to_dev(ca.W, "f16")
    bias = to_dev(ca.bias, "f16")
    CB, SCB = B.lli8_quant_weight_rowwise(W)
    ws = B.Workspace(T, K, N, torch.float16, "cuda")
    out = torch.empty((T, N), dtype=torch.float16, device="cuda")
    ref_a, _ = B.lli8_int8_linear(Xa, CB, SCB, bias, 6.0)
    ref_b, _ = B.lli8_int8_linear(Xb, CB, SCB, bias, 6.0)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        B.lli8_int8_linear(Xa, CB, SCB, bias, 6.0, out=out, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        B.lli8_int8_linear(Xa, CB, SCB, bias, 6.0, out=out, ws=ws)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_a)
        got_b, _ = B.lli8_int8_linear(Xb, CB, SCB, bias, 6.0, out=out, ws=ws)  # eager, same buffers
        torch.cuda.synchronize()
        assert torch.equal(got_b, ref_b)


def test_workspace_reused_across_outlier_paths():
    """One workspace through calls whose outlier columns move between the
    paths of the persistent kernel (five chunks staged through LDS, a few
    taken from registers, every column an outlier, none at all) and back:
    each call equals the oracle, so nothing an earlier call left in the
    workspace (bitmap, list, count, recovered weights) reaches a later one."""
    import torch
    B = _lib()
    T, K, N = 512, 256, 16384  # 128 whole 256 x 256 tiles: the persistent kernel
    base = random_case(T, K, N, seed=801, n_out=0)
    W = to_dev(base.W, "f16")
    bias = to_dev(base.bias, "f16")
    CB, SCB = B.lli8_quant_weight_rowwise(W)
    CBr, SCBr = O.quantize_weight_bits(base.W, "f16")
    assert np.array_equal(CB.cpu().numpy(), CBr)
    ws = B.Workspace(T, K, N, torch.float16, "cuda", want_acc=True)
    out = torch.empty((T, N), dtype=torch.float16, device="cuda")
    for i, (n_out, tau) in enumerate([(150, 6.0), (3, 6.0), (0, 0.01), (2, 0.0), (100, 6.0), (150, 6.0)]):
        case = random_case(T, K, N, seed=810 + i, n_out=n_out)
        B.lli8_int8_linear(to_dev(case.X, "f16"), CB, SCB, bias, tau, out=out, ws=ws, want_acc=True)
        torch.cuda.synchronize()
        r = O.linear_forward(case.X, "f16", CBr, SCBr, base.bias, tau)
        n = int(ws.n_idx.item())
        assert n == r["idx"].size, (i, n_out, tau)
        assert np.array_equal(ws.idx[:n].cpu().numpy(), r["idx"]), (i, n_out, tau)
        assert np.array_equal(ws.bitmap.cpu().numpy().view(np.uint32), O.outlier_bitmap(r["idx"], K)), i
        assert np.array_equal(ws.CA.cpu().numpy(), r["CA"]), i
        assert np.array_equal(ws.SCA[:T].cpu().numpy(), r["SCA"]), i
        assert np.array_equal(ws.acc.cpu().numpy(), r["acc"]), i
        assert_out(bits_of(out), r, "f16", what=f"call {i} (n_out={n_out}, tau={tau})")


@pytest.mark.parametrize("T,K,N,n_out,tau,dtype", PC.PERSISTENT)
def test_persistent_tiles(T, K, N, n_out, tau, dtype):
    case = PC.persistent_case(T, K, N, n_out, tau, dtype)
    g, r = _check_full(case, tau)
    if tau == 0.0:
        assert g["n"] == 0
    else:
        assert g["n"] >= min(n_out, K) and (tau > 0.1 or g["n"] == K)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,K,N,n_out,tau", PC.MANY_CHUNKS)
def test_many_outlier_chunks_large_tiles(T, K, N, n_out, tau, dtype):
    case = PC.many_chunks_case(T, K, N, n_out, tau, dtype)
    g, r = _check_full(case, tau)
    assert g["n"] >= min(n_out, K) and (tau > 0.1 or g["n"] == K)


@pytest.mark.parametrize("n_out", [1, 31, 32, 33, 100])
def test_persistent_route_recovered_outlier_weights(n_out):
    """On the persistent 256 x 256 route (up to four outlier chunks kept in
    the epilogue's registers) the recovered outlier weights in scratch are
    bit for bit the oracle's dtype(fl32(fl32(CB * SCB) / 127)), chunk padding
    zeroed, whatever the scratch held before; the forward matches the
    oracle."""
    B = _lib()
    import torch
    T, K, N = 2048, 512, 4096  # 8 x 16 tiles of 256 x 256: the persistent kernel
    case = random_case(T, K, N, dtype="bf16", seed=600 + n_out, n_out=n_out)
    X = to_dev(case.X, "bf16")
    CB, SCB = B.lli8_quant_weight_rowwise(to_dev(case.W, "bf16"))
    ws = B.Workspace(T, K, N, None, X.device, want_acc=True)
    ws.scratch.fill_(0xFF)  # whatever the scratch held before
    out, ws = B.lli8_int8_linear(X, CB, SCB, to_dev(case.bias, "bf16"), case.threshold, ws=ws, want_acc=True)
    torch.cuda.synchronize()
    n = int(ws.n_idx.item())
    assert n >= n_out and (n + 31) // 32 <= 4
    idx = ws.idx[:n].cpu().numpy()
    chunks = (n + 31) // 32
    xb = B.lli8_scratch_bytes(T, K)
    wo = ws.scratch[xb:xb + chunks * N * 64].cpu().numpy().view(np.uint16).reshape(chunks, N, 32)
    got = O.decode_bits(wo.transpose(1, 0, 2).reshape(N, chunks * 32), "bf16").astype(np.float64)
    ref = O.recover_weight(CB.cpu().numpy()[:, idx], SCB.cpu().numpy(), "bf16")
    np.testing.assert_array_equal(got[:, :n], ref)
    assert not got[:, n:].any()
    rCB, rSCB = O.quantize_weight_bits(case.W, "bf16")
    r = O.linear_forward(case.X, "bf16", rCB, rSCB, case.bias, case.threshold)
    assert np.array_equal(ws.acc.cpu().numpy(), r["acc"])
    assert_out(bits_of(out), r, "bf16")


@pytest.mark.parametrize("every_column", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_recovered_weights_bit_exact(dtype, every_column):
    """The recovered outlier weights the tile path writes to scratch (chunk-major
    [chunk][N][32], zero past n) equal the oracle's dtype(fl32(fl32(CB * SCB) /
    127)) bit for bit.  For bf16 some weight rows are scaled far down or up, so
    that products below 2^-100 and above 2^101 take the full division and the
    rest the multiply-and-correct form.  With every column an outlier (a tiny
    threshold) the pieces are runs of consecutive columns, whose row-scale
    range test is taken once per piece."""
    B = _lib()
    import torch
    T, K, N = 512, 512, 300  # past 256 tokens the recovery runs before the tiles
    case = random_case(T, K, N, dtype=dtype, seed=77, n_out=40)
    Wb = case.W
    if dtype == "bf16":
        vals = O.decode_bits(Wb, dtype).astype(np.float64)
        vals[0::7] *= 1e-34
        vals[3::11] *= 1e34
        Wb = O.round_to_dtype_bits(vals, dtype)
    CB, SCB = B.lli8_quant_weight_rowwise(to_dev(Wb, dtype))
    tau = 1e-30 if every_column else 6.0
    ws = B.Workspace(T, K, N, None, CB.device, scratch_bytes="full")
    _, ws = B.lli8_int8_linear(to_dev(case.X, dtype), CB, SCB, None, tau, ws=ws)
    torch.cuda.synchronize()
    n = int(ws.n_idx.item())
    assert n == K if every_column else n >= 40
    idx = ws.idx[:n].cpu().numpy()
    chunks = (n + 31) // 32
    xb = B.lli8_scratch_bytes(T, K)  # the recovered weights follow the minimum scratch
    wo = ws.scratch[xb:xb + chunks * N * 64].cpu().numpy().view(np.uint16).reshape(chunks, N, 32)
    got = O.decode_bits(wo.transpose(1, 0, 2).reshape(N, chunks * 32), dtype).astype(np.float64)
    ref = O.recover_weight(CB.cpu().numpy()[:, idx], SCB.cpu().numpy(), dtype)
    np.testing.assert_array_equal(got[:, :n], ref)
    assert not got[:, n:].any()


@pytest.mark.parametrize("seed", PC.SWEEP_SEEDS)
def test_random_sweep(seed):
    case, tau = PC.sweep_case(seed)
    _check_full(case, tau)


@pytest.mark.parametrize("T,K,N,dtype,tau", PC.SPLIT_SMALL)
def test_few_rows_one_launch_split(T, K, N, dtype, tau, monkeypatch):
    """Outputs of the one-launch split (also with the fused decode off, so T <= 16
    takes it inside lli8_int8_linear) and the gathered outlier columns it leaves
    in scratch ([chunk][T][32], zero past n) against the oracle."""
    B = _lib()
    import torch
    monkeypatch.setenv("LLI8_FUSED_DECODE", "0")
    case = PC.split_small_case(T, K, N, dtype)
    g, r = _check_full(case, tau)
    CA, SCA, bitmap, idx, n_idx = B.lli8_quant_rowwise_outliers(to_dev(case.X, dtype), tau)
    n = int(n_idx.item())
    assert n == r["idx"].size
    assert np.array_equal(idx[:n].cpu().numpy(), r["idx"])
    assert np.array_equal(CA.cpu().numpy(), r["CA"])
    assert np.array_equal(SCA.cpu().numpy(), r["SCA"])
    assert np.array_equal(bitmap.cpu().numpy().view(np.uint32), O.outlier_bitmap(r["idx"], K))
    if n > 0:
        X = to_dev(case.X, dtype)
        CB, SCB = B.lli8_quant_weight_rowwise(to_dev(case.W, dtype))
        _, ws = B.lli8_int8_linear(X, CB, SCB, None, tau)
        torch.cuda.synchronize()
        chunks = (n + 31) // 32
        xo = ws.scratch[:chunks * T * 64].cpu().numpy().view(np.uint16).reshape(chunks, T, 32)
        got = xo.transpose(1, 0, 2).reshape(T, chunks * 32)
        assert np.array_equal(got[:, :n], case.X[:, r["idx"]])
        assert not got[:, n:].any()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N,K", [(300, 512), (7, 13), (1, 1), (130, 4104), (64, 8)])
def test_recover_weight_entry_point(N, K, dtype):
    """lli8_recover_weight gives dtype(fl32(fl32(CB * SCB) / 127)) bit for bit,
    including row scales far outside the range where the division is taken
    by multiply-and-correct (bf16 rows scaled by 1e-34 and 1e34)."""
    B = _lib()
    import torch
    case = random_case(1, K, N, dtype=dtype, seed=N + K, n_out=0)
    Wb = case.W
    if dtype == "bf16":
        vals = O.decode_bits(Wb, dtype).astype(np.float64)
        vals[0::7] *= 1e-34
        vals[3::11] *= 1e34
        Wb = O.round_to_dtype_bits(vals, dtype)
    CB, SCB = B.lli8_quant_weight_rowwise(to_dev(Wb, dtype))
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    W = B.lli8_recover_weight(CB, SCB, dtype=tdt)
    torch.cuda.synchronize()
    ref = O.recover_weight(CB.cpu().numpy(), SCB.cpu().numpy(), dtype)
    np.testing.assert_array_equal(O.decode_bits(bits_of(W), dtype).astype(np.float64), ref)
