"""Parity of the HIP path (through the C-ABI) with the CPU oracle.

Bit-exact: CB, SCB, CA, SCA, the outlier bitmap, idx, n_idx and the int32
accumulators.  Output: normwise max-abs-rel <= 1e-2 (fp32 accumulation order
and the single final rounding differ from the oracle's float64 sum).
"""
import numpy as np
import pytest

import oracle as O
from tests.gpu_helpers import OUT_TOL, bits_of, normwise_rel, to_dev
from workloads import config_case, make_case, random_case

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
    err = normwise_rel(g["out"], r["out64"], case.dtype)
    assert err <= OUT_TOL, f"out normwise rel err {err}"
    return g, r


def test_tiny_config():
    case = config_case("tiny")
    g, r = _check_full(case)
    assert g["idx"].tolist() == [3, 17]


SHAPES = [
    (1, 64, 64), (3, 24, 5), (8, 8, 4), (16, 4096, 130), (17, 520, 300), (33, 136, 65),
    (100, 264, 257), (130, 1000, 129), (257, 512, 513), (300, 136, 40), (64, 8, 1), (5, 100, 7),
    (2, 17, 3), (40, 37, 11), (600, 640, 520),
    # T, N >= 512 with fewer than 128 tiles of 256 x 256: small tiles
    (600, 768, 520), (513, 256, 777), (512, 512, 512), (530, 520, 515), (515, 100, 520),
    # large tiles (at least 128 of them): 128-byte steps in pairs (K % 256 ==
    # 0; two steps only at K = 256), 64-byte steps (K % 64 == 0), register
    # staging (8-byte, 4-byte loads), each with ragged T and N tails
    (2000, 768, 4100), (2050, 256, 4097), (2048, 576, 4096), (2000, 520, 4100), (2001, 100, 4100),
    # 16 < T <= 64 with K % 16 == 0 and N <= 4096 (K <= 4096 past 32 tokens): the
    # weight-streaming kernel, 2 or 4 token blocks; otherwise the tiles
    (17, 512, 300), (32, 4096, 520), (33, 256, 65), (48, 2048, 1000), (64, 1024, 130),
    (65, 512, 100), (128, 4096, 260), (100, 1040, 33),
    # T < 512 with at least 256 tiles of 128 x 128: the 128 x 128 tile path (others take 64 x 64)
    (300, 256, 11000),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,K,N", SHAPES)
def test_random_shapes(T, K, N, dtype):
    case = random_case(T, K, N, dtype=dtype, seed=T * 7 + K * 3 + N, n_out=min(3, K))
    _check_full(case)


@pytest.mark.parametrize("tau", [0.0, -1.0, float("inf"), 0.1, 2.5])
def test_thresholds(tau):
    case = random_case(40, 200, 70, seed=11, n_out=4)
    g, r = _check_full(case, tau)
    if tau <= 0 or tau == float("inf"):
        assert g["n"] == 0
    if tau == 0.1:
        assert g["n"] == case.K  # every column flagged, as in the issue's repro


def test_issue_repro_shape_all_columns():
    """x[2, 8] with threshold 0.1 flags all 8 columns (state.idx = [0..7])."""
    rng = np.random.default_rng(1609)
    x = rng.standard_normal((2, 8)).astype(np.float32)
    case = make_case("issue", 2, 8, 4, n_out=0, bias="normal", threshold=0.1, seed=1609)
    case.X = x.astype(np.float16).view(np.uint16)
    g, r = _check_full(case)
    assert g["idx"].tolist() == list(range(8))
    assert not g["CA"].any() and not g["SCA"].any() and not g["acc"].any()


def test_threshold_edge_exact_value():
    """A column whose largest magnitude is exactly the threshold is not flagged."""
    case = random_case(12, 64, 16, seed=4, n_out=0)
    x = O.decode_bits(case.X, "f16").copy()
    x[:, 5] = 0.5
    x[3, 5] = 6.0
    x[:, 9] = 0.25
    x[7, 9] = -6.00390625
    case.X = x.astype(np.float16).view(np.uint16)
    g, r = _check_full(case, 6.0)
    assert g["idx"].tolist() == [9]


def test_zero_rows_and_columns():
    case = random_case(20, 96, 33, seed=8, n_out=2)
    x = O.decode_bits(case.X, "f16").copy()
    x[4] = 0.0          # a zero row: SCA = 0, CA = 0
    x[:, 50] = 0.0      # a zero column
    case.X = x.astype(np.float16).view(np.uint16)
    w = O.decode_bits(case.W, "f16").copy()
    w[3] = 0.0          # a zero weight row: SCB = 0
    case.W = w.astype(np.float16).view(np.uint16)
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


SMALL_T = [(1, 64, 64), (3, 48, 5), (16, 4096, 130), (8, 8192, 40), (16, 8448, 33), (5, 1024, 4097),
           (16, 256, 16), (2, 512, 3000), (11, 2048, 1000), (16, 64, 8192)]


@pytest.mark.parametrize("fused", ["1", "0"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,K,N", SMALL_T)
def test_small_T_both_decode_paths(T, K, N, dtype, fused, monkeypatch):
    """T <= 16 runs the single-launch path by default; LLI8_FUSED_DECODE=0 selects the
    multi-kernel path.  Both must match the oracle."""
    monkeypatch.setenv("LLI8_FUSED_DECODE", fused)
    case = random_case(T, K, N, dtype=dtype, seed=T + K + N, n_out=min(4, K))
    _check_full(case)


@pytest.mark.parametrize("tau", [0.0, 0.1, 2.0, float("inf")])
def test_fused_decode_thresholds(tau):
    """Degenerate and dense thresholds on the single-launch path (T <= 16)."""
    case = random_case(16, 1024, 512, seed=77, n_out=3)
    _check_full(case, tau)


def test_fused_decode_many_blocks_per_workgroup():
    """N well beyond one 16-feature block per CU: each workgroup walks several blocks."""
    case = random_case(7, 512, 16 * 256 * 3 + 5, seed=78, n_out=2)
    _check_full(case)


@pytest.mark.parametrize("room_chunks", ["full", 0, 1])
def test_recovered_outlier_weights_scratch_sizes(room_chunks):
    """The recovered outlier weights come from scratch for as many 32-column
    chunks as fit and are gathered in the tiles for the rest; every split
    gives the oracle's results (here 70 outlier columns: three chunks)."""
    B = _lib()
    import torch
    case = random_case(300, 512, 260, seed=31, n_out=70)
    X = to_dev(case.X, case.dtype)
    W = to_dev(case.W, case.dtype)
    CB, SCB = B.lli8_quant_weight_rowwise(W)
    if room_chunks == "full":
        nbytes = None
    else:
        nbytes = B.lli8_scratch_bytes(case.T, case.K) + room_chunks * case.N * 64
    ws = B.Workspace(case.T, case.K, case.N, X.dtype, X.device, want_acc=True, scratch_bytes=nbytes)
    out, ws = B.lli8_int8_linear(X, CB, SCB, None, case.threshold, ws=ws, want_acc=True)
    torch.cuda.synchronize()
    rCB, rSCB = O.quantize_weight_bits(case.W, case.dtype)
    r = O.linear_forward(case.X, case.dtype, rCB, rSCB, None, case.threshold)
    assert int(ws.n_idx.item()) == r["idx"].size == 70
    assert np.array_equal(ws.acc.cpu().numpy(), r["acc"])
    assert normwise_rel(bits_of(out), r["out64"], case.dtype) <= OUT_TOL


def test_every_column_an_outlier_skips_nothing_it_needs():
    """All K columns flagged (tiny threshold): the int8 product is skipped and
    the output is the 16-bit product alone."""
    case = random_case(290, 256, 300, seed=33, n_out=0)
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


@pytest.mark.parametrize("T,K,N,n_out,tau,dtype", [
    # whole 256 x 256 tiles, more tiles than compute units: workgroups walk
    # several tiles each, the next tile's first steps loaded during the
    # current tile's epilogue when the outlier columns fit in registers
    (2048, 256, 8448, 3, 6.0, "f16"),      # two K steps per tile, one chunk
    (2048, 512, 8448, 100, 6.0, "bf16"),   # four chunks: still from registers
    (2048, 512, 8448, 150, 6.0, "f16"),    # five chunks: staged through LDS, no cross-tile loads
    (2048, 256, 8448, 0, 0.01, "bf16"),    # every column an outlier: no int8 product at all
    (2048, 768, 8448, 2, 0.0, "f16"),      # threshold off: no outlier columns
])
def test_persistent_tiles(T, K, N, n_out, tau, dtype):
    case = random_case(T, K, N, dtype=dtype, seed=T + K + N + n_out, n_out=n_out)
    g, r = _check_full(case, tau)
    if tau == 0.0:
        assert g["n"] == 0
    else:
        assert g["n"] >= min(n_out, K) and (tau > 0.1 or g["n"] == K)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,K,N,n_out,tau", [
    (600, 512, 520, 150, 6.0),    # 5 outlier chunks: 4 through the 2-slot pipeline, 1 through the ring
    (520, 768, 530, 0, 0.01),     # every column an outlier: 24 chunks, all through the pipeline
    (512, 1024, 512, 260, 6.0),   # 9 chunks: 8 + 1
    # the same on 256 x 256 tiles (at least 128 of them)
    (2000, 512, 4100, 150, 6.0), (2000, 768, 4100, 0, 0.01), (2000, 1024, 4100, 260, 6.0),
])
def test_many_outlier_chunks_large_tiles(T, K, N, n_out, tau, dtype):
    case = random_case(T, K, N, dtype=dtype, seed=T + K + n_out, n_out=n_out)
    g, r = _check_full(case, tau)
    assert g["n"] >= min(n_out, K) and (tau > 0.1 or g["n"] == K)


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
    _, ws = B.lli8_int8_linear(to_dev(case.X, dtype), CB, SCB, None, tau)
    torch.cuda.synchronize()
    n = int(ws.n_idx.item())
    assert n == K if every_column else n >= 40
    idx = ws.idx[:n].cpu().numpy()
    chunks = (n + 31) // 32
    xb = T * ((K + 31) // 32 * 32) * 2
    wo = ws.scratch[xb:xb + chunks * N * 64].cpu().numpy().view(np.uint16).reshape(chunks, N, 32)
    got = O.decode_bits(wo.transpose(1, 0, 2).reshape(N, chunks * 32), dtype).astype(np.float64)
    ref = O.recover_weight(CB.cpu().numpy()[:, idx], SCB.cpu().numpy(), dtype)
    np.testing.assert_array_equal(got[:, :n], ref)
    assert not got[:, n:].any()


def _sweep_case(seed):
    """A seeded random shape across the launch routes: whole 256 x 256 tiles
    (persistent kernel), few rows (strip scan, weight streaming, small tiles),
    ragged large shapes and small ones; either dtype, a few outlier counts and
    thresholds."""
    rng = np.random.default_rng(1000 + seed)
    kind = seed % 4
    if kind == 0:
        T, N, K = 256 * int(rng.integers(2, 9)), 256 * int(rng.integers(2, 40)), 256 * int(rng.integers(1, 9))
    elif kind == 1:
        T, N, K = int(rng.integers(1, 300)), int(rng.integers(1, 3000)), 8 * int(rng.integers(1, 600))
    elif kind == 2:
        T, N, K = int(rng.integers(500, 1500)), int(rng.integers(500, 3000)), int(rng.integers(1, 1200))
    else:
        T, N, K = int(rng.integers(1, 200)), int(rng.integers(1, 500)), int(rng.integers(1, 700))
    if T * N * K > 3e8:  # keep the oracle quick
        if kind == 0:
            N = max(256, int(3e8 // (T * K)) // 256 * 256)
        else:
            K = max(1, int(3e8 // (T * N)))
    dtype = "f16" if rng.integers(0, 2) == 0 else "bf16"
    n_out = int(rng.choice([0, 1, 3, 17, 40, 150]))
    tau = float(rng.choice([6.0, 6.0, 6.0, 2.5, 0.0]))
    return random_case(T, K, N, dtype=dtype, seed=int(rng.integers(0, 1 << 30)), n_out=min(n_out, K)), tau


@pytest.mark.parametrize("seed", range(48))
def test_random_sweep(seed):
    case, tau = _sweep_case(seed)
    _check_full(case, tau)


# Few rows (T <= 32, K % 8 == 0, K <= 4096): the scan and the quantiser run
# as one launch; each register depth (8, 16, 24, 32 rows), K not a multiple
# of 16 or 32, either dtype, thresholds that flag nothing; and a few shapes
# just past it, on the two-launch split.
SPLIT_SMALL = [(1, 8, 5, "f16", 6.0), (7, 40, 33, "bf16", 6.0), (8, 4096, 64, "f16", 6.0),
               (12, 1000, 70, "f16", 2.5), (17, 4088, 100, "bf16", 6.0), (24, 4096, 300, "f16", 6.0),
               (25, 520, 48, "bf16", 0.0), (32, 4096, 256, "f16", 6.0), (32, 2056, 40, "bf16", float("inf")),
               (31, 96, 17, "f16", 1.0), (33, 4096, 64, "f16", 6.0), (47, 1032, 20, "bf16", 6.0),
               (64, 4096, 128, "f16", 6.0), (64, 8, 9, "bf16", 0.0)]


@pytest.mark.parametrize("T,K,N,dtype,tau", SPLIT_SMALL)
def test_few_rows_one_launch_split(T, K, N, dtype, tau, monkeypatch):
    """Outputs of the one-launch split (also with the fused decode off, so T <= 16
    takes it inside lli8_int8_linear) and the gathered outlier columns it leaves
    in scratch ([chunk][T][32], zero past n) against the oracle."""
    B = _lib()
    import torch
    monkeypatch.setenv("LLI8_FUSED_DECODE", "0")
    case = random_case(T, K, N, dtype=dtype, seed=500 + T + K, n_out=min(6, K))
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
