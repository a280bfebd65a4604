"""The seeded cases whose outputs the GPU parity tests compare with the oracle,
in one place, so that the CPU check of the output comparison
(tests/test_out_check.py) runs on exactly the shapes and inputs the GPU tests
use.  Nothing here touches a GPU."""
import numpy as np

import oracle as O
from workloads import CONFIG_ORDER, config_case, make_case, random_case

INF = float("inf")

# -------------------------------------------------- test_gpu_parity.py ----

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


def shape_case(T, K, N, dtype):
    return random_case(T, K, N, dtype=dtype, seed=T * 7 + K * 3 + N, n_out=min(3, K))


THRESHOLDS = [0.0, -1.0, INF, 0.1, 2.5]


def threshold_case():
    return random_case(40, 200, 70, seed=11, n_out=4)


def issue_case():
    """x [2, 8] ~ N(0, 1) with threshold 0.1: every column flagged."""
    x = np.random.default_rng(1609).standard_normal((2, 8)).astype(np.float32)
    case = make_case("issue", 2, 8, 4, n_out=0, bias="normal", threshold=0.1, seed=1609)
    case.X = x.astype(np.float16).view(np.uint16)
    return case


def threshold_edge_case():
    """Column 5's largest magnitude is exactly 6.0 (not flagged), column 9's
    is 6.00390625 (flagged)."""
    case = random_case(12, 64, 16, seed=4, n_out=0)
    x = O.decode_bits(case.X, "f16").copy()
    x[:, 5] = 0.5
    x[3, 5] = 6.0
    x[:, 9] = 0.25
    x[7, 9] = -6.00390625
    case.X = x.astype(np.float16).view(np.uint16)
    return case


def zero_rows_case():
    case = random_case(20, 96, 33, seed=8, n_out=2)
    x = O.decode_bits(case.X, "f16").copy()
    x[4] = 0.0          # a zero row: SCA = 0, CA = 0
    x[:, 50] = 0.0      # a zero column
    case.X = x.astype(np.float16).view(np.uint16)
    w = O.decode_bits(case.W, "f16").copy()
    w[3] = 0.0          # a zero weight row: SCB = 0
    case.W = w.astype(np.float16).view(np.uint16)
    return case


# An outlier column beside a kept one, in rows whose kept values are tiny: the
# outlier's value times the row's scale runs far past 16 bits (60 / 1e-3 x 127),
# and the discarded code must not reach its neighbour.  One shape per route:
# fused decode, one-launch split, strip scan over every row, scan over row
# ranges, any-K quantiser.
WIDE_RATIO = [(8, 64, 40), (24, 64, 40), (100, 64, 40), (300, 64, 40), (300, 66, 40)]


def wide_ratio_case(T, K, N, dtype):
    case = random_case(T, K, N, dtype=dtype, seed=T * 3 + K + N, n_out=0)
    x = O.decode_bits(case.X, dtype).astype(np.float64)
    x[1::2] *= 1e-3                      # every other row: kept values around 1e-3
    for c in (2, 10, K - 2):             # even columns: outliers in every row
        x[:, c] = np.where(np.arange(T) % 3 == 0, -60.0, 60.0)
    case.X = _bits(x, dtype)
    return case


def _bits(x, dtype):
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    return O.round_to_dtype_bits(x, "bf16").astype(np.uint16)


SCATTERED = [(4096, 4096, 256), (300, 1024, 64), (100, 512, 64), (24, 256, 40)]


def scattered_flags_case(T, K, N, dtype):
    """Outlier values in single rows only, so that the bits of one bitmap
    word come from many workgroups of 16 rows spread over the chip: column j
    of the first 32 (and column 64 + 3 j of the next 96) exceeds the
    threshold in one row of workgroup 8 j + j % 8 (taken modulo the
    workgroups there are), and nowhere else."""
    case = random_case(T, K, N, dtype=dtype, seed=T + 5 * K + N, n_out=0)
    x = O.decode_bits(case.X, dtype).astype(np.float64)
    groups = (T + 15) // 16
    for j in range(32):
        g = (8 * j + j % 8) % groups
        for c in (j, 64 + 3 * j):
            if c < K:
                x[min(T - 1, 16 * g + j % 16), c] = 7.0 + j
    case.X = _bits(x, dtype)
    return case


SMALL_T = [(1, 64, 64), (3, 48, 5), (16, 4096, 130), (8, 8192, 40), (16, 8448, 33), (5, 1024, 4097),
           (16, 256, 16), (2, 512, 3000), (11, 2048, 1000), (16, 64, 8192)]


def small_t_case(T, K, N, dtype):
    return random_case(T, K, N, dtype=dtype, seed=T + K + N, n_out=min(4, K))


FUSED_THRESHOLDS = [0.0, 0.1, 2.0, INF]


def fused_threshold_case():
    return random_case(16, 1024, 512, seed=77, n_out=3)


def fused_many_blocks_case():
    return random_case(7, 512, 16 * 256 * 3 + 5, seed=78, n_out=2)


def fused_many_blocks_dense_case():
    # all 16 rows, three blocks for most workgroups; with tau 0.1 more outlier
    # columns than the 64 staged in LDS, so later blocks also take the rest
    # from memory
    return random_case(16, 1024, 16 * 256 * 2 + 3, seed=79, n_out=3)


def scratch_sizes_case():
    return random_case(300, 512, 260, seed=31, n_out=70)


def every_column_case():
    return random_case(290, 256, 300, seed=33, n_out=0)


PERSISTENT = [
    # whole 256 x 256 tiles, more tiles than compute units: workgroups walk
    # several tiles each, the next tile's first steps loaded during the
    # current tile's epilogue when the outlier columns fit in registers
    (2048, 256, 8448, 3, 6.0, "f16"),      # two K steps per tile, one chunk
    (2048, 512, 8448, 100, 6.0, "bf16"),   # four chunks: still from registers
    (2048, 512, 8448, 150, 6.0, "f16"),    # five chunks: staged through LDS, no cross-tile loads
    (2048, 256, 8448, 0, 0.01, "bf16"),    # every column an outlier: no int8 product at all
    (2048, 768, 8448, 2, 0.0, "f16"),      # threshold off: no outlier columns
]


def persistent_case(T, K, N, n_out, tau, dtype):
    return random_case(T, K, N, dtype=dtype, seed=T + K + N + n_out, n_out=n_out)


MANY_CHUNKS = [
    (600, 512, 520, 150, 6.0),    # 5 outlier chunks: 4 through the 2-slot pipeline, 1 through the ring
    (520, 768, 530, 0, 0.01),     # every column an outlier: 24 chunks, all through the pipeline
    (512, 1024, 512, 260, 6.0),   # 9 chunks: 8 + 1
    # the same on 256 x 256 tiles (at least 128 of them)
    (2000, 512, 4100, 150, 6.0), (2000, 768, 4100, 0, 0.01), (2000, 1024, 4100, 260, 6.0),
]


def many_chunks_case(T, K, N, n_out, tau, dtype):
    return random_case(T, K, N, dtype=dtype, seed=T + K + n_out, n_out=n_out)


SWEEP_SEEDS = range(48)


def sweep_case(seed):
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


# Few rows (T <= 32, K % 8 == 0, K <= 4096): the scan and the quantiser run
# as one launch; each register depth (8, 16, 24, 32 rows), K not a multiple
# of 16 or 32, either dtype, thresholds that flag nothing; and a few shapes
# just past it, on the two-launch split.
SPLIT_SMALL = [(1, 8, 5, "f16", 6.0), (7, 40, 33, "bf16", 6.0), (8, 4096, 64, "f16", 6.0),
               (12, 1000, 70, "f16", 2.5), (17, 4088, 100, "bf16", 6.0), (24, 4096, 300, "f16", 6.0),
               (25, 520, 48, "bf16", 0.0), (32, 4096, 256, "f16", 6.0), (32, 2056, 40, "bf16", INF),
               (31, 96, 17, "f16", 1.0), (33, 4096, 64, "f16", 6.0), (47, 1032, 20, "bf16", 6.0),
               (64, 4096, 128, "f16", 6.0), (64, 8, 9, "bf16", 0.0)]


def split_small_case(T, K, N, dtype):
    return random_case(T, K, N, dtype=dtype, seed=500 + T + K, n_out=min(6, K))


# -------------------------------------------------- test_gpu_module.py ----

MODULE_THRESHOLDS = [0.0, 6.0]


def module_case(dtype):
    return random_case(37, 136, 72, dtype=dtype, seed=91, n_out=3)


def module_requant_case():
    return random_case(9, 64, 24, seed=5, n_out=2)


def module_reuse_case():
    return random_case(24, 64, 16, seed=6, n_out=1)


# ------------------------------------------------ test_gpu_max_sizes.py ----

KMAX = 133144
MAX_K_SHAPES = [(8, KMAX - 8, 24), (3, KMAX, 5), (40, KMAX, 33)]


def max_k_case(T, K, N):
    return random_case(T, K, N, seed=K % 97 + T, n_out=3)


def large_k_tiles_case():
    return random_case(520, 133120, 600, seed=5, n_out=4)


LARGE_K_ROWS = np.array([0, 1, 255, 256, 511, 512, 519])
LARGE_K_COLS = np.array([0, 7, 255, 256, 300, 511, 512, 599])

# ------------------------------------------------- test_gpu_configs.py ----

FULL_CONFIGS = [c for c in CONFIG_ORDER if c != "tiny"]


def sample_indices(n, k_edge, k_rand, seed):
    """The first and last k_edge indices of range(n) and k_rand seeded random ones."""
    rng = np.random.default_rng(seed)
    edge = list(range(min(k_edge, n))) + list(range(max(0, n - k_edge), n))
    mid = rng.choice(n, size=min(k_rand, n), replace=False).tolist()
    return np.array(sorted(set(edge + mid)), dtype=np.int64)


def config_sample(case):
    """Output rows and columns the full-size config test compares."""
    return sample_indices(case.T, 8, 24, 2), sample_indices(case.N, 128, 768, 3)


# ----------------------------------------------------------- registry ----

def output_checks():
    """Every output comparison of the GPU tests as (label, build, rows, cols):
    build() returns (case, threshold the test passes), rows / cols the sampled
    outputs (None: all; "config": the full-size config test's sample)."""
    out = [("tiny", lambda: _own(config_case("tiny")), None, None)]
    for T, K, N in SHAPES:
        for dt in ("f16", "bf16"):
            out.append((f"shape{T}x{K}x{N}-{dt}", lambda T=T, K=K, N=N, dt=dt: _own(shape_case(T, K, N, dt)),
                        None, None))
    for tau in THRESHOLDS:
        out.append((f"threshold{tau}", lambda tau=tau: (threshold_case(), tau), None, None))
    out += [("issue", lambda: _own(issue_case()), None, None),
            ("edge", lambda: (threshold_edge_case(), 6.0), None, None),
            ("zero_rows", lambda: _own(zero_rows_case()), None, None)]
    for T, K, N in SMALL_T:
        for dt in ("f16", "bf16"):
            out.append((f"small{T}x{K}x{N}-{dt}", lambda T=T, K=K, N=N, dt=dt: _own(small_t_case(T, K, N, dt)),
                        None, None))
    for tau in FUSED_THRESHOLDS:
        out.append((f"fused_threshold{tau}", lambda tau=tau: (fused_threshold_case(), tau), None, None))
    out += [("fused_blocks", lambda: _own(fused_many_blocks_case()), None, None),
            ("scratch_sizes", lambda: _own(scratch_sizes_case(), bias=False), None, None),
            ("every_column", lambda: (every_column_case(), 0.01), None, None)]
    for p in PERSISTENT:
        out.append((f"persistent{p}", lambda p=p: (persistent_case(*p), p[4]), None, None))
    for m in MANY_CHUNKS:
        for dt in ("f16", "bf16"):
            out.append((f"chunks{m}-{dt}", lambda m=m, dt=dt: (many_chunks_case(*m, dt), m[4]), None, None))
    for s in SWEEP_SEEDS:
        out.append((f"sweep{s}", lambda s=s: sweep_case(s), None, None))
    for T, K, N, dt, tau in SPLIT_SMALL:
        out.append((f"split{T}x{K}x{N}-{dt}", lambda T=T, K=K, N=N, dt=dt, tau=tau:
                    (split_small_case(T, K, N, dt), tau), None, None))
    for dt in ("f16", "bf16"):
        for tau in MODULE_THRESHOLDS:
            out.append((f"module-{dt}-{tau}", lambda dt=dt, tau=tau: (module_case(dt), tau), None, None))
    out += [("module_requant", lambda: (module_requant_case(), 6.0), None, None),
            ("module_reuse", lambda: (module_reuse_case(), 6.0), None, None)]
    for T, K, N in WIDE_RATIO:
        for dt in ("f16", "bf16"):
            out.append((f"wide_ratio{T}x{K}x{N}-{dt}", lambda T=T, K=K, N=N, dt=dt: _own(wide_ratio_case(T, K, N, dt)),
                        None, None))
    for T, K, N in SCATTERED:
        for dt in ("f16", "bf16"):
            out.append((f"scattered{T}x{K}x{N}-{dt}", lambda T=T, K=K, N=N, dt=dt:
                        _own(scattered_flags_case(T, K, N, dt)), None, None))
    for T, K, N in MAX_K_SHAPES:
        out.append((f"maxk{T}x{K}x{N}", lambda T=T, K=K, N=N: _own(max_k_case(T, K, N)), None, None))
    out.append(("large_k_tiles", lambda: _own(large_k_tiles_case(), bias=False), LARGE_K_ROWS, LARGE_K_COLS))
    for name in FULL_CONFIGS:
        out.append((f"config-{name}", lambda name=name: _own(config_case(name)), "config", "config"))
    return out


def _own(case, bias=True):
    """(case, its own threshold); bias=False: the test passes no bias."""
    if not bias:
        case.bias = None
    return case, case.threshold
