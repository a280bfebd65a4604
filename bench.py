"""Benchmark of the LLM.int8() mixed-precision linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one forward of the whole path over one synthetic batch: outlier
column scan, row-wise activation quantisation, int8 GEMM with the fused
dequantisation, 16-bit outlier product and bias (and, for the workloads whose
weights are quantised on every call, the weight quantisation before it).

The headline workload (default) is the 175B-class FFN up-projection, 4096
tokens x 12288 -> 49152 in fp16, the largest configuration, on which the
metric is quoted.  The same JSON line carries, under "workloads", the
16-token decode step (4096 -> 4096, HBM-bound) and the 4096-token 7B-class
MLP up-projection (4096 -> 11008), each measured the same way, so one run
covers the int8-MFMA targets of the 4096-token shapes and the HBM target of
the decode shape (--extra "" measures the headline only).

Timing protocol.  All inputs are resident in HBM before the timed region.
Untimed steps run for --settle-ms (200 ms) so the clocks have left idle, then
the W warm-up steps.
They exist in R identical copies at different addresses (R chosen so that one
pass over the copies moves >= 768 MiB, three times the 256 MB Infinity
Cache), and step i uses copy i mod R -- the way consecutive layers of a model
stream different weights -- so no step finds its operands in cache.  The K
steps run back to back between one pair of HIP events on the library's
stream; ms_per_step is the elapsed time divided by K.  (A per-step event pair
would add the ~6 us floor of an event-bracketed launch on this platform.)
The same number of steps then runs again in up to 10 blocks with one event
pair each; "dispersion" gives the 10th, 50th and 90th percentiles of the
blocks' per-step times.

"achievable" holds measured ceilings beside the nominal peaks: the rate of
a loop of int8 matrix-core instructions on register operands, once with
every operand byte 1 and once with pseudo-random operands (the board's clock
under matrix load depends on how much the operands switch; a GEMM's switch
like random ones), and the bytes per second of a plain 1 GiB device copy;
each roofline's "frac_of_achievable" divides its achieved rate by the
random-operand loop's rate (int8) or the copy's (HBM).

--vendor instead times the vendor's GEMMs on the workload's shape (the int8
product through torch._int_mm and an fp8 e4m3 product through
torch._scaled_mm, both hipBLASLt) beside this library's forward, each after
the same settling, and prints one JSON line of the three.

Prints one JSON line on stdout.  `value` is the effective throughput
2*T*N*K / t in TOPS.  `roofline` describes the kernel with the largest average
duration: for a one-kernel step that is the step time above; otherwise a
second pass of K steps records HIP events around each kernel on the library's
stream.  `cpu_baseline` times the CPU oracle on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LLM.int8 linear effective TOPS (2TNK/t) + % of MI355X int8-MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5033.2        # MI355X dense int8 MFMA: 256 CUs x 2.4 GHz x 8192 ops/clock, TOP/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense fp16/bf16 MFMA, TFLOP/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="ffn_175b")
    p.add_argument("--extra", default="decode,prefill_mlp_up",
                   help="comma-separated workloads measured after the headline one and reported "
                        "under 'workloads' in the same line")
    p.add_argument("--rotate-mib", type=float, default=768.0,
                   help="input copies are rotated until one pass moves this many MiB")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU-oracle time")
    p.add_argument("--settle-ms", type=float, default=200.0,
                   help="untimed steps run for this long before the warm-up, so the clocks have settled")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--vectorwise", default="",
                   help="SCHEME:AXIS (absmax|zeropoint : rows|cols): time lli8_quant_vectorwise on the "
                        "workload's activation matrix instead of the forward")
    p.add_argument("--api", choices=["binding", "module", "graph"], default="binding",
                   help="how a step is issued: the C-ABI binding, the Linear8bitLt module, "
                        "or a HIP graph of the binding's launches captured once per input copy")
    p.add_argument("--vendor", action="store_true",
                   help="time the vendor's int8 and fp8 GEMMs (hipBLASLt through torch) on the workload's "
                        "shape beside this library's forward, and exit")
    p.add_argument("--copy-mib", type=float, default=0.0,
                   help="instead of the benchmark, run 10 plain device-to-device copies of this "
                        "many MiB (the calibration for HBM byte counters) and exit")
    return p.parse_args()


def kernel_bytes(name, case, n_idx):
    """Algorithmic HBM bytes of one launch of a kernel: each operand once."""
    T, K, N = case.T, case.K, case.N
    npad = (n_idx + 31) // 32 * 32
    bias = 2 * N if case.bias is not None else 0
    if name == "int8_gemm":
        return T * K + 4 * T + N * K + 4 * N + bias + 2 * T * N + 2 * T * npad + 4 * n_idx
    if name == "quant_activations":
        return 2 * T * K + T * K + 4 * T + 2 * T * npad + 4 * n_idx
    if name == "outlier_scan":
        return 2 * T * K
    if name == "activation_split":  # scan and quantiser in one launch: X once, codes, list
        return 2 * T * K + T * K + 4 * T + 2 * T * npad + 4 * n_idx + 4 * ((K + 31) // 32)
    if name == "quant_weight":
        return 2 * N * K + N * K + 4 * N
    if name == "decode_fused":  # the whole forward in one launch
        return 2 * T * K + N * K + 4 * N + bias + 2 * T * N
    if name == "bitmap_clear":
        return 4 * ((K + 31) // 32)
    if name == "recover_outliers":  # CB at the outlier columns in, recovered rows out
        return N * n_idx + 4 * N + 4 * n_idx + 2 * N * npad
    if name == "recover_weight":  # CB and SCB in, the 16-bit weight out
        return N * K + 4 * N + 2 * N * K
    return 0


def step_bytes(case):
    """Algorithmic bytes of the whole step: inputs once, outputs once."""
    T, K, N = case.T, case.K, case.N
    bias = 2 * N if case.bias is not None else 0
    w = 2 * N * K if case.weights_each_call else N * K + 4 * N
    return 2 * T * K + w + bias + 2 * T * N


KERNEL_SOURCES = {
    "int8_gemm": "lli8_gemm.hip", "decode_fused": "lli8_decode.hip", "quant_activations": "lli8_quant.hip",
    "outlier_scan": "lli8_quant.hip", "quant_weight": "lli8_quant.hip", "bitmap_clear": "lli8_quant.hip",
    "activation_split": "lli8_quant.hip",
    "recover_outliers": "lli8_quant.hip", "recover_weight": "lli8_recover.hip",
}


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the stored counter runs (FETCH_SIZE + WRITE_SIZE,
    each scaled by what the counter reads for a plain copy of known size), or None
    when none were taken for this kernel and workload or its source has changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    src = KERNEL_SOURCES.get(kernel)
    if src is None or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("kernels", {}).get(f"{workload}/{kernel}")
    if rec is None:
        return None
    with open(os.path.join(ROOT, "bit_quantized_matmul_amd", "csrc", src), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None
    return int(rec["bytes_per_launch"])


def achievable_peaks():
    """Measured ceilings beside the nominal peaks: the int8 matrix cores in a
    loop on register operands (no memory traffic; run long enough for the
    board's clock under sustained matrix load to settle), once with every
    operand byte 1 and once with pseudo-random operands that switch like a
    GEMM's (the board's clock under matrix load depends on the values), and a
    plain 1 GiB device-to-device copy (bytes read plus bytes written per
    second)."""
    import torch
    import bit_quantized_matmul_amd as B
    iters = 4096  # about a millisecond per launch
    res = {}
    for pattern, key in ((0, "mfma_i8_loop_ones"), (1, "mfma_i8_loop_random")):
        sink, ops = B.lli8_mfma_i8_loop(iters, pattern=pattern)
        torch.cuda.synchronize()
        if pattern == 0:
            expect = ((4096 * iters + 2 ** 31) % 2 ** 32) - 2 ** 31
            if int(sink[0].item()) != expect or int(sink[-1].item()) != expect:
                raise RuntimeError("int8 matrix-core loop returned a wrong sum")
        for _ in range(100):
            B.lli8_mfma_i8_loop(iters, sink, pattern=pattern)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            B.lli8_mfma_i8_loop(iters, sink, pattern=pattern)
        e1.record()
        torch.cuda.synchronize()
        tops = ops * 20 / (e0.elapsed_time(e1) * 1e-3) / 1e12
        res[key + "_tops"] = round(tops, 1)
        res[key + "_frac"] = round(tops / INT8_PEAK_TOPS, 4)
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    res["hbm_copy_gbs"] = round(copy_gbs, 1)
    res["hbm_copy_frac"] = round(copy_gbs / HBM_PEAK_GBS, 4)
    return res


def frac_of_achievable(roof, ach):
    """A roofline's achieved rate against the measured ceiling of its unit (int8
    and HBM only): for int8, the matrix-core loop on pseudo-random operands."""
    if ach is None:
        return None
    if roof["bound"] == "mfma" and roof["peak"] == INT8_PEAK_TOPS:
        return round(roof["achieved"] / ach["mfma_i8_loop_random_tops"], 4)
    if roof["bound"] == "hbm":
        return round(roof["achieved"] / ach["hbm_copy_gbs"], 4)
    return None


def copy_calibration(mib):
    """Ten device-to-device copies of `mib` MiB (one copy kernel each)."""
    import torch
    n = int(mib * 2 ** 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 10}), flush=True)


def cpu_baseline(case, CB_np, SCB_np, seconds):
    """The CPU oracle on the host, on a bounded sample of the same workload."""
    import numpy as np
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    try:  # the BLAS pool the oracle's matrix products run on, sized to the cores it may use
        from threadpoolctl import threadpool_limits
        threadpool_limits(cores)
    except Exception:
        pass
    # rows of X per oracle call: whole workload when small, else a row sample
    flops_per_row = 2.0 * case.N * case.K
    rows = case.T if case.T * flops_per_row <= 2e10 else max(1, int(2e10 // flops_per_row))
    sel = None if rows == case.T else np.arange(rows)
    times = []
    t_end = time.perf_counter() + seconds
    while True:
        t0 = time.perf_counter()
        if case.weights_each_call:
            CB_np, SCB_np = O.quantize_weight_bits(case.W, case.dtype)
        O.linear_forward(case.X, case.dtype, CB_np, SCB_np, case.bias, case.threshold, rows=sel)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() > t_end or len(times) >= 50:
            break
    t = sum(times) / len(times)
    what = "full workload" if sel is None else f"first {rows} of {case.T} rows (outlier scan over all rows)"
    return {"value": round(2.0 * rows * case.N * case.K / t / 1e12, 6), "unit": "TOPS",
            "cores": int(cores), "cpu": cpu_model(), "kind": "oracle",
            "sample": f"{what}; {len(times)} calls, mean {t * 1e3:.1f} ms per call"
                      + ("; weight quantisation included" if case.weights_each_call else "")}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_vectorwise(args):
    """Vector-wise quantisation (absmax or zero-point, per row or per column)
    of the workload's activation matrix X [T, K]: one JSON line, GB/s of the
    algorithmic bytes (X read once, codes written once, one scale and zero
    point per vector) against the HBM peak, with the oracle on the host beside it."""
    import numpy as np
    import torch
    import bit_quantized_matmul_amd as B
    from workloads import config_case
    scheme, axis = args.vectorwise.split(":")
    case = config_case(args.workload)
    dev = torch.device("cuda:0")
    X0 = torch.from_numpy(np.ascontiguousarray(case.X).view(np.int16)).view(
        torch.float16 if case.dtype == "f16" else torch.bfloat16).to(dev)
    R, C = X0.shape
    nvec = R if axis == "rows" else C
    copy_bytes = X0.numel() * 2
    Rn = max(1, min(64, -(-int(args.rotate_mib * 2 ** 20) // copy_bytes)))
    xs = [X0] + [X0.clone() for _ in range(Rn - 1)]
    codes = torch.empty((R, C), dtype=torch.int8, device=dev)
    scale = torch.empty((nvec,), dtype=torch.float32, device=dev)
    zp = torch.empty((nvec,), dtype=torch.int32, device=dev)

    def step(i):
        B.lli8_quant_vectorwise(xs[i % Rn], scheme, axis, codes, scale, zp if scheme == "zeropoint" else None)

    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        for _ in range(8):
            step(n)
            n += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    alg = R * C * 2 + R * C + nvec * (8 if scheme == "zeropoint" else 4)
    gbs = alg / (ms * 1e-3) / 1e9
    line = {"metric": f"vector-wise {scheme} quantisation per {axis[:-1]}, GB/s of algorithmic bytes",
            "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": case.dtype, "data": "synthetic",
            "config": {"workload": f"{args.workload} activations", "R": R, "C": C, "scheme": scheme,
                       "axis": axis, "input_copies_rotated": Rn, "algorithmic_bytes": alg},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}}
    if not args.no_cpu_baseline:
        import oracle as O
        Xf = O.decode_bits(case.X, case.dtype)
        ax = 1 if axis == "rows" else 0
        times = []
        t_end = time.perf_counter() + args.cpu_seconds
        while time.perf_counter() < t_end and len(times) < 20:
            t = time.perf_counter()
            if scheme == "zeropoint":
                O.zeropoint_quantize(Xf, ax)
            else:
                O.absmax_quantize(Xf, ax)
            times.append(time.perf_counter() - t)
        tc = sum(times) / len(times)
        line["cpu_baseline"] = {"value": round(alg / tc / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                                "sample": f"full matrix (decoded to float32 beforehand); {len(times)} calls, "
                                          f"mean {tc * 1e3:.1f} ms per call"}
    print(json.dumps(line), flush=True)


def bench_vendor(args):
    """The vendor's GEMMs on the workload's shape beside this library's
    forward: torch._int_mm (int8 x int8 -> int32) on the workload's own codes
    CA and CB, and torch._scaled_mm in fp8 e4m3 (unit scales, bf16 out) on X
    and W cast to fp8.  Same protocol for each: operands rotated over copies
    of >= --rotate-mib, --settle-ms of untimed calls, --warmup calls, then
    --steps calls between one event pair."""
    import numpy as np
    import torch
    import bit_quantized_matmul_amd as B
    from workloads import config_case
    case = config_case(args.workload)
    dev = torch.device("cuda:0")
    dt = torch.float16 if case.dtype == "f16" else torch.bfloat16
    T, K, N = case.T, case.K, case.N
    X0 = torch.from_numpy(np.ascontiguousarray(case.X).view(np.int16)).view(dt).to(dev)
    W0 = torch.from_numpy(np.ascontiguousarray(case.W).view(np.int16)).view(dt).to(dev)
    bias = None if case.bias is None else torch.from_numpy(np.ascontiguousarray(case.bias).view(np.int16)).view(dt).to(dev)
    CB0, SCB0 = B.lli8_quant_weight_rowwise(W0)
    R = max(2, -(-int(args.rotate_mib * 2 ** 20) // (N * K)))
    CBs = [CB0] + [CB0.clone() for _ in range(R - 1)]
    SCBs = [SCB0] + [SCB0.clone() for _ in range(R - 1)]
    ws = B.Workspace(T, K, N, dt, dev)
    out = torch.empty((T, N), dtype=dt, device=dev)
    B.lli8_int8_linear(X0, CB0, SCB0, bias, case.threshold, out=out, ws=ws)
    CA = ws.CA.clone()

    def timed(fn):
        t0, n = time.perf_counter(), 0
        while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
            for _ in range(4):
                fn(n)
                n += 1
            torch.cuda.synchronize()
        for i in range(args.warmup):
            fn(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ops = 2.0 * T * N * K
    res = {}
    res["lli8_forward_ms"] = timed(lambda i: B.lli8_int8_linear(X0, CBs[i % R], SCBs[i % R], bias, case.threshold,
                                                                out=out, ws=ws))
    B.lli8_trace_enable(True)
    B.lli8_trace_read()
    g = []
    for i in range(args.steps):
        B.lli8_int8_linear(X0, CBs[i % R], SCBs[i % R], bias, case.threshold, out=out, ws=ws)
        g += [ms for k, ms in B.lli8_trace_read() if k == "int8_gemm"]
    torch.cuda.synchronize()
    B.lli8_trace_enable(False)
    res["lli8_int8_gemm_kernel_ms"] = sum(g) / len(g) if g else None
    try:
        res["vendor_int8_ms"] = timed(lambda i: torch._int_mm(CA, CBs[i % R].t()))
    except RuntimeError as ex:
        res["vendor_int8_ms"] = None
        res["vendor_int8_error"] = str(ex).splitlines()[0][:160]
    del CBs, SCBs
    torch.cuda.empty_cache()
    try:
        f8 = torch.float8_e4m3fn
        A8 = X0.to(f8)
        W8s = [W0.to(f8) for _ in range(R)]
        one = torch.ones((), device=dev)
        res["vendor_fp8_ms"] = timed(lambda i: torch._scaled_mm(A8, W8s[i % R].t(), scale_a=one, scale_b=one,
                                                                out_dtype=torch.bfloat16))
    except RuntimeError as ex:
        res["vendor_fp8_ms"] = None
        res["vendor_fp8_error"] = str(ex).splitlines()[0][:160]
    line = {"metric": "vendor GEMMs beside the LLM.int8 forward, ms per call and fraction of the 5033.2 "
                      "TOP/s int8 / fp8 dense peak",
            "config": {"workload": args.workload, "T": T, "K": K, "N": N, "act_dtype": case.dtype,
                       "copies_rotated": R, "steps": args.steps, "settle_ms": args.settle_ms}}
    for k, v in res.items():
        if k.endswith("_ms"):
            line[k] = None if v is None else round(v, 5)
            if v is not None:
                line[k[:-3] + "_frac"] = round(ops / (v * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)
        else:
            line[k] = v
    print(json.dumps(line), flush=True)


def measure(name, case, args):
    """One workload: inputs resident in rotated copies, the timed region, the
    per-kernel trace pass; returns the JSON line without the CPU baseline."""
    import numpy as np
    import torch
    import bit_quantized_matmul_amd as B

    dev = torch.device("cuda:0")

    def to_dev(bits):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.view(torch.float16 if case.dtype == "f16" else torch.bfloat16).to(dev)

    X0 = to_dev(case.X)
    W0 = to_dev(case.W)
    bias0 = to_dev(case.bias) if case.bias is not None else None
    T, K, N = case.T, case.K, case.N
    CB0 = torch.empty((N, K), dtype=torch.int8, device=dev)
    SCB0 = torch.empty((N,), dtype=torch.float32, device=dev)
    B.lli8_quant_weight_rowwise(W0, CB0, SCB0)   # placement (untimed unless quantised per call)
    copy_bytes = X0.numel() * 2 + (W0.numel() * 2 if case.weights_each_call else CB0.numel() + SCB0.numel() * 4) \
        + (bias0.numel() * 2 if bias0 is not None else 0)
    R = max(1, min(64, -(-int(args.rotate_mib * 2 ** 20) // copy_bytes)))
    copies = []
    for r in range(R):
        cp = dict(X=X0 if r == 0 else X0.clone(), bias=None if bias0 is None else (bias0 if r == 0 else bias0.clone()))
        if case.weights_each_call:
            cp["W"] = W0 if r == 0 else W0.clone()
            cp["CB"] = CB0 if r == 0 else torch.empty_like(CB0)
            cp["SCB"] = SCB0 if r == 0 else torch.empty_like(SCB0)
        else:
            cp["CB"] = CB0 if r == 0 else CB0.clone()
            cp["SCB"] = SCB0 if r == 0 else SCB0.clone()
        copies.append(cp)
    if not case.weights_each_call:
        del W0
    # with most columns outliers (the stress workloads) the caller gives the
    # scratch room for every recovered outlier weight; otherwise the default
    # one-buffer workspace (room for 8 outlier chunks)
    scratch = "full" if case.weights_each_call else None
    ws = B.Workspace(T, K, N, X0.dtype, dev, scratch_bytes=scratch)
    out = torch.empty((T, N), dtype=X0.dtype, device=dev)

    def bound_step(i):
        cp = copies[i % R]
        if case.weights_each_call:
            B.lli8_quant_weight_rowwise(cp["W"], cp["CB"], cp["SCB"])
        B.lli8_int8_linear(cp["X"], cp["CB"], cp["SCB"], cp["bias"], case.threshold, out=out, ws=ws)

    step = bound_step
    if args.api == "module":
        # one Linear8bitLt per input copy, sharing nothing but the device
        from bit_quantized_matmul_amd.nn import Linear8bitLt
        layers = []
        for cp in copies:
            layer = Linear8bitLt(K, N, bias=cp["bias"] is not None, has_fp16_weights=case.weights_each_call,
                                 threshold=case.threshold, device="meta", dtype=X0.dtype)
            if case.weights_each_call:
                layer.weight = torch.nn.Parameter(cp["W"], requires_grad=False)
            else:
                layer._set_int8(cp["CB"], cp["SCB"])
            layer.bias = None if cp["bias"] is None else torch.nn.Parameter(cp["bias"], requires_grad=False)
            layers.append(layer)

        def step(i):
            layers[i % R](copies[i % R]["X"])
    elif args.api == "graph":
        # the binding's launches of one step, captured once per input copy on a
        # side stream (default priority) and replayed; the workspace and the
        # output buffer are shared by every graph, as by the eager steps
        graphs = []
        cap = torch.cuda.Stream()
        for _ in range(2):  # eager runs on the capture stream first
            with torch.cuda.stream(cap):
                bound_step(0)
        torch.cuda.synchronize()
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                bound_step(r)
            graphs.append(g)
        torch.cuda.synchronize()

        def step(i):
            graphs[i % R].replay()

    # clocks: an idle GPU ramps up over tens of milliseconds; run untimed
    # steps until they have settled, then the W warm-up steps
    t_settle = time.perf_counter()
    n_settle = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(8):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    bound_step(0)  # the binding's workspace holds the outlier count whatever the api
    torch.cuda.synchronize()
    n_idx = int(ws.n_idx.item())

    # timed region: K steps back to back
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps

    # dispersion: the same number of steps again, in blocks with one event
    # pair each (an event pair around every step would add more than a
    # decode step costs), reported as percentiles of the per-block means
    nb = min(10, args.steps)
    per = max(1, args.steps // nb)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    evs[0].record()
    for b in range(nb):
        for j in range(per):
            step(args.warmup + args.steps + b * per + j)
        evs[b + 1].record()
    torch.cuda.synchronize()
    blocks = [evs[b].elapsed_time(evs[b + 1]) / per for b in range(nb)]
    p10, p50, p90 = (float(v) for v in np.percentile(blocks, [10, 50, 90]))
    dispersion = {"blocks": nb, "steps_per_block": per, "ms_per_step_p10": round(p10, 5),
                  "ms_per_step_median": round(p50, 5), "ms_per_step_p90": round(p90, 5)}

    # per-kernel durations: a second pass with events around each kernel
    # (through the binding: events cannot be recorded inside a replayed graph)
    B.lli8_trace_enable(True)
    B.lli8_trace_read()
    kern_ms = {}
    for i in range(args.steps):
        bound_step(i)
        for kname, kms in B.lli8_trace_read():
            kern_ms.setdefault(kname, []).append(kms)
    torch.cuda.synchronize()
    B.lli8_trace_enable(False)
    avg = {k: sum(v) / len(v) for k, v in kern_ms.items()}
    if len(avg) == 1:
        avg = {k: ms for k in avg}  # one kernel per step: the timed region is that kernel
    ops = 2.0 * T * N * K
    value = ops / (ms * 1e-3) / 1e12
    dom = max(avg, key=avg.get)
    dom_ms = avg[dom]
    if dom == "int8_gemm" and ops / kernel_bytes(dom, case, n_idx) > INT8_PEAK_TOPS / HBM_PEAK_GBS * 1e3:
        if n_idx * 2 > K:
            roof = {"bound": "mfma", "achieved": round(ops / (dom_ms * 1e-3) / 1e12, 3),
                    "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
        else:
            roof = {"bound": "mfma", "achieved": round(ops / (dom_ms * 1e-3) / 1e12, 3),
                    "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s"}
    else:
        gbs = kernel_bytes(dom, case, n_idx) / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(name, dom)
    roof["kernel"] = dom
    roof["kernel_ms"] = round(dom_ms, 5)

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": name, "api": args.api, "T": T, "K": K, "N": N, "act_dtype": case.dtype,
                   "threshold": case.threshold, "n_idx": n_idx, "bias": case.bias is not None,
                   "weights": "quantised every call" if case.weights_each_call else "pre-quantised",
                   "scratch": "full" if scratch else "default",
                   "input_copies_rotated": R, "rotation_mib": round(R * copy_bytes / 2 ** 20, 1),
                   "settle_steps": n_settle,
                   "step_algorithmic_bytes": step_bytes(case),
                   "step_hbm_frac": round(step_bytes(case) / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                   "kernels_ms": {k: round(v, 5) for k, v in avg.items()},
                   "timed_wall_s": round(t_wall, 3)},
        "roofline": roof,
        "dispersion": dispersion,
    }
    return line


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this path is not sharded across GPUs).", file=sys.stderr)
        sys.exit(2)
    if args.copy_mib > 0:
        copy_calibration(args.copy_mib)
        return
    if args.vectorwise:
        bench_vectorwise(args)
        return
    if args.vendor:
        bench_vendor(args)
        return

    import torch
    from workloads import CONFIGS, config_case

    names = [args.workload] + [w for w in args.extra.split(",") if w and w != args.workload]
    for w in names:
        if w not in CONFIGS:
            sys.exit(f"unknown workload {w!r}; choose from {sorted(CONFIGS)}")
    torch.cuda.set_device(torch.device("cuda:0"))
    ach = achievable_peaks()
    case = config_case(args.workload)
    line = measure(args.workload, case, args)
    line["roofline"]["frac_of_achievable"] = frac_of_achievable(line["roofline"], ach)
    print(f"[bench] {args.workload}: {line['ms_per_step']} ms per step, {line['value']} TOPS", file=sys.stderr,
          flush=True)
    extra = {}
    for w in names[1:]:
        torch.cuda.empty_cache()
        sub = measure(w, config_case(w), args)
        sub["roofline"]["frac_of_achievable"] = frac_of_achievable(sub["roofline"], ach)
        print(f"[bench] {w}: {sub['ms_per_step']} ms per step, {sub['value']} TOPS", file=sys.stderr, flush=True)
        c = sub["config"]
        extra[w] = {"value": sub["value"], "unit": sub["unit"], "ms_per_step": sub["ms_per_step"],
                    "T": c["T"], "K": c["K"], "N": c["N"], "n_idx": c["n_idx"],
                    "step_hbm_frac": c["step_hbm_frac"], "kernels_ms": c["kernels_ms"],
                    "roofline": sub["roofline"], "dispersion": sub["dispersion"]}
    if extra:
        line["workloads"] = extra
    line["achievable"] = ach
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        import oracle as O
        CB_np, SCB_np = O.quantize_weight_bits(case.W, case.dtype)  # the oracle's own codes
        line["cpu_baseline"] = cpu_baseline(case, CB_np, SCB_np, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
