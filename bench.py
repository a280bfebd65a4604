"""Benchmark of the LLM.int8() mixed-precision linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one forward of the whole path over one synthetic batch: outlier
column scan, row-wise activation quantisation, int8 GEMM with the fused
dequantisation, 16-bit outlier product and bias (and, for the workloads whose
weights are quantised on every call, the weight quantisation before it).  The
inputs are resident in HBM before the timed region; before every step a
1 GiB buffer is overwritten so that the 256 MB Infinity Cache and the L2s hold
nothing of the step's operands (the flush is outside the step's events).

Prints one JSON line on stdout.  `value` is the effective throughput
2*T*N*K / t in TOPS; `roofline` describes the kernel with the largest average
duration, timed with HIP events on the library's stream inside the timed
region; `cpu_baseline` times the CPU oracle on the host.
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
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOP/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA, TFLOP/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode")
    p.add_argument("--no-flush", action="store_true", help="keep caches warm between steps")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU-oracle time")
    p.add_argument("--no-cpu-baseline", action="store_true")
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
    if name == "quant_weight":
        return 2 * N * K + N * K + 4 * N
    if name == "bitmap_clear":
        return 4 * ((K + 31) // 32)
    return 0


def step_bytes(case):
    """Algorithmic bytes of the whole step: inputs once, outputs once."""
    T, K, N = case.T, case.K, case.N
    bias = 2 * N if case.bias is not None else 0
    w = 2 * N * K if case.weights_each_call else N * K + 4 * N
    return 2 * T * K + w + bias + 2 * T * N


def cpu_baseline(case, CB_np, SCB_np, seconds):
    """The CPU oracle on the host, on a bounded sample of the same workload."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        cores = 1
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
            "cores": int(cores), "kind": "oracle",
            "sample": f"{what}; {len(times)} calls, mean {t * 1e3:.1f} ms per call"
                      + ("; weight quantisation included" if case.weights_each_call else "")}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this path is not sharded across GPUs).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import bit_quantized_matmul_amd as B
    from workloads import CONFIGS, config_case

    if args.workload not in CONFIGS:
        sys.exit(f"unknown workload {args.workload!r}; choose from {sorted(CONFIGS)}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = config_case(args.workload)

    def to_dev(bits):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.view(torch.float16 if case.dtype == "f16" else torch.bfloat16).to(dev)

    X = to_dev(case.X)
    W = to_dev(case.W)
    bias = to_dev(case.bias) if case.bias is not None else None
    T, K, N = case.T, case.K, case.N
    CB = torch.empty((N, K), dtype=torch.int8, device=dev)
    SCB = torch.empty((N,), dtype=torch.float32, device=dev)
    B.lli8_quant_weight_rowwise(W, CB, SCB)          # placement (untimed unless quantised per call)
    ws = B.Workspace(T, K, N, X.dtype, dev)
    out = torch.empty((T, N), dtype=X.dtype, device=dev)
    flush = None if args.no_flush else torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def step():
        if case.weights_each_call:
            B.lli8_quant_weight_rowwise(W, CB, SCB)
        B.lli8_int8_linear(X, CB, SCB, bias, case.threshold, out=out, ws=ws)

    for i in range(args.warmup):
        if flush is not None:
            flush.fill_(i & 0xFF)
        step()
    torch.cuda.synchronize()
    n_idx = int(ws.n_idx.item())

    B.lli8_trace_enable(True)
    B.lli8_trace_read()  # start a fresh record
    kern_ms = {}
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_((i + 7) & 0xFF)
        ev[i][0].record()
        step()
        ev[i][1].record()
        for name, ms in B.lli8_trace_read():
            kern_ms.setdefault(name, []).append(ms)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    B.lli8_trace_enable(False)
    step_ms = [a.elapsed_time(b) for a, b in ev]
    ms = sum(step_ms) / len(step_ms)

    ops = 2.0 * T * N * K
    value = ops / (ms * 1e-3) / 1e12
    avg = {k: sum(v) / len(v) for k, v in kern_ms.items()}
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
    roof["traffic"] = None
    roof["kernel"] = dom
    roof["kernel_ms"] = round(dom_ms, 5)

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": args.workload, "T": T, "K": K, "N": N, "act_dtype": case.dtype,
                   "threshold": case.threshold, "n_idx": n_idx, "bias": case.bias is not None,
                   "weights": "quantised every call" if case.weights_each_call else "pre-quantised",
                   "cache_flush_between_steps": flush is not None,
                   "step_algorithmic_bytes": step_bytes(case),
                   "step_hbm_frac": round(step_bytes(case) / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                   "kernels_ms": {k: round(v, 5) for k, v in avg.items()},
                   "timed_wall_s": round(t_wall, 3)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        import oracle as O
        CB_np, SCB_np = O.quantize_weight_bits(case.W, case.dtype)  # the oracle's own codes
        line["cpu_baseline"] = cpu_baseline(case, CB_np, SCB_np, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
