"""bench.py's contract on the CPU: the multi-GPU request is refused with a
message, and every kernel the library times by name has an algorithmic byte
count and a source file for its stored counter figures."""
import os
import re
import subprocess
import sys

import bench
from workloads import config_case

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _traced_names():
    src = open(os.path.join(ROOT, "bit_quantized_matmul_amd", "csrc", "lli8_api.cpp")).read()
    names = set(re.findall(r'TRACED\(\s*s\s*,\s*"([a-z0-9_]+)"', src))
    assert names, "no timed launches found"
    return names


def test_every_timed_kernel_is_accounted():
    case = config_case("tiny")
    for name in _traced_names():
        assert bench.kernel_bytes(name, case, 2) > 0, name
        src = bench.KERNEL_SOURCES.get(name)
        assert src is not None, name
        assert os.path.exists(os.path.join(ROOT, "bit_quantized_matmul_amd", "csrc", src)), src


def test_step_bytes_cover_inputs_and_output():
    for w in ("tiny", "decode"):
        case = config_case(w)
        T, K, N = case.T, case.K, case.N
        assert bench.step_bytes(case) >= 2 * T * K + N * K + 2 * T * N
