"""Every kernel of the library runs without scratch memory.

Each HIP source is compiled for gfx950 with the library's own flags into a
plain device code object, and the kernel descriptors' metadata is read back
(`llvm-readelf --notes`): every kernel must have a zero private segment.  A
kernel whose registers spill to scratch sends them through memory on every
use; in the persistent GEMM and the fused decode that would cost far more
than any schedule change could win, and a different tile walk or loop shape
can tip the register allocator there without any other sign.  (Spills of
scalar registers into vector-register lanes stay in registers and are not
counted.)  Needs only the ROCm compiler, no GPU."""
import os
import re
import shutil
import subprocess

import pytest

from bit_quantized_matmul_amd import build as B

READELF = "/opt/rocm/llvm/bin/llvm-readelf"


def _kernels(co_path):
    """[(kernel name, private segment bytes, vgpr spill count)] from a code object."""
    out = subprocess.run([READELF, "--notes", co_path], capture_output=True, text=True, check=True).stdout
    res, name, priv, spill = [], None, None, 0
    for line in out.splitlines():
        m = re.match(r"\s+\.name:\s+(\S+)", line)
        if m and m.group(1).startswith("_Z"):
            name = m.group(1)
        m = re.match(r"\s+\.private_segment_fixed_size:\s+(\d+)", line)
        if m:
            priv = int(m.group(1))
        m = re.match(r"\s+\.vgpr_spill_count:\s+(\d+)", line)
        if m:
            spill = int(m.group(1))
        if re.match(r"\s+\.wavefront_size:", line) and name is not None and priv is not None:
            res.append((name, priv, spill))
            name, priv, spill = None, None, 0
    return res


@pytest.mark.skipif(not os.path.exists(READELF) or shutil.which("hipcc") is None and
                    not os.path.exists("/opt/rocm/bin/hipcc"), reason="ROCm compiler not installed")
def test_no_kernel_uses_scratch(tmp_path):
    srcs = [s for s in B.sources() if s.endswith(".hip")]
    procs = []
    for s in srcs:
        co = str(tmp_path / (os.path.basename(s) + ".co"))
        cmd = [B.hipcc()] + B.COMMON + ["--cuda-device-only", "--no-gpu-bundle-output", "-c", s, "-o", co]
        procs.append((s, co, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    kernels = []
    for s, co, p in procs:
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{s}: {err[-2000:]}"
        kernels += [(os.path.basename(s),) + k for k in _kernels(co)]
    names = {k[1] for k in kernels}
    assert any("linear_persist_kernel" in n for n in names) and any("decode_fused_kernel" in n for n in names)
    assert len(kernels) >= 20, kernels
    with_scratch = [(f, n, priv) for f, n, priv, _ in kernels if priv != 0]
    assert not with_scratch, with_scratch
