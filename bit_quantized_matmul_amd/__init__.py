"""LLM.int8() mixed-precision decomposition linear on AMD MI355X (gfx950).

A thin ctypes binding over the C-ABI library ``liblli8.so`` (declared in
``include/lli8.h``).  The binding only marshals arguments: it takes device
pointers of torch tensors and torch's current HIP stream, and every step of
the computation runs in the library's HIP kernels.  PyTorch supplies device
memory and streams.

The library must have been built (``python -m bit_quantized_matmul_amd.build``);
importing the compute entry points without it raises an error -- there is no
CPU fallback.
"""
from __future__ import annotations

from ._lib import (LLI8_BF16, LLI8_F16, Lli8Error, Workspace, lib,  # noqa: F401
                   library_path, lli8_int8_linear, lli8_quant_rowwise_outliers, lli8_quant_vectorwise,
                   lli8_quant_weight_rowwise, lli8_recover_weight, lli8_scratch_bytes, lli8_scratch_bytes_full,
                   lli8_status_string, lli8_trace_enable, lli8_trace_read, lli8_version, lli8_workspace_bytes,
                   lli8_int8_linear_noalloc, lli8_noalloc_scratch_bytes, lli8_mfma_i8_loop,
                   lli8_mfma_i8_loop_sink_ints)

__all__ = [
    "LLI8_F16", "LLI8_BF16", "Lli8Error", "Workspace", "lib", "library_path",
    "lli8_int8_linear", "lli8_quant_rowwise_outliers", "lli8_quant_vectorwise", "lli8_quant_weight_rowwise",
    "lli8_recover_weight", "lli8_workspace_bytes", "lli8_int8_linear_noalloc", "lli8_noalloc_scratch_bytes",
    "lli8_scratch_bytes", "lli8_scratch_bytes_full", "lli8_status_string", "lli8_trace_enable", "lli8_trace_read",
    "lli8_version", "lli8_mfma_i8_loop", "lli8_mfma_i8_loop_sink_ints",
]
