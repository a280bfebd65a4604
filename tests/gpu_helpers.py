"""Helpers for the GPU parity tests: move seeded numpy inputs to the device and
compare the HIP path's results with the oracle's."""
import numpy as np

import oracle as O


def to_dev(bits: np.ndarray, dtype: str, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.to(device)


def bits_of(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def normwise_rel(gpu_bits: np.ndarray, ref64: np.ndarray, dtype: str) -> float:
    """max |g - o| / max(max |o|, 1e-6), the output tolerance measure."""
    g = O.decode_bits(gpu_bits, dtype).astype(np.float64)
    den = max(float(np.abs(ref64).max()) if ref64.size else 0.0, 1e-6)
    return float(np.abs(g - ref64).max() / den) if ref64.size else 0.0


OUT_TOL = 1e-2
