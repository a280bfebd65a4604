"""CPU oracle (test infrastructure only).

Imported by the test suite, by the smoke check and by the benchmark's CPU
baseline leg, never by the product path.  It shares no code with the HIP
library.  Every function is pinned by CPU tests; the 16-bit output is
compared with the GPU path's within a tolerance (several roundings of it are
correct), everything else bit for bit.
"""
from .lli8_oracle import *  # noqa: F401,F403
from .lli8_oracle import (absmax_quantize_rows, decode_bits, dequantize,  # noqa: F401
                          int8_accumulate, linear_forward, outlier_bitmap, outlier_columns,
                          quantize_activations, quantize_weight,
                          quantize_weight_bits, recover_weight,
                          round_half_away, round_to_dtype_bits)
