"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path."""
from .gen import (BF16, CONFIG_ORDER, CONFIGS, F16, Case, config_case,  # noqa: F401
                  make_case, matrix_bits, random_case)
