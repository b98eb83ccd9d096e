"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This package holds no attention arithmetic.  It draws random numbers, rounds
them to the storage formats (bf16 with round-to-nearest-even, OCP e4m3fn with
a per-(token, KV-head) fp32 scale) and lays them out in the paged storage the
library reads.  Both the oracle and the GPU path consume the same bytes.
"""
from .synth import CONFIGS, Workload, make_workload, quantize_e4m3, to_bf16_bits

__all__ = ["CONFIGS", "Workload", "make_workload", "quantize_e4m3", "to_bf16_bits"]
