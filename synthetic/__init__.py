"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

Holds random draws and input shaping only: no quantization, scale or GEMM
arithmetic of the method lives here.
"""
from .workloads import WORKLOADS, make, calibration_batches, bf16_round, smooth_factors  # noqa: F401
