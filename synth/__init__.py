"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

Holds only input generation (counter-based random bits and the workload recipes);
none of the MoE layer's arithmetic lives here."""
from . import rng, workloads  # noqa: F401
from .workloads import (ALL, QWEN35B_4BIT, QWEN35B_8BIT, QWEN35B_BATCHED, QWEN80B_4BIT, TINY,  # noqa: F401
                        LayerStack, MoeShape, Workload, algorithmic_decode_bytes, make_stack,
                        make_workload, make_x, with_zipf_bias, zipf_bias)
