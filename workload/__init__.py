"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the benchmark."""
from .gen import WORKLOADS, Workload, layer_inputs, score_vector, SCORE_KINDS, round_bf16, span_slots  # noqa: F401
