"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the benchmark."""
from .inputs import WORKLOADS, Workload, generate, scaled, to_bf16_bits, bf16_bits_to_f32

__all__ = ["WORKLOADS", "Workload", "generate", "scaled", "to_bf16_bits", "bf16_bits_to_f32"]
