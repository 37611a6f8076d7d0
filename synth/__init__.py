"""Seeded synthetic workload generator (inputs only; no verify-path arithmetic)."""
from .workload import (Workload, WORKLOADS, sweep_workloads, StepInputs, step_inputs,
                       raw_prefix, pooled_prefix, draft_tree, target_tokens,
                       f32_to_bf16_bits, bf16_bits_to_f32)

__all__ = ["Workload", "WORKLOADS", "sweep_workloads", "StepInputs", "step_inputs",
           "raw_prefix", "pooled_prefix", "draft_tree", "target_tokens",
           "f32_to_bf16_bits", "bf16_bits_to_f32"]
