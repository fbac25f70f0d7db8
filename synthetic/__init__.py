"""Seeded synthetic inputs for the KV-selection workloads.

This module is the only code shared by the CPU oracle and the GPU path. It
holds no arithmetic of the selection methods themselves: it draws Gaussian
queries, keys and values, plants the boosted key spans that make attention
votes heavy-tailed, and rounds to bfloat16 bit patterns.

Every array is reproducible from (workload seed, batch index, head index), so a
single head of a very long workload can be regenerated on its own.
"""
from .bf16 import f32_to_bf16_bits, bf16_bits_to_f32
from .workloads import (
    SnapKVWorkload,
    H2OWorkload,
    SNAPKV_WORKLOADS,
    H2O_WORKLOADS,
    snapkv_head,
    snapkv_batch,
    h2o_prompt_head,
    h2o_prompt_batch,
    h2o_step_inputs,
)

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "SnapKVWorkload",
    "H2OWorkload",
    "SNAPKV_WORKLOADS",
    "H2O_WORKLOADS",
    "snapkv_head",
    "snapkv_batch",
    "h2o_prompt_head",
    "h2o_prompt_batch",
    "h2o_step_inputs",
]
