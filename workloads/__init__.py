"""Seeded synthetic decode-attention workloads.

This package only draws inputs: request lengths, page tables and the Q/K/V
(and FP8 scale) tensors.  It contains none of the attention or scheduling
arithmetic, so both the CPU oracle and the HIP path can consume its output
without sharing any of the method's code.
"""

from .configs import CONFIGS, TABLE3, WorkloadConfig, get_config
from .gen import (
    draw_lengths,
    draw_page_table,
    make_layer,
    make_workload,
    poison_tail_slots,
    quantize_query_e4m3,
    rope_cos_sin_table,
    make_prologue_inputs,
    Workload,
    Layer,
)

__all__ = [
    "CONFIGS",
    "TABLE3",
    "WorkloadConfig",
    "get_config",
    "draw_lengths",
    "draw_page_table",
    "make_layer",
    "make_workload",
    "poison_tail_slots",
    "quantize_query_e4m3",
    "rope_cos_sin_table",
    "make_prologue_inputs",
    "Workload",
    "Layer",
]
