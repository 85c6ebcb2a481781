"""The five decode workloads used for parity tests and the benchmark.

Shapes follow the GQA shape the vLLM x HPC-Ops page gives for Hy3 in its
"note on the Hy3 model family" (64 query heads, 8 KV heads, head_dim 128)
and the 64-token page the SGLang x HPC-Ops page uses in its launch example
("Attention and MoE", ``--page-size 64``).  Length mixes stand in for the
A x B mixes of the vLLM x HPC-Ops page, Table 3 (mixed-length decode):
uniform, log-uniform and one-very-long-request skew.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    seed: int                      # numpy seed for lengths and page table
    batch: int
    num_q_heads: int
    num_kv_heads: int
    kv_dtype: str                  # "bf16" or "fp8_e4m3"
    lengths_kind: str              # "fixed" | "uniform" | "loguniform" | "skewed"
    fixed_lengths: Optional[Tuple[int, ...]] = None
    length_lo: int = 0
    length_hi: int = 0
    long_length: int = 0           # "skewed": length of request 0
    layers: int = 1                # distinct KV tensors sharing one task map
    head_dim: int = 128
    page_size: int = 64
    fp8_scale_lo: float = 0.01
    fp8_scale_hi: float = 0.1

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def sm_scale(self) -> float:
        return 1.0 / (self.head_dim ** 0.5)

    @property
    def kv_bytes_per_token_head(self) -> int:
        """Bytes of K+V the method must read per (token, KV head)."""
        if self.kv_dtype == "bf16":
            return 2 * self.head_dim * 2
        # one byte per e4m3 code for K and V, plus one fp32 scale each
        return 2 * self.head_dim * 1 + 2 * 4


CONFIGS = {
    "tiny": WorkloadConfig(
        name="tiny", seed=0, batch=4, num_q_heads=8, num_kv_heads=1,
        kv_dtype="bf16", lengths_kind="fixed", fixed_lengths=(17, 64, 200, 1000)),
    "uniform": WorkloadConfig(
        name="uniform", seed=1, batch=32, num_q_heads=64, num_kv_heads=8,
        kv_dtype="bf16", lengths_kind="uniform", length_lo=4096, length_hi=4096),
    "mixed": WorkloadConfig(
        name="mixed", seed=2, batch=64, num_q_heads=64, num_kv_heads=8,
        kv_dtype="bf16", lengths_kind="loguniform", length_lo=256,
        length_hi=65536, layers=8),
    "skewed": WorkloadConfig(
        name="skewed", seed=3, batch=16, num_q_heads=8, num_kv_heads=1,
        kv_dtype="bf16", lengths_kind="skewed", long_length=131072,
        length_lo=512, length_hi=2048),
    "fp8": WorkloadConfig(
        name="fp8", seed=4, batch=128, num_q_heads=64, num_kv_heads=8,
        kv_dtype="fp8_e4m3", lengths_kind="loguniform", length_lo=1024,
        length_hi=262144),
}


def get_config(name: str) -> WorkloadConfig:
    try:
        return CONFIGS[name]
    except KeyError as e:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from e
