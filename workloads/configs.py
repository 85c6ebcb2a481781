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


def _mix(*parts):
    """Lengths of an A x B mix: `count` requests at KV length `length` per part."""
    return tuple(length for count, length in parts for _ in range(count))


K = 1024

# The six FP8-KV length mixes of the vLLM x HPC-Ops page, Table 3 (decode
# latency across KV-length distributions; "A x B" = A requests of KV length
# B, K = 1024 tokens), at one GPU's tensor-parallel share of the Hy3 shape:
# 8 query heads, 1 KV head.  The page does not state the head count; one KV
# head is the share that makes its H20 timings possible (at 8 KV heads the
# 1 x 128K + 31 x 4K mix would need more than twice the H20's bandwidth).
TABLE3 = {
    name: WorkloadConfig(name=f"t3-{name}", seed=10 + i, batch=len(lengths), num_q_heads=8,
                         num_kv_heads=1, kv_dtype="fp8_e4m3", lengths_kind="fixed",
                         fixed_lengths=lengths)
    for i, (name, lengths) in enumerate([
        ("64x0.5K", _mix((64, K // 2))),
        ("64x4K", _mix((64, 4 * K))),
        ("32x0.125K+32x4K", _mix((32, K // 8), (32, 4 * K))),
        ("2x32K+30x4K", _mix((2, 32 * K), (30, 4 * K))),
        ("1x64K+15x4K", _mix((1, 64 * K), (15, 4 * K))),
        ("1x128K+31x4K", _mix((1, 128 * K), (31, 4 * K))),
    ])
}


def get_config(name: str) -> WorkloadConfig:
    if name in CONFIGS:
        return CONFIGS[name]
    if name in TABLE3:
        return TABLE3[name]
    raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS) + sorted(TABLE3)}")
