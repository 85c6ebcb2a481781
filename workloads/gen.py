"""Seeded generators for decode-attention inputs.

Recipe (stated once here and relied on by tests and the benchmark):

* Request lengths come first from ``numpy.random.default_rng(seed)``.
  Log-uniform draws are ``clip(floor(exp(U[ln lo, ln hi))), lo, hi)``; the
  skewed mix puts ``long_length`` at request 0 and draws the others as
  integers uniform on ``[lo, hi]``.
* The page table is drawn next from the same generator: the pool has
  ``P = sum(ceil(L_r / 64))`` pages, ``rng.permutation(P)`` is dealt to the
  requests in order, and unused page-table entries are 0 (a valid page, so a
  stray read can never leave the pool).
* Tensors are drawn with a torch generator seeded ``1000 * seed + layer`` on
  the target device: first ``q [B, Hq, D]`` bf16 ~ N(0, 1); then the caches
  page-chunk by page-chunk (``PAGE_CHUNK`` pages at a time), K before V in
  each chunk.  KV caches are ``[P, H_kv, 64, D]`` (page, head, slot, dim).
* FP8 queries (``quantize_query_e4m3``) are derived from the BF16 ``q``:
  per (request, query head) scale = max |q| / 448, codes = e4m3 RNE of
  ``q / scale``.
* FP8 caches: ``x ~ N(0, 1)`` fp32 and a scale ``s ~ U[lo, hi]`` per
  (page, head, slot); the stored code is the OCP e4m3 round-to-nearest-even
  of ``clamp(x / s, -448, 448)`` (torch's e4m3 cast does not saturate, so the
  clamp comes first).  The scales are ``[P, H_kv, 64]`` fp32.

Nothing here implements attention or scheduling.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

from .configs import WorkloadConfig

PAGE_CHUNK = 2048
E4M3_MAX = 448.0


def draw_lengths(cfg: WorkloadConfig, rng: np.random.Generator) -> np.ndarray:
    B = cfg.batch
    if cfg.lengths_kind == "fixed":
        lens = np.asarray(cfg.fixed_lengths, dtype=np.int64)
        assert lens.shape == (B,)
    elif cfg.lengths_kind == "uniform":
        lens = np.full(B, cfg.length_lo, dtype=np.int64)
    elif cfg.lengths_kind == "loguniform":
        u = rng.uniform(math.log(cfg.length_lo), math.log(cfg.length_hi), size=B)
        lens = np.clip(np.floor(np.exp(u)).astype(np.int64), cfg.length_lo, cfg.length_hi)
    elif cfg.lengths_kind == "skewed":
        rest = rng.integers(cfg.length_lo, cfg.length_hi + 1, size=B - 1)
        lens = np.concatenate([[cfg.long_length], rest]).astype(np.int64)
    else:
        raise ValueError(cfg.lengths_kind)
    return lens.astype(np.int32)


def draw_page_table(lengths: Sequence[int], rng: np.random.Generator,
                    page_size: int = 64, max_pages_per_seq: Optional[int] = None):
    """Returns (page_table int32 [B, max_pages], num_pages)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    n_pages = (lengths + page_size - 1) // page_size
    P = int(n_pages.sum())
    width = int(n_pages.max()) if len(n_pages) else 0
    if max_pages_per_seq is not None:
        assert max_pages_per_seq >= width
        width = max_pages_per_seq
    width = max(width, 1)
    perm = rng.permutation(P) if P > 0 else np.zeros(0, dtype=np.int64)
    table = np.zeros((len(lengths), width), dtype=np.int32)
    off = 0
    for r, n in enumerate(n_pages):
        table[r, :n] = perm[off:off + n]
        off += n
    return table, P


@dataclasses.dataclass
class Layer:
    q: torch.Tensor                       # [B, Hq, D] bf16
    k_cache: torch.Tensor                 # [P, H_kv, 64, D] bf16 or uint8 (e4m3 codes)
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor] = None  # [P, H_kv, 64] fp32 (FP8 only)
    v_scale: Optional[torch.Tensor] = None


@dataclasses.dataclass
class Workload:
    cfg: WorkloadConfig
    lengths: np.ndarray                   # int32 [B]
    page_table: np.ndarray                # int32 [B, max_pages]
    num_pages: int
    layers: list

    @property
    def total_tokens(self) -> int:
        return int(np.asarray(self.lengths, dtype=np.int64).sum())

    @property
    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one layer's attention must read."""
        return self.total_tokens * self.cfg.num_kv_heads * self.cfg.kv_bytes_per_token_head


def _fp8_codes(x: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    y = torch.clamp(x / s.unsqueeze(-1), -E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def quantize_query_e4m3(q: torch.Tensor):
    """An FP8 query in the form the fused attention prologue hands it over:
    one fp32 scale per (request, query head) = max |q| over the head's dims
    / 448 (1 for an all-zero row), codes = e4m3 RNE of q / scale.  Returns
    (codes uint8 [B, Hq, D], scale fp32 [B, Hq]) on q's device."""
    x = q.float()
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    return _fp8_codes(x, scale), scale


def rope_cos_sin_table(max_position: int, head_dim: int = 128, theta: float = 1.0e6,
                       device="cpu") -> torch.Tensor:
    """The caller-side RoPE table the prologue reads: row p holds cos(p * f_i)
    for the head_dim / 2 frequencies f_i = theta^(-2i / head_dim), then
    sin(p * f_i); computed in fp64 and stored as fp32."""
    h = head_dim // 2
    f = theta ** (-2.0 * np.arange(h) / head_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * f[None, :]
    tab = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    return torch.from_numpy(tab).to(device)


def make_prologue_inputs(batch: int, num_q_heads: int, num_kv_heads: int, seed: int,
                         device="cpu", head_dim: int = 128):
    """Seeded inputs of the fused prologue: the QKV projection of one token per
    request (bf16 ~ N(0, 1) * 2, query heads then key then value heads) and the
    two QK-Norm weight vectors (fp32 ~ 1 + 0.1 N(0, 1))."""
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(7000 + seed)
    H3 = num_q_heads + 2 * num_kv_heads
    qkv = (2 * torch.randn((batch, H3 * head_dim), generator=g, device=device)).to(torch.bfloat16)
    qw = 1 + 0.1 * torch.randn(head_dim, generator=g, device=device)
    kw = 1 + 0.1 * torch.randn(head_dim, generator=g, device=device)
    return qkv, qw, kw


def make_layer(*, batch: int, num_q_heads: int, num_kv_heads: int, num_pages: int,
               kv_dtype: str, seed: int, layer: int, device="cpu", head_dim: int = 128,
               page_size: int = 64, fp8_scale_lo: float = 0.01,
               fp8_scale_hi: float = 0.1) -> Layer:
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(1000 * seed + layer)
    q = torch.randn((batch, num_q_heads, head_dim), generator=g, device=device,
                    dtype=torch.float32).to(torch.bfloat16)
    shape = (num_pages, num_kv_heads, page_size, head_dim)
    if kv_dtype == "bf16":
        k = torch.empty(shape, dtype=torch.bfloat16, device=device)
        v = torch.empty(shape, dtype=torch.bfloat16, device=device)
        for p0 in range(0, num_pages, PAGE_CHUNK):
            p1 = min(num_pages, p0 + PAGE_CHUNK)
            cs = (p1 - p0,) + shape[1:]
            k[p0:p1] = torch.randn(cs, generator=g, device=device, dtype=torch.float32)
            v[p0:p1] = torch.randn(cs, generator=g, device=device, dtype=torch.float32)
        return Layer(q, k, v)
    if kv_dtype != "fp8_e4m3":
        raise ValueError(kv_dtype)
    k = torch.empty(shape, dtype=torch.uint8, device=device)
    v = torch.empty(shape, dtype=torch.uint8, device=device)
    ks = torch.empty(shape[:3], dtype=torch.float32, device=device)
    vs = torch.empty(shape[:3], dtype=torch.float32, device=device)
    span = fp8_scale_hi - fp8_scale_lo
    for p0 in range(0, num_pages, PAGE_CHUNK):
        p1 = min(num_pages, p0 + PAGE_CHUNK)
        cs = (p1 - p0,) + shape[1:]
        for codes, scales in ((k, ks), (v, vs)):
            x = torch.randn(cs, generator=g, device=device, dtype=torch.float32)
            s = fp8_scale_lo + span * torch.rand(cs[:3], generator=g, device=device,
                                                 dtype=torch.float32)
            codes[p0:p1] = _fp8_codes(x, s)
            scales[p0:p1] = s
    return Layer(q, k, v, ks, vs)


def make_workload(cfg: WorkloadConfig, device="cpu", layers: Optional[int] = None,
                  lengths: Optional[Sequence[int]] = None) -> Workload:
    rng = np.random.default_rng(cfg.seed)
    lens = draw_lengths(cfg, rng) if lengths is None else np.asarray(lengths, np.int32)
    table, P = draw_page_table(lens, rng, cfg.page_size)
    n_layers = cfg.layers if layers is None else layers
    ls = [make_layer(batch=cfg.batch if lengths is None else len(lens),
                     num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
                     num_pages=P, kv_dtype=cfg.kv_dtype, seed=cfg.seed, layer=i,
                     device=device, head_dim=cfg.head_dim, page_size=cfg.page_size,
                     fp8_scale_lo=cfg.fp8_scale_lo, fp8_scale_hi=cfg.fp8_scale_hi)
          for i in range(n_layers)]
    return Workload(cfg, lens, table, P, ls)


BF16_NAN_BITS = 0x7FC0
E4M3_NAN_CODE = 0x7F


def poison_tail_slots(layer: Layer, lengths, page_table, page_size: int = 64) -> None:
    """Fill every slot past a request's last token (inside its last page) with NaN."""
    for r, L in enumerate(np.asarray(lengths)):
        L = int(L)
        if L % page_size == 0 or L == 0:
            continue
        page = int(page_table[r, L // page_size])
        slot0 = L % page_size
        if layer.k_cache.dtype == torch.bfloat16:
            nan = torch.tensor(BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16).item()
            layer.k_cache[page, :, slot0:, :] = nan
            layer.v_cache[page, :, slot0:, :] = nan
        else:
            layer.k_cache[page, :, slot0:, :] = E4M3_NAN_CODE
            layer.v_cache[page, :, slot0:, :] = E4M3_NAN_CODE
            layer.k_scale[page, :, slot0:] = float("nan")
            layer.v_scale[page, :, slot0:] = float("nan")
