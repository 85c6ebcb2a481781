"""fp64 oracle of the fused attention prologue (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this package; the product never does.

What the step computes (SGLang x HPC-Ops page, "A fused attention
prologue"; vLLM x HPC-Ops page, the HpcRopeNorm paragraph of the Attention
backend section): from the fused QKV projection of one decode token per
request, QK-Norm is applied to every query and key head before RoPE, K and V
are written straight into the paged cache, and with an FP8 cache the query
is emitted in FP8 with one scale per token and head.  Readings where the
pages are silent:

* QK-Norm is RMSNorm over the head's 128 dims with a learned weight per dim
  (one weight vector for query heads, one for key heads):
  y = x / sqrt(mean(x^2) + eps) * w.
* RoPE rotates dim pairs (i, i + 64) ("rotate half") by the angles of the
  token's position, taken from a caller-supplied table whose row p holds
  cos(p * f_i) for i < 64 followed by sin(p * f_i).
* The T new tokens of request r (T = 1 for plain decode) sit at positions
  seq_lens[r] - T + j (the lengths already count them); negative positions
  have no token; positions past the table use its last row.
* FP8 outputs (the query; K and V in an FP8 cache) use one scale per
  (token, head) = max |x| / 448 (1 for an all-zero row); the code is the
  e4m3 value nearest to x / scale, ties to even.
* A BF16 cache stores K after norm and RoPE rounded to BF16 (nearest, ties
  to even) and V as given.

Everything is fp64 except the final roundings, which are exact.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import E4M3_TABLE

E4M3_MAX = 448.0

# finite non-negative e4m3 values in increasing order with their codes
_POS_CODES = np.array([c for c in range(0x80) if np.isfinite(E4M3_TABLE[c])], dtype=np.int64)
_POS_VALUES = E4M3_TABLE[_POS_CODES]


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope_rotate_half(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate pairs (i, i + D/2) of the last axis by angles with the given
    cos and sin (both [..., D/2], broadcast against x's leading axes)."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def e4m3_round(y: np.ndarray) -> np.ndarray:
    """Codes of the e4m3 values nearest to y (|y| <= 448), ties to the even
    code; the sign bit follows the sign of y (negative values that round to
    zero give the negative-zero code 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("e4m3_round needs |y| <= 448")
    a = np.abs(y)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, None)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    mag = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    sign = np.signbit(y).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8)


def quantize_rows_e4m3(x: np.ndarray):
    """Per-row (last axis) FP8 quantization: scale = max |x| / 448 (1 for an
    all-zero row) and codes = e4m3_round(x / scale).  Returns (codes uint8,
    scale fp64, the unrounded x / scale)."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / E4M3_MAX, 1.0)
    # |x / scale| <= 448 holds exactly; the clip only removes the fp64
    # rounding of the row maximum's own quotient
    y = np.clip(x / scale[..., None], -E4M3_MAX, E4M3_MAX)
    return e4m3_round(y), scale, y


def bf16_round(x: np.ndarray) -> np.ndarray:
    """x rounded to the nearest BF16 value (8 significant bits), ties to
    even, returned as fp64 (normal range)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                    # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def prologue(qkv: np.ndarray, seq_lens, num_q_heads: int, num_kv_heads: int,
             q_norm_w: np.ndarray, k_norm_w: np.ndarray, eps: float, cos_sin: np.ndarray):
    """The exact (unrounded) outputs of the prologue for the new tokens of one
    step.

    qkv: [B, (Hq + 2 Hkv) * D] (one new token per request) or
    [B, T, (Hq + 2 Hkv) * D] (T new tokens, token j of request r at position
    seq_lens[r] - T + j): query heads, then key heads, then value heads.
    cos_sin: [max_position, D] (cos of the D/2 frequencies, then their sin).
    Returns dict with q [..., Hq, D] and k [..., Hkv, D] (normed and
    rotated), v [..., Hkv, D], and pos (the position used; negative: no
    token), where ... is [B] or [B, T] like qkv.
    """
    qkv = np.asarray(qkv, dtype=np.float64)
    single = qkv.ndim == 2
    if single:
        qkv = qkv[:, None, :]
    B, T = qkv.shape[:2]
    D = cos_sin.shape[1]
    H3 = num_q_heads + 2 * num_kv_heads
    x = qkv.reshape(B, T, H3, D)
    q = x[:, :, :num_q_heads]
    k = x[:, :, num_q_heads:num_q_heads + num_kv_heads]
    v = x[:, :, num_q_heads + num_kv_heads:]
    L = np.asarray(seq_lens, dtype=np.int64)
    pos = L[:, None] - T + np.arange(T)[None, :]          # [B, T]
    row = np.clip(pos, 0, cos_sin.shape[0] - 1)
    cos = cos_sin[row, :D // 2][:, :, None, :]
    sin = cos_sin[row, D // 2:][:, :, None, :]
    qn = rope_rotate_half(rms_norm(q, q_norm_w, eps), cos, sin)
    kn = rope_rotate_half(rms_norm(k, k_norm_w, eps), cos, sin)
    out = {"q": qn, "k": kn, "v": v.copy(), "pos": np.where(pos >= 0, pos, -1)}
    if single:
        out = {key: val[:, 0] for key, val in out.items()}
    return out
