"""fp64 paged GQA decode attention (oracle; test infrastructure only).

What the hot path computes, written out plainly:

* Decode attention: each request contributes one query token per query head;
  it attends over all of the request's cached tokens (SGLang x HPC-Ops page,
  "Attention: load balancing for mixed-length decode").
* GQA: the query heads are split into ``H_kv`` contiguous groups of
  ``G = Hq / H_kv`` heads, and group g reads KV head g (the Hy3 shape of the
  vLLM x HPC-Ops page has 64 query heads over 8 KV heads; the pages do not
  spell out the head map, contiguous groups is the plain reading).
* Paged KV: token t of request r lives in page ``page_table[r][t // 64]`` at
  slot ``t % 64``; the cache is ``[page][kv_head][slot][dim]``.
* Scores ``s_t = sm_scale * <q, k_t>``, a softmax over the request's tokens,
  output ``sum_t p_t v_t``.
* Split form (SGLang x HPC-Ops page, "Scheduling around live KV work"; vLLM x
  HPC-Ops page, "Compute and combine"): attention over a token range gives a
  normalised partial output and its log-sum-exp; partials of one
  (KV head, request) pair merge under the global softmax normalisation.
* FP8 KV: a stored value is ``e4m3(code) * scale`` with one fp32 scale per
  (token, KV head).

All arithmetic is float64.  bf16 inputs are taken as raw 16-bit patterns and
widened exactly (a bf16 is the top half of an IEEE binary32).
"""

from __future__ import annotations

import numpy as np

from . import e4m3

PAGE_TOKENS = 64


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def gather_pair_kv(cache, page_table_row, kv_head: int, length: int,
                   kv_dtype: str = "bf16", scale=None) -> np.ndarray:
    """Logical [length, D] fp64 rows of one (request, KV head) from the paged cache."""
    t = np.arange(length)
    pages = np.asarray(page_table_row, dtype=np.int64)[t // PAGE_TOKENS]
    slots = t % PAGE_TOKENS
    raw = np.asarray(cache)[pages, kv_head, slots, :]
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if kv_dtype == "fp8_e4m3":
        s = np.asarray(scale, dtype=np.float64)[pages, kv_head, slots]
        return e4m3.decode(raw) * s[:, None]
    raise ValueError(kv_dtype)


def attend_range(q_group: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """Softmax attention of G query rows over n key/value rows.

    Returns (o [G, D] normalised, lse [G] natural log).  With n == 0 the
    output is zero and the log-sum-exp is -inf (no mass).
    """
    q_group = np.asarray(q_group, dtype=np.float64)
    G, D = q_group.shape
    if K.shape[0] == 0:
        return np.zeros((G, V.shape[1] if V.ndim == 2 else D)), np.full(G, -np.inf)
    s = sm_scale * (q_group @ K.T)                 # [G, n]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1, keepdims=True)
    o = (w @ V) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def combine(partials):
    """Merge (o_k, lse_k) partials of one pair under the global normalisation."""
    partials = list(partials)
    if not partials:
        raise ValueError("no partials")
    lses = np.stack([p[1] for p in partials])      # [k, G]
    G, D = partials[0][0].shape
    M = lses.max(axis=0)                           # [G]
    out = np.zeros((G, D))
    tot = np.zeros(G)
    for o_k, lse_k in partials:
        w = np.where(np.isneginf(lse_k), 0.0, np.exp(lse_k - np.where(np.isneginf(M), 0.0, M)))
        out += w[:, None] * o_k
        tot += w
    has = tot > 0
    out[has] /= tot[has, None]
    lse = np.where(has, M + np.log(np.where(has, tot, 1.0)), -np.inf)
    return out, lse


def paged_decode_attention(q, k_cache, v_cache, page_table, seq_lens, num_kv_heads: int,
                           sm_scale: float, kv_dtype: str = "bf16", k_scale=None,
                           v_scale=None, pairs=None):
    """out [B, Hq, D] and lse [B, Hq] (float64) of paged GQA decode attention.

    ``q`` is float64 [B, Hq, D] (see :func:`bf16_bits_to_f64`).  ``pairs``
    optionally restricts the work to an iterable of (kv_head, request); rows
    outside it are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    G = Hq // num_kv_heads
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    todo = [(g, r) for g in range(num_kv_heads) for r in range(B)] if pairs is None else pairs
    for g, r in todo:
        L = int(seq_lens[r])
        K = gather_pair_kv(k_cache, page_table[r], g, L, kv_dtype, k_scale)
        V = gather_pair_kv(v_cache, page_table[r], g, L, kv_dtype, v_scale)
        o, l = attend_range(q[r, g * G:(g + 1) * G], K, V, sm_scale)
        out[r, g * G:(g + 1) * G] = o
        lse[r, g * G:(g + 1) * G] = l
    return out, lse


def paged_verify_attention(q, k_cache, v_cache, page_table, seq_lens, num_kv_heads: int,
                           sm_scale: float, kv_dtype: str = "bf16", k_scale=None,
                           v_scale=None, pairs=None):
    """Multi-token decode (speculative verification): out [B, T, Hq, D] and
    lse [B, T, Hq] for T query tokens per request.

    ``q`` is float64 [B, T, Hq, D].  Token j of request r sits at position
    L_r - T + j and attends causally to the KV positions up to and including
    its own, i.e. to the first max(0, L_r - T + j + 1) tokens of the request
    (no position: zeros and lse -inf).  T = 1 is plain decode.
    """
    q = np.asarray(q, dtype=np.float64)
    B, T, Hq, D = q.shape
    L = np.asarray(seq_lens, dtype=np.int64)
    out = np.full((B, T, Hq, D), np.nan)
    lse = np.full((B, T, Hq), np.nan)
    for j in range(T):
        visible = np.clip(L - T + j + 1, 0, L)
        out[:, j], lse[:, j] = paged_decode_attention(q[:, j], k_cache, v_cache, page_table,
                                                      visible, num_kv_heads, sm_scale, kv_dtype,
                                                      k_scale, v_scale, pairs)
    return out, lse


def split_decode_attention(q, k_cache, v_cache, page_table, seq_lens, num_kv_heads: int,
                           sm_scale: float, desc, kv_dtype: str = "bf16", k_scale=None,
                           v_scale=None):
    """Attention computed per task descriptor, then merged per pair.

    ``desc`` rows are (kv_head, request, token_begin, token_end).  Returns the
    merged out [B, Hq, D]; pairs without descriptors give zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    G = Hq // num_kv_heads
    parts = {}
    for g, r, a, b in np.asarray(desc).reshape(-1, 4):
        g, r, a, b = int(g), int(r), int(a), int(b)
        K = gather_pair_kv(k_cache, page_table[r], g, b, kv_dtype, k_scale)[a:b]
        V = gather_pair_kv(v_cache, page_table[r], g, b, kv_dtype, v_scale)[a:b]
        parts.setdefault((g, r), []).append(attend_range(q[r, g * G:(g + 1) * G], K, V,
                                                         sm_scale))
    out = np.zeros((B, Hq, D))
    for (g, r), ps in parts.items():
        out[r, g * G:(g + 1) * G] = combine(ps)[0]
    return out
