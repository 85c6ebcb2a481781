"""Shared set-up for the GPU parity tests.

Builds seeded workloads on the device, runs the HIP path through the C ABI
(via the ctypes binding) and computes the CPU oracle's answer on host copies
of the very same tensors.
"""

from __future__ import annotations

import dataclasses
import math
import sys
from typing import Optional, Sequence

import numpy as np
import torch

import load_balanced_paged_amd as lbp
import oracle
from workloads import WorkloadConfig, make_workload, poison_tail_slots

BF16_MAX_ABS = 1e-2
BF16_REL_RMS = 5e-3
FP8_MAX_ABS = 3e-2
# Per (KV head, request) pair, every KV format: ||out - ref||_2 / ||ref||_2 over
# the pair's G x 128 (x q_len) outputs.  The output's own BF16 rounding gives
# about 1.1e-3 and a BF16 probability about as much again; a pair whose rows
# were zeroed or lost gives 1.  Long rows are small in magnitude (about
# sqrt(e / L) at unit-spread inputs), so the absolute bounds alone cannot see
# them.
PAIR_REL_RMS = 1e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class Case:
    wcfg: WorkloadConfig
    wl: object
    cfg: lbp.lbp_config
    seq_lens: torch.Tensor
    page_table: torch.Tensor
    plan_ws: torch.Tensor
    split_ws: torch.Tensor
    info: Optional[lbp.lbp_plan_info] = None

    @property
    def G(self):
        return self.wcfg.group


def build_case(wcfg: WorkloadConfig, layers: int = 1, lengths: Optional[Sequence[int]] = None,
               num_workgroups: int = 0, min_tiles: int = 0, poison: bool = True,
               policy: int = lbp.LBP_POLICY_DYNAMIC, param: int = 0,
               max_pages_per_seq: Optional[int] = None, q_len: int = 1) -> Case:
    say(f"[case] {wcfg.name} B={wcfg.batch if lengths is None else len(lengths)} "
        f"Hq={wcfg.num_q_heads} Hkv={wcfg.num_kv_heads} kv={wcfg.kv_dtype} layers={layers} "
        f"W={num_workgroups} F={min_tiles} policy={policy} param={param}")
    wl = make_workload(wcfg, device="cuda", layers=layers, lengths=lengths)
    if poison:
        for layer in wl.layers:
            poison_tail_slots(layer, wl.lengths, wl.page_table)
    mp = max_pages_per_seq or wl.page_table.shape[1]
    table = np.zeros((len(wl.lengths), mp), dtype=np.int32)
    table[:, :wl.page_table.shape[1]] = wl.page_table
    cfg = lbp.make_config(wcfg.num_q_heads, wcfg.num_kv_heads, len(wl.lengths), mp,
                          kv_dtype=wcfg.kv_dtype, num_workgroups=num_workgroups,
                          min_tiles_per_bin=min_tiles, sm_scale=wcfg.sm_scale, q_len=q_len)
    pb, sb = lbp.lbp_query_workspace(cfg, policy, param)
    case = Case(wcfg, wl, cfg,
                torch.from_numpy(np.asarray(wl.lengths, dtype=np.int32)).cuda(),
                torch.from_numpy(table).cuda(),
                torch.zeros(pb, dtype=torch.uint8, device="cuda"),
                torch.zeros(sb, dtype=torch.uint8, device="cuda"))
    if policy == lbp.LBP_POLICY_DYNAMIC:
        case.info = lbp.lbp_plan(cfg, case.seq_lens, case.page_table, case.plan_ws)
    else:
        case.info = lbp.lbp_plan_static(cfg, policy, param, case.seq_lens, case.page_table,
                                        case.plan_ws)
    return case


def run_attend(case: Case, layer: int = 0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    L = case.wl.layers[layer]
    if out is None:
        out = torch.empty_like(L.q)
    lbp.lbp_attend(case.cfg, case.info, case.plan_ws, L.q, L.k_cache, L.v_cache, L.k_scale,
                   L.v_scale, case.split_ws, out)
    torch.cuda.synchronize()
    return out


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_taskmap(case: Case):
    info = case.info
    L = np.asarray(case.wl.lengths)
    H = case.wcfg.num_kv_heads
    if info.policy == lbp.LBP_POLICY_DYNAMIC:
        return oracle.assign.assign_dynamic(L, H, info.num_bins, info.param)
    if info.policy == lbp.LBP_POLICY_STATIC_SPLITS:
        return oracle.assign.assign_static_splits(L, H, info.param)
    return oracle.assign.assign_static_chunk(L, H, info.param, case.cfg.max_pages_per_seq)


def assert_taskmap_matches(case: Case):
    got = lbp.read_taskmap(case.plan_ws, case.info)
    ref = oracle_taskmap(case)
    assert got["magic"] == lbp.LBP_PLAN_MAGIC
    assert got["status"] == 0
    assert got["num_bins"] == ref.num_bins == case.info.num_bins
    assert got["header"] == ref.header(), (got["header"], ref.header())
    assert np.array_equal(got["bin_offset"], ref.bin_offset)
    assert np.array_equal(got["desc"], ref.desc)
    assert np.array_equal(got["pair_first"], ref.pair_first)
    assert np.array_equal(got["pair_count"], ref.pair_count)
    assert np.array_equal(got["split_list"], expected_split_list(ref))
    for b in range(ref.num_bins):
        d0, d1 = ref.bin_offset[b], ref.bin_offset[b + 1]
        want = ref.desc[d0] if d1 > d0 else np.zeros(4, np.int32)
        assert np.array_equal(got["bin_first"][b], want), b
    assert np.array_equal(got["bin_pages"], expected_bin_pages(ref, np.asarray(case.wl.page_table)))
    return got, ref


def expected_bin_pages(ref, table):
    """Per bin, the pages of its first descriptor's first tile and of the
    next one (the first again for a one-tile descriptor); zeros for an empty
    bin."""
    out = np.zeros((ref.num_bins, 2), np.int32)
    for b in range(ref.num_bins):
        d0, d1 = ref.bin_offset[b], ref.bin_offset[b + 1]
        if d1 > d0:
            _, r, lo, hi = (int(x) for x in ref.desc[d0])
            t0 = lo // 64
            out[b] = (table[r, t0], table[r, min(t0 + 1, (hi - 1) // 64)])
    return out


def expected_split_list(ref):
    """(pair, first, count, 0) for every pair the oracle's map splits, in pair order."""
    rows = [(p, ref.pair_first[p], c, 0) for p, c in enumerate(ref.pair_count) if c >= 2]
    return np.asarray(rows, dtype=np.int32).reshape(-1, 4)


def oracle_pairs(case: Case, layer: int, pairs, q64: Optional[np.ndarray] = None):
    """fp64 oracle output rows for (kv_head, request) pairs, from host copies.

    q64, if given, replaces the layer's BF16 query ([B, Hq, 128] fp64, e.g.
    the values of an FP8 query).

    The pages of each sampled request are gathered on the device into a
    compact cache (identity page table) before the host copy, so only the
    bytes the sampled pairs need cross PCIe; the oracle then does its own
    per-token page and slot indexing on that cache.
    """
    Lyr = case.wl.layers[layer]
    G = case.G
    fp8 = case.wcfg.kv_dtype == "fp8_e4m3"
    res = {}
    for g, r in pairs:
        Lr = int(case.wl.lengths[r])
        n = max(1, (Lr + 63) // 64)
        pages = case.page_table[r, :n].long()
        kc = Lyr.k_cache.index_select(0, pages)[:, g:g + 1].contiguous()
        vc = Lyr.v_cache.index_select(0, pages)[:, g:g + 1].contiguous()
        if q64 is None:
            q = oracle.attention.bf16_bits_to_f64(bits(Lyr.q[r:r + 1, g * G:(g + 1) * G]))
        else:
            q = q64[r:r + 1, g * G:(g + 1) * G]
        table = np.arange(n, dtype=np.int32)[None]
        if fp8:
            ks = Lyr.k_scale.index_select(0, pages)[:, g:g + 1].contiguous().cpu().numpy()
            vs = Lyr.v_scale.index_select(0, pages)[:, g:g + 1].contiguous().cpu().numpy()
            o, lse = oracle.attention.paged_decode_attention(
                q, kc.cpu().numpy(), vc.cpu().numpy(), table, [Lr], 1, case.wcfg.sm_scale,
                kv_dtype="fp8_e4m3", k_scale=ks, v_scale=vs)
        else:
            o, lse = oracle.attention.paged_decode_attention(
                q, bits(kc), bits(vc), table, [Lr], 1, case.wcfg.sm_scale)
        if Lr == 0:
            o = np.zeros_like(o)   # a pair with no tokens outputs zeros
        res[(g, r)] = o[0]
    return res


def oracle_verify_pairs(case: Case, layer: int, pairs, q64: np.ndarray):
    """fp64 oracle rows [T, G, D] of multi-token verification for (kv_head,
    request) pairs; q64 is the query [B, T, Hq, D] in fp64."""
    Lyr = case.wl.layers[layer]
    G = case.G
    fp8 = case.wcfg.kv_dtype == "fp8_e4m3"
    res = {}
    for g, r in pairs:
        Lr = int(case.wl.lengths[r])
        n = max(1, (Lr + 63) // 64)
        pages = case.page_table[r, :n].long()
        kc = Lyr.k_cache.index_select(0, pages)[:, g:g + 1].contiguous()
        vc = Lyr.v_cache.index_select(0, pages)[:, g:g + 1].contiguous()
        q = q64[r:r + 1, :, g * G:(g + 1) * G]
        table = np.arange(n, dtype=np.int32)[None]
        if fp8:
            ks = Lyr.k_scale.index_select(0, pages)[:, g:g + 1].contiguous().cpu().numpy()
            vs = Lyr.v_scale.index_select(0, pages)[:, g:g + 1].contiguous().cpu().numpy()
            o, _ = oracle.attention.paged_verify_attention(
                q, kc.cpu().numpy(), vc.cpu().numpy(), table, [Lr], 1, case.wcfg.sm_scale,
                kv_dtype="fp8_e4m3", k_scale=ks, v_scale=vs)
        else:
            o, _ = oracle.attention.paged_verify_attention(q, bits(kc), bits(vc), table, [Lr], 1,
                                                           case.wcfg.sm_scale)
        res[(g, r)] = o[0]
    return res


def oracle_verify_layer(case: Case, layer: int, q64: np.ndarray, pairs=None,
                        workers: Optional[int] = None):
    """fp64 oracle rows [T, G, D] of multi-token verification for `pairs`
    (default: every pair) of a layer, for whole-layer verification parity.

    Like oracle_layer: the layer's caches are copied to the host once, and
    the pairs run longest first on a thread pool (one BLAS thread per
    worker), each through oracle.attention.paged_verify_attention over its
    own pages."""
    import concurrent.futures
    import os
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    Lyr = case.wl.layers[layer]
    G = case.G
    fp8 = case.wcfg.kv_dtype == "fp8_e4m3"
    lengths = np.asarray(case.wl.lengths)
    if pairs is None:
        pairs = all_pairs(case)
    if fp8:
        kc, vc = Lyr.k_cache.cpu().numpy(), Lyr.v_cache.cpu().numpy()
        ks, vs = Lyr.k_scale.cpu().numpy(), Lyr.v_scale.cpu().numpy()
    else:
        kc, vc, ks, vs = bits(Lyr.k_cache), bits(Lyr.v_cache), None, None
    table = np.asarray(case.wl.page_table)

    def one(pair):
        g, r = pair
        Lr = int(lengths[r])
        n = max(1, (Lr + 63) // 64)
        pages = table[r, :n].astype(np.int64)
        sub = np.arange(n, dtype=np.int32)[None]
        q = q64[r:r + 1, :, g * G:(g + 1) * G]
        kw = {}
        if fp8:
            kw = dict(kv_dtype="fp8_e4m3", k_scale=ks[pages][:, g:g + 1],
                      v_scale=vs[pages][:, g:g + 1])
        o, _ = oracle.attention.paged_verify_attention(
            q, kc[pages][:, g:g + 1], vc[pages][:, g:g + 1], sub, [Lr], 1,
            case.wcfg.sm_scale, **kw)
        return pair, o[0]

    order = sorted(pairs, key=lambda p: -int(lengths[p[1]]))
    n = workers or min(16, len(os.sched_getaffinity(0)))
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        with concurrent.futures.ThreadPoolExecutor(n) as ex:
            res = dict(ex.map(one, order))
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    return {p: res[p] for p in pairs}


def parity_stats(got_rows, ref_rows, lengths=None):
    """Error statistics of stacked pair outputs ([n_pairs, ...] fp64 each).

    Returns max-abs, the relative RMS over everything compared, and the
    worst per-pair relative RMS with its index (pairs whose reference is
    exactly zero, i.e. no visible token, must be exactly zero instead)."""
    a = np.asarray(got_rows, dtype=np.float64)
    b = np.asarray(ref_rows, dtype=np.float64)
    diff = a - b
    n = a.shape[0]
    d2 = np.sqrt(np.sum(diff.reshape(n, -1) ** 2, axis=1))
    r2 = np.sqrt(np.sum(b.reshape(n, -1) ** 2, axis=1))
    zero_ref = r2 == 0
    per_pair = np.where(zero_ref, np.where(d2 == 0, 0.0, np.inf), d2 / np.where(zero_ref, 1, r2))
    worst = int(np.argmax(per_pair)) if n else 0
    return {
        "finite": bool(np.all(np.isfinite(a))),
        "max_abs": float(np.max(np.abs(diff))) if n else 0.0,
        "rel_rms": float(np.linalg.norm(diff) / max(np.linalg.norm(b), 1e-30)),
        "pair_rel_max": float(per_pair[worst]) if n else 0.0,
        "pair_rel_median": float(np.median(per_pair)) if n else 0.0,
        "worst": worst,
        "worst_len": int(lengths[worst]) if lengths is not None and n else None,
    }


def check_parity(kv_dtype, st, what=""):
    """The tolerances: BF16 KV max-abs <= 1e-2 and relative RMS <= 5e-3, FP8
    KV max-abs <= 3e-2, and every pair within PAIR_REL_RMS."""
    assert st["finite"], f"{what}: non-finite output"
    if kv_dtype == "bf16":
        assert st["max_abs"] <= BF16_MAX_ABS, (what, st)
        assert st["rel_rms"] <= BF16_REL_RMS, (what, st)
    else:
        assert st["max_abs"] <= FP8_MAX_ABS, (what, st)
    assert st["pair_rel_max"] <= PAIR_REL_RMS, (what, st)


def _report(what, keys, st):
    g, r = keys[st["worst"]] if keys else (None, None)
    say(f"[parity] {what}: pairs={len(keys)} max_abs={st['max_abs']:.3e} "
        f"rel_rms={st['rel_rms']:.3e} pair_rel median={st['pair_rel_median']:.3e} "
        f"worst={st['pair_rel_max']:.3e} at (kv_head {g}, request {r}, L={st['worst_len']})")


def compare_verify(case: Case, got: torch.Tensor, ref_rows: dict, what=""):
    """compare() for [B, T, Hq, D] outputs: rows [r, :, g*G:(g+1)*G] per pair."""
    G = case.G
    gv = bf16_to_f64(got)
    keys = list(ref_rows)
    a = np.stack([gv[r, :, g * G:(g + 1) * G] for (g, r) in keys])
    b = np.stack([ref_rows[k] for k in keys])
    st = parity_stats(a, b, [case.wl.lengths[r] for _, r in keys])
    _report(what, keys, st)
    check_parity(case.wcfg.kv_dtype, st, what)
    return st["max_abs"], st["rel_rms"]


def compare(case: Case, got: torch.Tensor, ref_rows: dict, what=""):
    """Stack the compared pairs and apply the tolerances of the KV dtype; with
    every pair present the relative RMS is over the whole output tensor."""
    G = case.G
    gv = bf16_to_f64(got)
    keys = list(ref_rows)
    a = np.stack([gv[r, g * G:(g + 1) * G] for (g, r) in keys])
    b = np.stack([ref_rows[k] for k in keys])
    st = parity_stats(a, b, [case.wl.lengths[r] for _, r in keys])
    _report(what, keys, st)
    check_parity(case.wcfg.kv_dtype, st, what)
    return st["max_abs"], st["rel_rms"]


def oracle_layer(case: Case, layer: int, pairs=None, q64: Optional[np.ndarray] = None,
                 workers: Optional[int] = None):
    """fp64 oracle output rows [G, 128] for `pairs` (default: every pair) of a
    decode layer, for whole-layer parity.

    The layer's query and caches are copied to the host once; the oracle
    then gathers each pair's pages itself.  Pairs run longest first on a
    thread pool (one BLAS thread per worker; NumPy releases the GIL in the
    gathers and products)."""
    import concurrent.futures
    import os
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    Lyr = case.wl.layers[layer]
    G = case.G
    fp8 = case.wcfg.kv_dtype == "fp8_e4m3"
    lengths = np.asarray(case.wl.lengths)
    if pairs is None:
        pairs = all_pairs(case)
    q = q64 if q64 is not None else oracle.attention.bf16_bits_to_f64(bits(Lyr.q))
    if fp8:
        kc, vc = Lyr.k_cache.cpu().numpy(), Lyr.v_cache.cpu().numpy()
        ks, vs = Lyr.k_scale.cpu().numpy(), Lyr.v_scale.cpu().numpy()
    else:
        kc, vc, ks, vs = bits(Lyr.k_cache), bits(Lyr.v_cache), None, None
    table = case.wl.page_table
    kv_dtype = case.wcfg.kv_dtype

    def one(pair):
        g, r = pair
        Lr = int(lengths[r])
        K = oracle.attention.gather_pair_kv(kc, table[r], g, Lr, kv_dtype, ks)
        V = oracle.attention.gather_pair_kv(vc, table[r], g, Lr, kv_dtype, vs)
        o, _ = oracle.attention.attend_range(q[r, g * G:(g + 1) * G], K, V, case.wcfg.sm_scale)
        return pair, o

    order = sorted(pairs, key=lambda p: -int(lengths[p[1]]))
    n = workers or min(16, len(os.sched_getaffinity(0)))
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        with concurrent.futures.ThreadPoolExecutor(n) as ex:
            res = dict(ex.map(one, order))
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    return {p: res[p] for p in pairs}


def sample_pairs(case: Case, k: int, seed: int = 0):
    """The longest and shortest requests of every KV head plus a seeded sample."""
    L = np.asarray(case.wl.lengths)
    H = case.wcfg.num_kv_heads
    rng = np.random.default_rng(seed)
    pairs = {(0, int(np.argmax(L))), (H - 1, int(np.argmin(L))), (H // 2, int(np.argmax(L)))}
    while len(pairs) < min(k, H * len(L)):
        pairs.add((int(rng.integers(H)), int(rng.integers(len(L)))))
    return sorted(pairs)


def all_pairs(case: Case):
    return [(g, r) for g in range(case.wcfg.num_kv_heads) for r in range(len(case.wl.lengths))]
