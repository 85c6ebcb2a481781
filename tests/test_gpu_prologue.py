"""GPU parity of the fused attention prologue (lbp_prologue) against the oracle.

The oracle (oracle/prologue.py) gives the exact normed and rotated values;
the kernel computes in fp32 and rounds once at the end, to BF16 or to e4m3
with a per-row scale.  Roundings are compared exactly, except for values
the exact result places within fp32 error of a rounding midpoint, where the
two neighbouring results are both correct: those must be rare and must be
one of the two neighbours.  Cache entries other than the new tokens' slots
must stay bit-for-bit unchanged.
"""

import dataclasses

import numpy as np
import pytest
import torch

import load_balanced_paged_amd as lbp
import oracle
from gpu_support import (all_pairs, bits, build_case, compare, compare_verify, oracle_pairs,
                         oracle_verify_pairs, say)
from workloads import CONFIGS, make_prologue_inputs, rope_cos_sin_table

pytestmark = pytest.mark.gpu

EPS = 1e-6
# fp32 evaluation error allowed around rounding midpoints: relative to the
# value plus absolute in units of the row's largest entry (RoPE can cancel
# two O(row max) terms into a small result)
REL_MID = 4e-6
ROW_MID = 1e-6


def row_max(exact):
    return np.max(np.abs(exact), axis=-1, keepdims=True) * np.ones_like(exact)


def check_bf16(got: np.ndarray, exact: np.ndarray, what: str):
    ref = oracle.prologue.bf16_round(exact)
    bad = got != ref
    if bad.any():
        mid = (got[bad] + ref[bad]) / 2
        tol = REL_MID * np.abs(exact[bad]) + ROW_MID * row_max(exact)[bad]
        ok = np.abs(exact[bad] - mid) <= tol
        assert ok.all(), (what, exact[bad][~ok][:4], got[bad][~ok][:4], ref[bad][~ok][:4])
        assert bad.mean() < 1e-3, (what, bad.mean())
    say(f"[prologue] {what}: {exact.size} values, {int(bad.sum())} at a midpoint")


def check_fp8(codes: np.ndarray, scale: np.ndarray, exact: np.ndarray, what: str):
    ref_codes, ref_scale, y = oracle.prologue.quantize_rows_e4m3(exact)
    assert np.allclose(scale, ref_scale, rtol=2e-6, atol=0), (what, np.max(np.abs(scale / ref_scale - 1)))
    bad = codes != ref_codes
    if bad.any():
        vg = oracle.e4m3.decode(codes[bad])
        vr = oracle.e4m3.decode(ref_codes[bad])
        mid = (vg + vr) / 2
        # y = x / scale spans +-448 per row
        tol = REL_MID * np.abs(y[bad]) + ROW_MID * 448.0
        ok = np.abs(y[bad] - mid) <= tol
        assert ok.all(), (what, y[bad][~ok][:4], vg[~ok][:4], vr[~ok][:4])
        assert bad.mean() < 1e-3, (what, bad.mean())
    say(f"[prologue] {what}: {exact.size} codes, {int(bad.sum())} at a midpoint")


def run_case(wcfg, lengths=None, q_fp8=None, seed=0, max_position=None, override=None,
             q_len=1, qkv_scale=1.0):
    """override: {request: length} applied to the device lengths after the plan
    (e.g. a length past the page table's capacity, which the plan would clamp).
    q_len: new tokens per request (token j of request r at position
    L_r - q_len + j); outputs keep the [B, q_len, ...] layout for q_len > 1.
    qkv_scale: a power of two applied to the projection (exact in BF16)."""
    T = q_len
    case = build_case(wcfg, lengths=lengths, poison=False, q_len=T)
    B = len(case.wl.lengths)
    L = np.asarray(case.wl.lengths).copy()
    for r, v in (override or {}).items():
        L[r] = v
    case.seq_lens.copy_(torch.from_numpy(L.astype(np.int32)))
    Hq, Hkv = wcfg.num_q_heads, wcfg.num_kv_heads
    fp8_kv = wcfg.kv_dtype == "fp8_e4m3"
    q_fp8 = fp8_kv if q_fp8 is None else q_fp8
    qkv, qw, kw = make_prologue_inputs(B * T, Hq, Hkv, seed, device="cuda")
    qkv = qkv * qkv_scale
    qkv = qkv.view(B, T, -1) if T > 1 else qkv
    maxpos = max_position or int(max(L.max(), 1))
    cs = rope_cos_sin_table(maxpos, device="cuda")
    lay = case.wl.layers[0]
    k0, v0 = lay.k_cache.clone(), lay.v_cache.clone()
    ks0 = lay.k_scale.clone() if fp8_kv else None
    vs0 = lay.v_scale.clone() if fp8_kv else None
    lead = (B, T) if T > 1 else (B,)
    q_out = torch.empty(lead + (Hq, 128), dtype=torch.uint8 if q_fp8 else torch.bfloat16,
                        device="cuda")
    q_scale = torch.empty(lead + (Hq,), dtype=torch.float32, device="cuda") if q_fp8 else None
    lbp.lbp_prologue(case.cfg, qkv, case.seq_lens, case.page_table, qw, kw, cs, q_out,
                     lay.k_cache, lay.v_cache, lay.k_scale, lay.v_scale, q_scale, EPS)
    torch.cuda.synchronize()
    ref = oracle.prologue.prologue(qkv.double().cpu().numpy(), L, Hq, Hkv,
                                   qw.double().cpu().numpy(), kw.double().cpu().numpy(), EPS,
                                   cs.double().cpu().numpy())
    has = ref["pos"] >= 0
    # query
    if q_fp8:
        check_fp8(q_out.cpu().numpy()[has], q_scale.cpu().numpy()[has], ref["q"][has], "q fp8")
    else:
        check_bf16(q_out.double().cpu().numpy()[has], ref["q"][has], "q bf16")
    # cache: the new tokens' slots, and nothing else
    cap = 64 * case.cfg.max_pages_per_seq
    table = case.page_table.cpu().numpy()
    changed = np.zeros(lay.k_cache.shape[:3], dtype=bool)
    pos = ref["pos"].reshape(B, T)
    rk = ref["k"].reshape(B, T, Hkv, 128)
    rv = ref["v"].reshape(B, T, Hkv, 128)
    rows_k, rows_v, gk = [], [], []
    for r in range(B):
        for j in range(T):
            p = int(pos[r, j])
            if p < 0 or p >= cap:
                continue
            page = int(table[r, p // 64])
            changed[page, :, p % 64] = True
            rows_k.append(rk[r, j])
            rows_v.append(rv[r, j])
            gk.append((page, p % 64))
    kc, vc = lay.k_cache.cpu(), lay.v_cache.cpu()
    conv = (lambda t: t.numpy()) if fp8_kv else (lambda t: t.double().numpy())
    if gk:
        got_k = np.stack([conv(kc[pg, :, sl]) for pg, sl in gk])
        got_v = np.stack([conv(vc[pg, :, sl]) for pg, sl in gk])
        ek, ev = np.stack(rows_k), np.stack(rows_v)
        if fp8_kv:
            ksc = np.stack([lay.k_scale[pg, :, sl].cpu().numpy() for pg, sl in gk])
            vsc = np.stack([lay.v_scale[pg, :, sl].cpu().numpy() for pg, sl in gk])
            check_fp8(got_k, ksc, ek, "k fp8")
            check_fp8(got_v, vsc, ev, "v fp8")
        else:
            check_bf16(got_k, ek, "k bf16")
            assert np.array_equal(got_v, ev)          # the value is copied exactly
    unchanged = ~changed
    assert torch.equal(lay.k_cache.view(torch.uint8)[torch.from_numpy(unchanged).cuda()],
                       k0.view(torch.uint8)[torch.from_numpy(unchanged).cuda()])
    assert torch.equal(lay.v_cache.view(torch.uint8)[torch.from_numpy(unchanged).cuda()],
                       v0.view(torch.uint8)[torch.from_numpy(unchanged).cuda()])
    if fp8_kv:
        m = torch.from_numpy(unchanged).cuda()
        assert torch.equal(lay.k_scale[m], ks0[m]) and torch.equal(lay.v_scale[m], vs0[m])
    return case, q_out, q_scale


@pytest.mark.parametrize("name", ["tiny", "mixed", "skewed"])
def test_prologue_bf16_cache(gpu_lib, name):
    run_case(CONFIGS[name], q_fp8=False)


def test_prologue_bf16_cache_fp8_query(gpu_lib):
    run_case(CONFIGS["mixed"], q_fp8=True, seed=1)


def test_prologue_fp8_cache(gpu_lib):
    run_case(CONFIGS["fp8"], seed=2)


@pytest.mark.parametrize("group,hkv", [(1, 4), (16, 1), (3, 3)])
def test_prologue_group_sizes(gpu_lib, group, hkv):
    wcfg = dataclasses.replace(CONFIGS["fp8"], name=f"pro-g{group}", batch=5,
                               num_q_heads=group * hkv, num_kv_heads=hkv)
    run_case(wcfg, lengths=[1, 64, 65, 700, 3000], seed=3)


def test_prologue_edges(gpu_lib):
    """No token (length 0), positions past the RoPE table, positions on page
    boundaries, and a position past the page table's capacity (no cache write)."""
    wcfg = dataclasses.replace(CONFIGS["tiny"], name="pro-edges", batch=6)
    case, _, _ = run_case(wcfg, lengths=[0, 1, 64, 129, 4000, 5000], max_position=100, seed=4,
                          override={5: 64 * 79 + 1})
    assert case.cfg.max_pages_per_seq == 79


def test_prologue_then_attention(gpu_lib):
    """The new token written by the prologue is seen by the attention: FP8 query
    and cache straight into lbp_attend_fp8q, checked against the oracle on the
    written cache and the emitted query."""
    wcfg = dataclasses.replace(CONFIGS["fp8"], name="pro-attend", batch=6)
    case, q_out, q_scale = run_case(wcfg, lengths=[1, 17, 64, 65, 700, 3000], seed=5)
    lay = case.wl.layers[0]
    out = torch.full((6, wcfg.num_q_heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lbp.lbp_attend_fp8q(case.cfg, case.info, case.plan_ws, q_out, q_scale, lay.k_cache,
                        lay.v_cache, lay.k_scale, lay.v_scale, case.split_ws, out)
    torch.cuda.synchronize()
    q64 = oracle.e4m3.dequantize(q_out.cpu().numpy(), q_scale.cpu().numpy())
    compare(case, out, oracle_pairs(case, 0, all_pairs(case), q64), "prologue + attention")


@pytest.mark.parametrize("T,fp8", [(3, False), (6, True)])
def test_prologue_multi_token(gpu_lib, T, fp8):
    """q_len new tokens per request (speculative verification): every token's
    query, K and V, including requests shorter than q_len (tokens before the
    sequence start write nothing) and tokens that straddle a page boundary."""
    base = CONFIGS["fp8"] if fp8 else CONFIGS["tiny"]
    wcfg = dataclasses.replace(base, name=f"pro-t{T}", batch=6)
    run_case(wcfg, lengths=[1, 2, 65, 66, 700, 3000], seed=6 + T, q_len=T)


def test_prologue_then_verify(gpu_lib):
    """Prologue for four new tokens, then verification attention over the cache
    it wrote, against the oracle on that cache and query.  The projection is
    halved so that V has the unit spread of the attention workloads, whose
    absolute tolerance this comparison uses."""
    wcfg = dataclasses.replace(CONFIGS["tiny"], name="pro-verify", batch=5)
    T = 4
    case, q_out, _ = run_case(wcfg, lengths=[2, 64, 67, 700, 3000], seed=11, q_len=T,
                              qkv_scale=0.5)
    lay = case.wl.layers[0]
    out = torch.full_like(q_out, float("nan"))
    lbp.lbp_attend(case.cfg, case.info, case.plan_ws, q_out, lay.k_cache, lay.v_cache, None,
                   None, case.split_ws, out)
    torch.cuda.synchronize()
    q64 = oracle.attention.bf16_bits_to_f64(bits(q_out))
    compare_verify(case, out, oracle_verify_pairs(case, 0, all_pairs(case), q64),
                   "prologue + verification")
