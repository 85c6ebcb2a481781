"""GPU parity of the attention path (persistent kernel + combine) against the oracle.

Tolerances: BF16 KV max-abs <= 1e-2 and relative RMS <= 5e-3; FP8 KV max-abs
<= 3e-2.  Unused slots of every request's last page hold NaN.
"""

import dataclasses

import numpy as np
import pytest
import torch

import load_balanced_paged_amd as lbp
import oracle
from gpu_support import (all_pairs, assert_taskmap_matches, bf16_to_f64, bits, build_case,
                         compare, oracle_layer, oracle_pairs, run_attend, say)
from workloads import CONFIGS, quantize_query_e4m3

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "uniform", "skewed"])
def test_attend_full_parity(gpu_lib, name):
    """Every output row against the oracle (these three fit the oracle in seconds)."""
    case = build_case(CONFIGS[name])
    assert_taskmap_matches(case)
    out = run_attend(case)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case)), name)


def test_attend_mixed_eight_layers(gpu_lib):
    """One task map reused by 8 layers with different KV: every pair of every
    layer against the oracle (the relative RMS over each whole output
    tensor), one layer at a time so that the host holds one layer's caches."""
    case = build_case(CONFIGS["mixed"], layers=8)
    assert_taskmap_matches(case)
    outs = [run_attend(case, layer) for layer in range(8)]
    for layer in range(8):
        compare(case, outs[layer], oracle_layer(case, layer), f"mixed layer {layer} all pairs")
    assert not torch.equal(outs[0], outs[7])


def test_attend_fp8_parity(gpu_lib):
    """Every (KV head, request) pair of the FP8 workload (1024 pairs, up to
    262144 tokens): whole-tensor relative RMS and the per-pair bound, which
    a lost or zeroed long row cannot pass."""
    case = build_case(CONFIGS["fp8"])
    assert_taskmap_matches(case)
    out = run_attend(case)
    compare(case, out, oracle_layer(case, 0), "fp8 all pairs")


def test_attend_fp8_small_full(gpu_lib):
    """FP8 KV on a small ragged batch, every row."""
    wcfg = dataclasses.replace(CONFIGS["fp8"], name="fp8-small", batch=6)
    case = build_case(wcfg, lengths=[1, 17, 64, 65, 700, 3000])
    out = run_attend(case)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case)), "fp8-small")


@pytest.mark.parametrize("group,hkv", [(1, 4), (4, 2), (16, 1), (3, 3)])
def test_attend_group_sizes(gpu_lib, group, hkv):
    wcfg = dataclasses.replace(CONFIGS["tiny"], name=f"g{group}", batch=5,
                               num_q_heads=group * hkv, num_kv_heads=hkv)
    case = build_case(wcfg, lengths=[33, 1, 128, 129, 900], num_workgroups=7, min_tiles=1)
    out = run_attend(case)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case)), f"group {group} hkv {hkv}")


def test_attend_length_one_is_exact(gpu_lib):
    """With one token the softmax weight is exactly 1, so out == v_0 bit for bit."""
    wcfg = dataclasses.replace(CONFIGS["tiny"], name="len1", batch=3)
    case = build_case(wcfg, lengths=[1, 1, 1])
    out = run_attend(case)
    lay = case.wl.layers[0]
    for r in range(3):
        page = int(case.wl.page_table[r, 0])
        v0 = lay.v_cache[page, 0, 0]
        assert torch.equal(out[r], v0.expand(8, -1)), r


def test_attend_zero_length_requests(gpu_lib):
    wcfg = dataclasses.replace(CONFIGS["tiny"], name="zeros", batch=4)
    case = build_case(wcfg, lengths=[0, 300, 0, 5], num_workgroups=3, min_tiles=1)
    assert_taskmap_matches(case)
    out = run_attend(case)
    assert torch.all(out[0] == 0) and torch.all(out[2] == 0)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case)), "zero-length")


@pytest.mark.parametrize("kv,q_len,entry", [("bf16", 1, "attend"), ("bf16", 1, "fused"),
                                             ("bf16", 3, "attend"), ("bf16", 6, "fused"),
                                             ("fp8_e4m3", 1, "attend"), ("fp8_e4m3", 1, "fp8q")])
def test_all_requests_empty(gpu_lib, kv, q_len, entry):
    """Every length zero (T = 0: no tile, no descriptor, every bin empty):
    every output row is exactly zero, and nothing is read from a KV cache
    (and scales) holding only NaN."""
    base = CONFIGS["tiny"] if kv == "bf16" else CONFIGS["fp8"]
    wcfg = dataclasses.replace(base, name=f"empty-{kv}", batch=3)
    case = build_case(wcfg, lengths=[0, 0, 0], max_pages_per_seq=1, q_len=q_len, poison=False)
    assert_taskmap_matches(case)
    lay = case.wl.layers[0]
    H, D = wcfg.num_kv_heads, 128
    if kv == "bf16":
        kc = torch.full((1, H, 64, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        vc, ks, vs = kc.clone(), None, None
    else:
        kc = torch.full((1, H, 64, D), 0x7F, dtype=torch.uint8, device="cuda")   # e4m3 NaN
        vc = kc.clone()
        ks = torch.full((1, H, 64), float("nan"), dtype=torch.float32, device="cuda")
        vs = ks.clone()
    q = torch.randn((3, q_len, wcfg.num_q_heads, D), device="cuda").to(torch.bfloat16)
    if q_len == 1:
        q = q[:, 0].contiguous()
    out = torch.full_like(q, float("nan"))
    if entry == "fp8q":
        codes, scale = quantize_query_e4m3(q)
        lbp.lbp_attend_fp8q(case.cfg, case.info, case.plan_ws, codes, scale, kc, vc, ks, vs,
                            case.split_ws, out)
    else:
        fn = lbp.lbp_attend if entry == "attend" else lbp.lbp_attend_fused
        fn(case.cfg, case.info, case.plan_ws, q, kc, vc, ks, vs, case.split_ws, out)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out)), f"{kv} q_len={q_len} {entry}"


@pytest.mark.parametrize("W,F", [(1, 1), (5, 1), (64, 1), (256, 4), (1024, 1)])
def test_attend_bin_shapes(gpu_lib, W, F):
    """Many splits per pair, one bin for everything, more bins than tiles."""
    case = build_case(CONFIGS["tiny"], num_workgroups=W, min_tiles=F)
    assert_taskmap_matches(case)
    out = run_attend(case)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case)), f"tiny W={W} F={F}")


@pytest.mark.parametrize("form,batch,W,group", [("wide", 1, 600, 8), ("pairs", 40, 400, 8),
                                                ("pairs", 40, 400, 16), ("columns", 20, 400, 16)])
def test_combine_rounds_every_form(gpu_lib, form, batch, W, group):
    """A pair split into more partials than one round of the combine's loads
    takes, through each combine form.  With a split-list capacity of cap
    entries: one workgroup per pair and chunk of 8 columns when
    cap x min(columns, 8) > 256 (300 partials, 8 per round per thread; one
    and two column chunks); else 512 threads per column when the
    (entries x columns) grid has at most 256 workgroups (600 partials, 256
    rows per round); else 256 threads per column (300 partials, 128 rows per
    round)."""
    n_long = 600 if batch == 1 else 300
    wcfg = dataclasses.replace(CONFIGS["skewed"], name=f"rounds-{form}", batch=batch,
                               num_q_heads=group)
    case = build_case(wcfg, lengths=[64 * n_long] + [64] * (batch - 1), num_workgroups=W,
                      min_tiles=1)
    assert_taskmap_matches(case)
    tm = lbp.read_taskmap(case.plan_ws, case.info)
    assert int(tm["pair_count"].max()) == n_long
    cap = min(batch, W - 1)
    expected = ("pairs" if cap * min(group, 8) > 256 else
                "wide" if cap * group <= 256 else "columns")
    assert expected == form
    out = run_attend(case)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case)), f"combine {form}")


@pytest.mark.parametrize("policy,param", [(lbp.LBP_POLICY_STATIC_SPLITS, 1),
                                          (lbp.LBP_POLICY_STATIC_SPLITS, 7),
                                          (lbp.LBP_POLICY_STATIC_CHUNK, 2)])
def test_attend_static_plans(gpu_lib, policy, param):
    case = build_case(CONFIGS["skewed"], policy=policy, param=param)
    assert_taskmap_matches(case)
    out = run_attend(case)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case)), f"skewed static {policy}/{param}")


def test_attend_deterministic(gpu_lib):
    case = build_case(CONFIGS["skewed"])
    a = run_attend(case).clone()
    b = run_attend(case).clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_partials_match_oracle_ranges(gpu_lib):
    """Split-buffer contents per descriptor of every split pair against the
    oracle's per-range attention; single-descriptor pairs are finished in place."""
    case = build_case(CONFIGS["tiny"], num_workgroups=5, min_tiles=1)
    lay = case.wl.layers[0]
    out = torch.zeros_like(lay.q)
    lbp.lbp_attend_partials(case.cfg, case.info, case.plan_ws, lay.q, lay.k_cache, lay.v_cache,
                            None, None, case.split_ws, out)
    torch.cuda.synchronize()
    tm = lbp.read_taskmap(case.plan_ws, case.info)
    assert sorted(tm["pair_count"]) == [1, 1, 2, 4]
    o_part, lse_part = lbp.split_views(case.split_ws, case.info, case.G)
    o_part = o_part.cpu().numpy()
    lse_part = lse_part.cpu().numpy()
    q = oracle.attention.bf16_bits_to_f64(bits(lay.q))
    kc, vc = bits(lay.k_cache), bits(lay.v_cache)
    got_out = bf16_to_f64(out)
    for d, (g, r, a, e) in enumerate(tm["desc"]):
        K = oracle.attention.gather_pair_kv(kc, case.wl.page_table[r], g, e)[a:e]
        V = oracle.attention.gather_pair_kv(vc, case.wl.page_table[r], g, e)[a:e]
        o, lse = oracle.attention.attend_range(q[r, g * 8:(g + 1) * 8], K, V, case.wcfg.sm_scale)
        if tm["pair_count"][g * 4 + r] == 1:
            assert np.max(np.abs(got_out[r, g * 8:(g + 1) * 8] - o)) < 1e-2, d
            continue
        assert np.max(np.abs(o_part[d] - o)) < 1e-2, d
        # the split buffer keeps base-2 log-sum-exp of log2(e)-scaled scores
        assert np.max(np.abs(lse_part[d] * np.log(2.0) - lse)) < 1e-3, d


def test_traced_run_records_every_workgroup(gpu_lib):
    """The traced entry point gives the same output plus one record per workgroup."""
    case = build_case(CONFIGS["skewed"])
    lay = case.wl.layers[0]
    ref = run_attend(case).clone()
    out = torch.zeros_like(lay.q)
    trace = torch.zeros(4 * case.info.num_bins, dtype=torch.int64, device="cuda")
    lbp.lbp_attend_traced(case.cfg, case.info, case.plan_ws, lay.q, lay.k_cache, lay.v_cache,
                          None, None, case.split_ws, out, trace)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    t = trace.view(-1, 4).cpu().numpy()
    tm = lbp.read_taskmap(case.plan_ws, case.info)
    assert np.all(t[:, 1] >= t[:, 0]) and np.all(t[:, 0] > 0)
    assert np.array_equal(t[:, 3], np.diff(tm["bin_offset"]))
    # MI355X has 8 XCDs; 256 workgroups (one per CU) land on more than one
    xcc = set((t[:, 2] >> 32).tolist())
    assert xcc <= set(range(8)), xcc
    assert case.info.num_bins < 8 or len(xcc) > 1, xcc


def test_workspace_reuse_across_batches(gpu_lib):
    """A workspace sized for max_batch serves a smaller batch's plan."""
    wcfg = dataclasses.replace(CONFIGS["tiny"], name="smallbatch", batch=2)
    case = build_case(wcfg, lengths=[500, 70])
    out = run_attend(case)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case)), "small batch")


def test_graph_replay_matches_eager(gpu_lib):
    """lbp_plan + lbp_attend captured into a HIP graph: every replay equals eager."""
    case = build_case(CONFIGS["skewed"], layers=2)
    eager = [run_attend(case, i).clone() for i in range(2)]
    outs = [torch.zeros_like(e) for e in eager]
    lay = case.wl.layers
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            lbp.lbp_plan(case.cfg, case.seq_lens, case.page_table, case.plan_ws, stream=s)
            for i in range(2):
                lbp.lbp_attend(case.cfg, case.info, case.plan_ws, lay[i].q, lay[i].k_cache,
                               lay[i].v_cache, None, None, case.split_ws, outs[i], stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        for o in outs:
            o.zero_()
        run_attend(case, 1 - rep % 2)          # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i].view(torch.int16), eager[i].view(torch.int16)), (rep, i)
