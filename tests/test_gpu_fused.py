"""GPU checks of lbp_attend_fused, the merge of split pairs inside the attention kernel.

On a dynamic plan it is one launch: the workgroup that completes a split
pair merges its partials (one level up to 16 partials, two levels above).
These tests compare that path with the oracle and with the two-launch path
(lbp_attend) on the same inputs, cover both merge levels with and without the
bin ticket queue, check that the arrival counters are back at zero after
every launch, and replay it from a HIP graph.
"""

import dataclasses

import numpy as np
import pytest
import torch

import load_balanced_paged_amd as lbp
from gpu_support import (all_pairs, assert_taskmap_matches, bf16_to_f64, build_case, compare,
                         oracle_layer, oracle_pairs, run_attend, sample_pairs, say)
from workloads import CONFIGS

pytestmark = pytest.mark.gpu


def fused(case, layer=0):
    lay = case.wl.layers[layer]
    out = torch.full_like(lay.q, float("nan"))
    lbp.lbp_attend_fused(case.cfg, case.info, case.plan_ws, lay.q, lay.k_cache, lay.v_cache,
                         lay.k_scale, lay.v_scale, case.split_ws, out)
    torch.cuda.synchronize()
    return out


def assert_counters_zero(case):
    tm = lbp.read_taskmap(case.plan_ws, case.info)
    assert len(tm["arrive"]) == 2 * case.info.max_desc
    assert not np.any(tm["arrive"]), np.nonzero(tm["arrive"])


def assert_close_to_two_launch(a, b):
    """Both paths round the same merge (in another association) to BF16: at
    most one BF16 step apart in every element."""
    x, y = bf16_to_f64(a), bf16_to_f64(b)
    assert np.all(np.isfinite(x)) and np.all(np.isfinite(y))
    tol = np.abs(y) * 2.0 ** -7 + 1e-6
    bad = np.abs(x - y) > tol
    assert not bad.any(), (np.argwhere(bad)[:5], x[bad][:5], y[bad][:5])


def max_pair_count(case):
    return int(lbp.read_taskmap(case.plan_ws, case.info)["pair_count"].max())


@pytest.mark.parametrize("W,F", [(5, 1), (64, 1), (1024, 1)])
def test_fused_tiny_all_rows(gpu_lib, W, F):
    case = build_case(CONFIGS["tiny"], num_workgroups=W, min_tiles=F)
    assert_taskmap_matches(case)
    got = fused(case)
    compare(case, got, oracle_pairs(case, 0, all_pairs(case)), f"fused tiny W={W}")
    assert_close_to_two_launch(got, run_attend(case))
    assert_counters_zero(case)


def test_fused_skewed_two_levels(gpu_lib):
    """The long request is split over about 205 bins: groups of 16, then 13 groups."""
    case = build_case(CONFIGS["skewed"])
    assert max_pair_count(case) > 16
    got = fused(case)
    compare(case, got, oracle_pairs(case, 0, all_pairs(case)), "fused skewed")
    assert_close_to_two_launch(got, run_attend(case))
    assert_counters_zero(case)


def test_fused_more_than_256_partials(gpu_lib):
    """313 partials (groups of 18) and 79 partials (groups of 16) with one tile
    per bin and more bins than CUs, so bins also come from the ticket queue."""
    wcfg = dataclasses.replace(CONFIGS["tiny"], name="long-split", batch=3)
    case = build_case(wcfg, lengths=[20000, 100, 5000], num_workgroups=1024, min_tiles=1)
    tm = lbp.read_taskmap(case.plan_ws, case.info)
    assert sorted(tm["pair_count"].tolist()) == [2, 79, 313]
    got = fused(case)
    compare(case, got, oracle_pairs(case, 0, all_pairs(case)), "fused 313 partials")
    assert_close_to_two_launch(got, run_attend(case))
    assert_counters_zero(case)


@pytest.mark.parametrize("group,hkv", [(1, 4), (16, 1), (3, 3)])
def test_fused_group_sizes(gpu_lib, group, hkv):
    """The merge's thread layout depends on the group size (rows per pass)."""
    wcfg = dataclasses.replace(CONFIGS["tiny"], name=f"fg{group}", batch=4,
                               num_q_heads=group * hkv, num_kv_heads=hkv)
    case = build_case(wcfg, lengths=[3000, 1, 129, 1500], num_workgroups=200, min_tiles=1)
    assert max_pair_count(case) > 16
    got = fused(case)
    compare(case, got, oracle_pairs(case, 0, all_pairs(case)), f"fused group {group}")
    assert_close_to_two_launch(got, run_attend(case))
    assert_counters_zero(case)


def test_fused_mixed_layers_and_fp8(gpu_lib):
    """Eight launches on one plan keep the counters consistent; FP8 KV too."""
    case = build_case(CONFIGS["mixed"], layers=2)
    pairs = sample_pairs(case, 10)
    for layer in range(2):
        for _ in range(3):
            got = fused(case, layer)
        ref = oracle_layer(case, layer, None if layer == 0 else pairs)
        compare(case, got, ref, f"fused mixed layer {layer}")
        assert_close_to_two_launch(got, run_attend(case, layer))
    assert_counters_zero(case)
    wcfg = dataclasses.replace(CONFIGS["fp8"], name="fp8-fused", batch=5)
    case = build_case(wcfg, lengths=[40000, 17, 700, 3000, 65], num_workgroups=256)
    assert max_pair_count(case) > 16
    got = fused(case)
    compare(case, got, oracle_pairs(case, 0, all_pairs(case)), "fused fp8")
    assert_close_to_two_launch(got, run_attend(case))
    assert_counters_zero(case)


def test_fused_is_deterministic(gpu_lib):
    case = build_case(CONFIGS["skewed"])
    a = fused(case).clone()
    b = fused(case).clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fused_static_plan_runs_two_launches(gpu_lib):
    case = build_case(CONFIGS["skewed"], policy=lbp.LBP_POLICY_STATIC_SPLITS, param=7)
    got = fused(case)
    assert torch.equal(got.view(torch.int16), run_attend(case).view(torch.int16))


def test_fused_graph_replay_matches_eager(gpu_lib):
    """Plan + two fused layers captured in a HIP graph: every replay equals eager,
    so the counters return to zero inside the graph too."""
    case = build_case(CONFIGS["skewed"], layers=2)
    eager = [fused(case, i).clone() for i in range(2)]
    outs = [torch.zeros_like(e) for e in eager]
    lay = case.wl.layers
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            lbp.lbp_plan(case.cfg, case.seq_lens, case.page_table, case.plan_ws, stream=s)
            for i in range(2):
                lbp.lbp_attend_fused(case.cfg, case.info, case.plan_ws, lay[i].q, lay[i].k_cache,
                                     lay[i].v_cache, None, None, case.split_ws, outs[i], stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        for o in outs:
            o.zero_()
        fused(case, 1 - rep % 2)          # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i].view(torch.int16), eager[i].view(torch.int16)), (rep, i)
    assert_counters_zero(case)
