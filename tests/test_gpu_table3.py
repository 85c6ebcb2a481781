"""GPU parity on the six FP8-KV length mixes of the vLLM x HPC-Ops page, Table 3.

Each mix runs at 8 query heads / 1 KV head (one GPU's tensor-parallel share
of the Hy3 shape) with e4m3 KV and fp32 per-token scales.  Every mix has at
most 64 (KV head, request) pairs, so every output row is checked against the
fp64 oracle (max-abs <= 3e-2), for the dynamic plan through both attend
entry points and for the static fixed-split plan the benchmark compares it
with.  Task maps are compared bit-exactly.
"""

import math

import pytest
import torch

import load_balanced_paged_amd as lbp
from gpu_support import all_pairs, assert_taskmap_matches, build_case, compare, oracle_pairs, say
from workloads import TABLE3

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("F", [0, 4])
@pytest.mark.parametrize("mix", list(TABLE3))
def test_table3_mix_dynamic(gpu_lib, mix, F):
    """The benchmark's plan (the library's default floor, F = 0 in the
    config: no floor) and the plan with F = 4, which binds on 64x0.5K."""
    case = build_case(TABLE3[mix], min_tiles=F)
    got, ref = assert_taskmap_matches(case)
    say(f"[table3] {mix} F={F}: T={ref.T} budget={ref.budget} D={ref.D} U={ref.U} "
        f"max splits={int(ref.pair_count.max())}")
    ref_rows = oracle_pairs(case, 0, all_pairs(case))
    lay = case.wl.layers[0]
    out = torch.full_like(lay.q, float("nan"))
    lbp.lbp_attend(case.cfg, case.info, case.plan_ws, lay.q, lay.k_cache, lay.v_cache,
                   lay.k_scale, lay.v_scale, case.split_ws, out)
    torch.cuda.synchronize()
    compare(case, out, ref_rows, f"table3 {mix}")
    fused = torch.full_like(lay.q, float("nan"))
    lbp.lbp_attend_fused(case.cfg, case.info, case.plan_ws, lay.q, lay.k_cache, lay.v_cache,
                         lay.k_scale, lay.v_scale, case.split_ws, fused)
    torch.cuda.synchronize()
    compare(case, fused, ref_rows, f"table3 {mix} fused")


@pytest.mark.parametrize("mix", ["64x4K", "1x128K+31x4K"])
def test_table3_mix_static_grid_matched(gpu_lib, mix):
    """The static comparison at the split count that fills one wave of workgroups."""
    wcfg = TABLE3[mix]
    S = max(1, math.ceil(256 / (wcfg.num_kv_heads * wcfg.batch)))
    case = build_case(wcfg, policy=lbp.LBP_POLICY_STATIC_SPLITS, param=S)
    assert_taskmap_matches(case)
    lay = case.wl.layers[0]
    out = torch.full_like(lay.q, float("nan"))
    lbp.lbp_attend(case.cfg, case.info, case.plan_ws, lay.q, lay.k_cache, lay.v_cache,
                   lay.k_scale, lay.v_scale, case.split_ws, out)
    torch.cuda.synchronize()
    compare(case, out, oracle_pairs(case, 0, all_pairs(case)), f"table3 {mix} static S={S}")
