"""GPU parity of lbp_attend_fp8q: FP8 (e4m3) queries with per-(request, head)
scales over the FP8 KV cache.

The oracle attends with the exact values of the FP8 query, e4m3(code) *
scale in fp64, so the tolerance is the FP8-KV one (max-abs <= 3e-2).
"""

import dataclasses

import numpy as np
import pytest
import torch

import load_balanced_paged_amd as lbp
import oracle
from gpu_support import all_pairs, build_case, compare, oracle_layer, oracle_pairs, say
from workloads import CONFIGS, TABLE3, quantize_query_e4m3

pytestmark = pytest.mark.gpu


def run_fp8q(case, layer=0):
    lay = case.wl.layers[layer]
    codes, scale = quantize_query_e4m3(lay.q)
    out = torch.full_like(lay.q, float("nan"))
    lbp.lbp_attend_fp8q(case.cfg, case.info, case.plan_ws, codes, scale, lay.k_cache,
                        lay.v_cache, lay.k_scale, lay.v_scale, case.split_ws, out)
    torch.cuda.synchronize()
    q64 = oracle.e4m3.dequantize(codes.cpu().numpy(), scale.cpu().numpy())
    return out, q64


def test_fp8q_fp8_workload_all_pairs(gpu_lib):
    """Every pair of the FP8 workload with the FP8 query."""
    case = build_case(CONFIGS["fp8"])
    out, q64 = run_fp8q(case)
    compare(case, out, oracle_layer(case, 0, q64=q64), "fp8q fp8 all pairs")


def test_fp8q_small_ragged_all_rows(gpu_lib):
    wcfg = dataclasses.replace(CONFIGS["fp8"], name="fp8q-small", batch=6)
    case = build_case(wcfg, lengths=[1, 17, 64, 65, 700, 3000], num_workgroups=7, min_tiles=1)
    out, q64 = run_fp8q(case)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case), q64), "fp8q small")


@pytest.mark.parametrize("mix", ["64x0.5K", "1x128K+31x4K"])
def test_fp8q_table3_all_rows(gpu_lib, mix):
    case = build_case(TABLE3[mix])
    out, q64 = run_fp8q(case)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case), q64), f"fp8q {mix}")


@pytest.mark.parametrize("group,hkv", [(1, 4), (3, 3), (16, 1)])
def test_fp8q_group_sizes(gpu_lib, group, hkv):
    wcfg = dataclasses.replace(CONFIGS["fp8"], name=f"fp8q-g{group}", batch=4,
                               num_q_heads=group * hkv, num_kv_heads=hkv)
    case = build_case(wcfg, lengths=[33, 1, 900, 129], num_workgroups=9, min_tiles=1)
    out, q64 = run_fp8q(case)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case), q64), f"fp8q group {group}")


def test_fp8q_zero_query_row_is_mean_of_v(gpu_lib):
    """A zero query gets scale 1 and zero codes: every score is 0."""
    wcfg = dataclasses.replace(CONFIGS["fp8"], name="fp8q-zero", batch=2)
    case = build_case(wcfg, lengths=[100, 64])
    case.wl.layers[0].q[0].zero_()
    out, q64 = run_fp8q(case)
    assert np.all(q64[0] == 0)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case), q64), "fp8q zero row")


def test_fp8q_matches_bf16_query_closely(gpu_lib):
    """Quantizing Q to e4m3 moves the output by far less than the tolerance."""
    wcfg = dataclasses.replace(CONFIGS["fp8"], name="fp8q-vs-bf16", batch=4)
    case = build_case(wcfg, lengths=[5000, 300, 64, 2000])
    lay = case.wl.layers[0]
    ref = torch.empty_like(lay.q)
    lbp.lbp_attend(case.cfg, case.info, case.plan_ws, lay.q, lay.k_cache, lay.v_cache,
                   lay.k_scale, lay.v_scale, case.split_ws, ref)
    out, _ = run_fp8q(case)
    d = (out.float() - ref.float()).abs().max().item()
    say(f"[fp8q] max |fp8 q - bf16 q| = {d:.3e}")
    assert d < 3e-2
