"""lbp_attend_noalloc: lbp_attend with the split buffer in the library's
fixed device array, for callers that cannot allocate.

Two calls in a row on one GPU, the second with a smaller input, each against
lbp_attend on the same inputs (bit for bit: same kernels, same arithmetic)
and against the oracle; and the size limit, rejected before any launch.
"""

import dataclasses

import pytest
import torch

import load_balanced_paged_amd as lbp
from gpu_support import all_pairs, build_case, compare, oracle_pairs, say
from workloads import CONFIGS

pytestmark = pytest.mark.gpu


def _noalloc(case, layer=0):
    lay = case.wl.layers[layer]
    out = torch.full_like(lay.q, float("nan"))
    lbp.lbp_attend_noalloc(case.cfg, case.info, case.plan_ws, lay.q, lay.k_cache, lay.v_cache,
                           lay.k_scale, lay.v_scale, out)
    torch.cuda.synchronize()
    return out


def _two_launch(case, layer=0):
    lay = case.wl.layers[layer]
    out = torch.full_like(lay.q, float("nan"))
    lbp.lbp_attend(case.cfg, case.info, case.plan_ws, lay.q, lay.k_cache, lay.v_cache,
                   lay.k_scale, lay.v_scale, case.split_ws, out)
    torch.cuda.synchronize()
    return out


def test_noalloc_two_calls_match_attend(gpu_lib):
    """The skewed workload (a 205-way split pair and short ones), then a
    smaller FP8 batch on the same array: each equals lbp_attend bit for bit
    and the oracle within tolerance."""
    big = build_case(CONFIGS["skewed"])
    got = _noalloc(big)
    assert torch.equal(got.view(torch.int16), _two_launch(big).view(torch.int16))
    compare(big, got, oracle_pairs(big, 0, all_pairs(big)), "noalloc skewed")

    wcfg = dataclasses.replace(CONFIGS["fp8"], name="noalloc-small", batch=5)
    small = build_case(wcfg, lengths=[3000, 17, 700, 64, 1], num_workgroups=9, min_tiles=1)
    got2 = _noalloc(small)
    assert torch.equal(got2.view(torch.int16), _two_launch(small).view(torch.int16))
    compare(small, got2, oracle_pairs(small, 0, all_pairs(small)), "noalloc fp8 small")
    # the first call's output is untouched by the second
    assert torch.equal(got.view(torch.int16), _two_launch(big).view(torch.int16))


def test_noalloc_rejects_a_plan_beyond_the_array(gpu_lib):
    """A plan whose split buffer exceeds the fixed array is refused with
    LBP_ERR_SCRATCH_LIMIT and launches nothing (the output keeps its NaN)."""
    wcfg = dataclasses.replace(CONFIGS["tiny"], name="noalloc-limit", batch=4)
    # 64 query columns x (4 pairs + 2047 bins) slots of 64 x 516 B > 32 MiB
    case = build_case(dataclasses.replace(wcfg, num_q_heads=16), lengths=[64, 128, 1000, 5],
                      num_workgroups=2048, min_tiles=1, q_len=4)
    need = lbp.lbp_query_workspace(case.cfg)[1]
    assert need > lbp.NOALLOC_SCRATCH_BYTES, need
    lay = case.wl.layers[0]
    q = torch.zeros((4, 4, 16, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, float("nan"))
    with pytest.raises(lbp.LbpError) as e:
        lbp.lbp_attend_noalloc(case.cfg, case.info, case.plan_ws, q, lay.k_cache, lay.v_cache,
                               None, None, out)
    assert e.value.status == lbp.LBP_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    say(f"[noalloc] split buffer of {need} B refused (limit {lbp.NOALLOC_SCRATCH_BYTES} B)")
