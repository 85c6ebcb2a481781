"""GPU parity of bins holding many short descriptors.

Where short requests pile up, one bin holds many descriptors of one or two
64-token tiles.  In decode, lbp_attend and lbp_attend_fp8q drain such a bin
(at least three descriptors averaging at most two tiles) one descriptor per
wave and write each result from the wave's registers; other bins of the
same launch, and every bin of the single-launch form, go through the
per-descriptor loop with its merge across waves.  These cases
make such bins, up to about twenty descriptors each (more than the waves),
with pairs finished in place and pairs split across bins, in every KV
format and entry point, and check every output row against the oracle.
"""

import dataclasses

import numpy as np
import pytest
import torch

import load_balanced_paged_amd as lbp
import oracle
from gpu_support import all_pairs, assert_taskmap_matches, build_case, compare, oracle_pairs, say
from workloads import CONFIGS, quantize_query_e4m3

pytestmark = pytest.mark.gpu


def short_bins(case):
    """(bins of at least three descriptors averaging at most two tiles, how
    many of their descriptors belong to split pairs) from the oracle-checked
    task map."""
    got, ref = assert_taskmap_matches(case)
    budget = got["header"][1]
    nd = np.diff(ref.bin_offset)
    bins = np.flatnonzero((nd >= 3) & (budget <= 2 * nd))
    split = 0
    for b in bins:
        for d in range(ref.bin_offset[b], ref.bin_offset[b + 1]):
            g, r = ref.desc[d][0], ref.desc[d][1]
            split += int(ref.pair_count[g * case.wcfg.batch + r] >= 2)
    return len(bins), split


def run(case, entry):
    lay = case.wl.layers[0]
    out = torch.full_like(lay.q, float("nan"))
    q64 = None
    if entry == "fp8q":
        codes, scale = quantize_query_e4m3(lay.q)
        lbp.lbp_attend_fp8q(case.cfg, case.info, case.plan_ws, codes, scale, lay.k_cache,
                            lay.v_cache, lay.k_scale, lay.v_scale, case.split_ws, out)
        q64 = oracle.e4m3.dequantize(codes.cpu().numpy(), scale.cpu().numpy())
    else:
        fn = lbp.lbp_attend if entry == "attend" else lbp.lbp_attend_fused
        fn(case.cfg, case.info, case.plan_ws, lay.q, lay.k_cache, lay.v_cache, lay.k_scale,
           lay.v_scale, case.split_ws, out)
    torch.cuda.synchronize()
    return out, q64


def short_lengths(batch, hi, seed):
    """Ragged short lengths in [1, hi], with the slice and tile edges."""
    rng = np.random.default_rng(seed)
    L = rng.integers(1, hi + 1, size=batch)
    edges = [1, 15, 16, 17, 63, 64, 65, 128][: batch // 4]
    L[: len(edges)] = [min(e, hi) for e in edges]
    return [int(x) for x in L]


# (name, KV format, entry, query heads, KV heads, batch, longest length, W,
# seed of the lengths): the "W=4" bins hold about twenty descriptors of one
# or two tiles each, more than the waves
CASES = [
    ("bf16 attend", "bf16", "attend", 16, 2, 48, 160, 24, 1),
    ("bf16 fused", "bf16", "fused", 16, 2, 48, 160, 24, 2),
    ("bf16 attend W=4", "bf16", "attend", 16, 2, 40, 96, 4, 4),
    ("bf16 fused W=4", "bf16", "fused", 16, 2, 40, 96, 4, 7),
    ("bf16 group 3", "bf16", "attend", 9, 3, 30, 128, 16, 9),
    ("bf16 group 16", "bf16", "fused", 16, 1, 60, 128, 12, 4),
    ("bf16 group 16 attend", "bf16", "attend", 16, 1, 60, 128, 12, 5),
    ("bf16 group 1", "bf16", "attend", 4, 4, 24, 128, 16, 1),
    ("fp8 attend", "fp8_e4m3", "attend", 16, 2, 48, 160, 24, 5),
    ("fp8 fused W=4", "fp8_e4m3", "fused", 16, 2, 40, 96, 4, 8),
    ("fp8 fp8q", "fp8_e4m3", "fp8q", 16, 2, 48, 160, 24, 6),
    ("fp8 fp8q W=4", "fp8_e4m3", "fp8q", 16, 2, 40, 96, 4, 11),
]


@pytest.mark.parametrize("name,kv,entry,hq,hkv,batch,hi,W,seed", CASES, ids=[c[0] for c in CASES])
def test_short_descriptor_bins(gpu_lib, name, kv, entry, hq, hkv, batch, hi, W, seed):
    base = CONFIGS["tiny"] if kv == "bf16" else CONFIGS["fp8"]
    wcfg = dataclasses.replace(base, name=f"short-{name}", batch=batch, num_q_heads=hq,
                               num_kv_heads=hkv)
    lengths = short_lengths(batch, hi, seed)
    case = build_case(wcfg, lengths=lengths, num_workgroups=W, min_tiles=1)
    nbins, nsplit = short_bins(case)
    say(f"[short] {name}: {nbins} bins of short descriptors, {nsplit} of their "
        f"descriptors split")
    assert nbins >= 2 and nsplit >= 1
    out, q64 = run(case, entry)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case), q64), f"short {name}")


def test_short_and_long_bins_in_one_launch(gpu_lib):
    """Forty short requests, then eight of 512 tokens: the same launch
    drains the bins of the short ones one descriptor per wave and the bins
    of the long ones descriptor by descriptor."""
    lengths = short_lengths(40, 128, 3) + [512] * 8
    wcfg = dataclasses.replace(CONFIGS["tiny"], name="short-long", batch=len(lengths),
                               num_q_heads=16, num_kv_heads=2)
    case = build_case(wcfg, lengths=lengths, num_workgroups=32, min_tiles=1)
    nbins, nsplit = short_bins(case)
    used = int(lbp.read_taskmap(case.plan_ws, case.info)["header"][3])
    say(f"[short] short and long: {nbins} of {used} bins of short descriptors, {nsplit} split")
    assert 2 <= nbins <= used - 2 and nsplit >= 1
    out, q64 = run(case, "attend")
    compare(case, out, oracle_pairs(case, 0, all_pairs(case), q64), "short and long")


@pytest.mark.parametrize("entry", ["attend", "fp8q"])
def test_short_requests_after_a_long_one(gpu_lib, entry):
    """One 8192-token request, then fifteen of 1-128 tokens, over 16 bins:
    fewer pairs than bins, yet the short ones pack six to nine to a bin
    behind the long one's last piece, one of them split across two such
    bins."""
    lengths = [8192] + short_lengths(15, 128, 9)
    wcfg = dataclasses.replace(CONFIGS["fp8"], name=f"short-after-long-{entry}",
                               batch=len(lengths), num_q_heads=8, num_kv_heads=1)
    case = build_case(wcfg, lengths=lengths, num_workgroups=16, min_tiles=1)
    nbins, nsplit = short_bins(case)
    say(f"[short] after a long one ({entry}): {nbins} bins of short descriptors, {nsplit} split")
    assert nbins >= 2 and nsplit >= 1
    out, q64 = run(case, entry)
    compare(case, out, oracle_pairs(case, 0, all_pairs(case), q64), f"short after long {entry}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_large_batch_of_short_requests(gpu_lib, kv):
    """1024 requests of 1-128 tokens at 64 query / 8 KV heads (8192 pairs,
    32 per bin at one bin per CU): the launch shape of the benchmark, every
    row against the oracle."""
    base = CONFIGS["uniform"] if kv == "bf16" else CONFIGS["fp8"]
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(1, 129, size=1024)]
    wcfg = dataclasses.replace(base, name=f"short-large-{kv}", batch=len(lengths))
    case = build_case(wcfg, lengths=lengths)
    nbins, nsplit = short_bins(case)
    used = int(lbp.read_taskmap(case.plan_ws, case.info)["header"][3])
    say(f"[short] large {kv}: {nbins} of {used} bins of short descriptors, {nsplit} split")
    assert nbins >= used // 2 and nsplit >= 1
    out, q64 = run(case, "attend")
    compare(case, out, oracle_pairs(case, 0, all_pairs(case), q64), f"short large {kv}")
