"""GPU parity of the task-map builders: bit-exact against the oracle."""

import dataclasses

import numpy as np
import pytest
import torch

import load_balanced_paged_amd as lbp
from gpu_support import (assert_taskmap_matches, build_case, expected_bin_pages,
                         expected_split_list, say)
from workloads import CONFIGS

pytestmark = pytest.mark.gpu


def plan_only(wcfg, lengths, H, W, F, policy=lbp.LBP_POLICY_DYNAMIC, param=0, max_pages=None):
    """Build a plan for explicit lengths without drawing any KV tensors."""
    lengths = np.asarray(lengths, dtype=np.int32)
    npages = (lengths.astype(np.int64) + 63) // 64
    mp = max_pages or max(1, int(npages.max()) if len(npages) else 1)
    cfg = lbp.make_config(8 * H, H, len(lengths), mp, num_workgroups=W, min_tiles_per_bin=F)
    pb, _ = lbp.lbp_query_workspace(cfg, policy, param)
    ws = torch.full((pb,), 0xA5, dtype=torch.uint8, device="cuda")   # stale bytes must not leak
    seq = torch.from_numpy(lengths).cuda()
    # distinct page ids (a seeded permutation), so that the per-bin first
    # pages the plan records are checkable
    host_table = np.random.default_rng(len(lengths) * 7 + mp).permutation(
        len(lengths) * mp).astype(np.int32).reshape(len(lengths), mp)
    table = torch.from_numpy(host_table).cuda()
    if policy == lbp.LBP_POLICY_DYNAMIC:
        info = lbp.lbp_plan(cfg, seq, table, ws)
    else:
        info = lbp.lbp_plan_static(cfg, policy, param, seq, table, ws)
    torch.cuda.synchronize()
    got = lbp.read_taskmap(ws, info)
    got["host_table"] = host_table
    return got, info, cfg


def check(got, ref):
    assert got["status"] == 0
    assert got["header"] == ref.header(), (got["header"], ref.header())
    assert np.array_equal(got["bin_offset"], ref.bin_offset)
    assert np.array_equal(got["desc"], ref.desc)
    assert np.array_equal(got["pair_first"], ref.pair_first)
    assert np.array_equal(got["pair_count"], ref.pair_count)
    assert np.array_equal(got["split_list"], expected_split_list(ref))
    if ref.num_bins and got["policy"] == lbp.LBP_POLICY_DYNAMIC:
        assert len(got["split_list"]) <= ref.num_bins - 1
    for b in range(ref.num_bins):
        d0, d1 = ref.bin_offset[b], ref.bin_offset[b + 1]
        want = ref.desc[d0] if d1 > d0 else np.zeros(4, np.int32)
        assert np.array_equal(got["bin_first"][b], want), b
    if "host_table" in got:
        assert np.array_equal(got["bin_pages"], expected_bin_pages(ref, got["host_table"]))


@pytest.mark.parametrize("F", [0, 4])
@pytest.mark.parametrize("name", list(CONFIGS))
def test_workload_taskmap_bitexact(gpu_lib, name, F):
    """The five workloads' maps at the benchmark's launch shape (one bin per
    CU): with the library's default floor (F = 0 in the config, which means
    F = 1, no floor) and with F = 4."""
    import oracle
    wcfg = CONFIGS[name]
    from workloads import draw_lengths
    L = draw_lengths(wcfg, np.random.default_rng(wcfg.seed))
    say(f"[plan] {name} F={F}")
    got, info, _ = plan_only(wcfg, L, wcfg.num_kv_heads, 0, F)
    ref = oracle.assign.assign_dynamic(L, wcfg.num_kv_heads, info.num_bins, F if F > 0 else 1)
    check(got, ref)
    say(f"[plan] {name}: W={info.num_bins} T={ref.T} budget={ref.budget} D={ref.D} U={ref.U}")


def random_cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 300))
        H = int(rng.choice([1, 2, 8]))
        W = int(rng.choice([1, 7, 256, 512, 1024]))
        F = int(rng.choice([1, 4, 16]))
        kind = i % 5
        if kind == 0:
            L = rng.integers(0, 5000, size=B)
        elif kind == 1:
            L = 64 * rng.integers(0, 40, size=B)
        elif kind == 2:
            L = np.exp(rng.uniform(0, np.log(200000), size=B)).astype(int)
        elif kind == 3:
            L = np.ones(B, dtype=int)
        else:
            L = np.where(rng.random(B) < 0.5, 0, rng.integers(1, 300, size=B))
        out.append((L.astype(np.int32), H, W, F))
    return out


@pytest.mark.parametrize("idx", range(30))
def test_dynamic_taskmap_random_bitexact(gpu_lib, idx):
    import oracle
    L, H, W, F = random_cases(2024, 30)[idx]
    say(f"[plan] random {idx}: B={len(L)} H={H} W={W} F={F} T={int(((L + 63) // 64).sum()) * H}")
    got, info, _ = plan_only(None, L, H, W, F)
    check(got, oracle.assign.assign_dynamic(L, H, W, F))


def test_large_pair_count_bitexact(gpu_lib):
    """More pairs than the 1024 threads of the assign workgroup."""
    import oracle
    rng = np.random.default_rng(5)
    L = rng.integers(0, 3000, size=700).astype(np.int32)
    got, info, _ = plan_only(None, L, 8, 512, 4)
    check(got, oracle.assign.assign_dynamic(L, 8, 512, 4))


def test_pair_count_past_lds_bitexact(gpu_lib):
    """More than 12288 pairs: the assign kernel keeps its flat starts and
    first slots in the plan workspace instead of LDS (dynamic and static
    plans)."""
    import oracle
    rng = np.random.default_rng(6)
    L = rng.integers(0, 3000, size=1600).astype(np.int32)
    assert 8 * len(L) > 12288
    got, info, _ = plan_only(None, L, 8, 512, 4)
    check(got, oracle.assign.assign_dynamic(L, 8, 512, 4))
    got, info, _ = plan_only(None, L, 8, 0, 4, lbp.LBP_POLICY_STATIC_SPLITS, 3)
    check(got, oracle.assign.assign_static_splits(L, 8, 3))


@pytest.mark.parametrize("S", [1, 2, 3, 8, 64])
def test_static_splits_bitexact(gpu_lib, S):
    import oracle
    rng = np.random.default_rng(S)
    L = np.concatenate([[0, 1, 64, 65], rng.integers(0, 20000, size=40)]).astype(np.int32)
    got, info, _ = plan_only(None, L, 2, 0, 4, lbp.LBP_POLICY_STATIC_SPLITS, S)
    check(got, oracle.assign.assign_static_splits(L, 2, S))
    assert info.num_bins == 2 * len(L) * S


@pytest.mark.parametrize("C", [1, 4, 16])
def test_static_chunk_bitexact(gpu_lib, C):
    import oracle
    rng = np.random.default_rng(100 + C)
    L = np.concatenate([[0, 1, 64, 65], rng.integers(0, 5000, size=30)]).astype(np.int32)
    mp = 100
    got, info, cfg = plan_only(None, L, 2, 0, 4, lbp.LBP_POLICY_STATIC_CHUNK, C, max_pages=mp)
    check(got, oracle.assign.assign_static_chunk(L, 2, C, mp))


def test_length_over_capacity_is_clamped_and_flagged(gpu_lib):
    L = np.array([100, 64 * 5 + 3], dtype=np.int32)
    got, info, cfg = plan_only(None, L, 1, 4, 1, max_pages=5)
    assert got["status"] == 1
    assert got["desc"][:, 3].max() == 64 * 5


def test_plan_matches_after_reuse_of_workspace(gpu_lib):
    """A second plan into the same workspace fully replaces the first."""
    import oracle
    wcfg = CONFIGS["skewed"]
    case = build_case(wcfg)
    assert_taskmap_matches(case)
    L2 = np.asarray(case.wl.lengths)[::-1].copy()
    case.seq_lens.copy_(torch.from_numpy(L2))
    info = lbp.lbp_plan(case.cfg, case.seq_lens, case.page_table, case.plan_ws)
    torch.cuda.synchronize()
    check(lbp.read_taskmap(case.plan_ws, info),
          oracle.assign.assign_dynamic(L2, 1, info.num_bins, info.param))


@pytest.mark.parametrize("B,H,W", [(1536, 8, 256), (4096, 8, 256), (12288, 1, 1024), (300, 64, 7),
                                   (5000, 8, 256)])
def test_large_batch_plans_bitexact(gpu_lib, B, H, W):
    """Large batches, up to 40000 pairs: per-pair arrays in LDS (up to 12288
    pairs), lengths only in LDS (up to 36864) and everything in the plan
    workspace; short requests among long ones, so bins hold many
    descriptors and a long pair spans many bins."""
    import oracle
    rng = np.random.default_rng(B + H)
    L = np.where(rng.random(B) < 0.9, rng.integers(0, 200, size=B),
                 rng.integers(1000, 100000, size=B)).astype(np.int32)
    say(f"[plan] large B={B} H={H} W={W} pairs={B * H}")
    got, info, _ = plan_only(None, L, H, W, 1)
    check(got, oracle.assign.assign_dynamic(L, H, W, 1))
    got, info, _ = plan_only(None, L, H, 0, 1, lbp.LBP_POLICY_STATIC_SPLITS, 2)
    check(got, oracle.assign.assign_static_splits(L, H, 2))


def test_taskmap_to_host_on_a_side_stream(gpu_lib):
    """lbp_taskmap_to_host, ordered on the stream that built the plan,
    returns exactly the workspace's first lbp_plan_layout(info).total bytes
    and agrees with the oracle's map."""
    import oracle
    rng = np.random.default_rng(77)
    L = rng.integers(0, 3000, size=40).astype(np.int32)
    H, W = 4, 64
    mp = int((L.max() + 63) // 64)
    cfg = lbp.make_config(8 * H, H, len(L), mp, num_workgroups=W, min_tiles_per_bin=1)
    pb, _ = lbp.lbp_query_workspace(cfg)
    ws = torch.full((pb,), 0x5A, dtype=torch.uint8, device="cuda")
    seq = torch.from_numpy(L).cuda()
    table = torch.arange(len(L) * mp, dtype=torch.int32, device="cuda").view(len(L), mp)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    info = lbp.lbp_plan(cfg, seq, table, ws, stream=s)
    raw = lbp.lbp_taskmap_to_host(ws, info, stream=s)
    torch.cuda.synchronize()
    total = lbp.lbp_plan_layout(info).total
    assert raw.nbytes == total
    assert np.array_equal(raw, ws[:total].cpu().numpy())
    got = lbp.read_taskmap(ws, info)
    got["host_table"] = table.cpu().numpy()
    check(got, oracle.assign.assign_dynamic(L, H, W, 1))
