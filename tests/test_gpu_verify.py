"""GPU parity of multi-token decode (speculative verification, cfg.q_len > 1).

Token j of request r sits at position L_r - q_len + j and attends causally to
the KV positions up to its own; the MFMA columns hold (token, head) pairs of
the KV head's group, G * q_len <= 64, as up to four 16-column MFMA tiles per
wave.  Every case is compared with the fp64
oracle (oracle.attention.paged_verify_attention) at the path's tolerance,
through lbp_attend, lbp_attend_fused and (FP8) lbp_attend_fp8q, including
tokens with no visible position (zeros) and descriptors in which a column
sees no token at all.
"""

import dataclasses
import time

import numpy as np

import pytest
import torch

import load_balanced_paged_amd as lbp
import oracle
from gpu_support import (all_pairs, assert_taskmap_matches, bits, build_case, compare_verify,
                         oracle_verify_layer, oracle_verify_pairs, say)
from workloads import CONFIGS, quantize_query_e4m3

pytestmark = pytest.mark.gpu


def make_q(case, T, seed=0):
    B = len(case.wl.lengths)
    g = torch.Generator(device="cuda").manual_seed(900 + seed)
    return torch.randn((B, T, case.wcfg.num_q_heads, 128), generator=g, device="cuda").to(
        torch.bfloat16)


def run(case, q, fn=lbp.lbp_attend):
    lay = case.wl.layers[0]
    out = torch.full_like(q, float("nan"))
    fn(case.cfg, case.info, case.plan_ws, q, lay.k_cache, lay.v_cache, lay.k_scale, lay.v_scale,
       case.split_ws, out)
    torch.cuda.synchronize()
    return out


def q64_of(q):
    return oracle.attention.bf16_bits_to_f64(bits(q))


@pytest.mark.parametrize("name", ["tiny", "skewed"])
def test_verify_two_tokens_all_rows(gpu_lib, name):
    case = build_case(CONFIGS[name], q_len=2)
    assert_taskmap_matches(case)
    q = make_q(case, 2)
    ref = oracle_verify_pairs(case, 0, all_pairs(case), q64_of(q))
    compare_verify(case, run(case, q), ref, f"verify {name} T=2")
    compare_verify(case, run(case, q, lbp.lbp_attend_fused), ref, f"verify {name} T=2 fused")


def test_verify_mixed_all_pairs(gpu_lib):
    """Two verification rows per request: every pair of the mixed-length
    workload against the oracle."""
    case = build_case(CONFIGS["mixed"], q_len=2)
    q = make_q(case, 2, seed=1)
    t0 = time.time()
    ref = oracle_verify_layer(case, 0, q64_of(q))
    say(f"[verify] mixed T=2 oracle over {len(ref)} pairs: {time.time() - t0:.1f} s")
    compare_verify(case, run(case, q), ref, "verify mixed T=2 all pairs")


@pytest.mark.parametrize("group,hkv,T", [(4, 2, 4), (1, 4, 16), (3, 3, 5), (16, 1, 1)])
def test_verify_shapes_short_requests(gpu_lib, group, hkv, T):
    """Requests shorter than T (early tokens see nothing), tile-sized bins."""
    wcfg = dataclasses.replace(CONFIGS["tiny"], name=f"v{group}x{T}", batch=6,
                               num_q_heads=group * hkv, num_kv_heads=hkv)
    case = build_case(wcfg, lengths=[1, 2, 3, 65, 130, 900], num_workgroups=7, min_tiles=1,
                      q_len=T)
    q = make_q(case, T, seed=2)
    ref = oracle_verify_pairs(case, 0, all_pairs(case), q64_of(q))
    out = run(case, q)
    compare_verify(case, out, ref, f"verify G={group} T={T}")
    compare_verify(case, run(case, q, lbp.lbp_attend_fused), ref, f"verify G={group} T={T} fused")
    # a token before the sequence start outputs exact zeros
    assert torch.all(out[0, :T - 1] == 0) if T > 1 else True


@pytest.mark.parametrize("group,hkv,T", [(8, 2, 6), (8, 1, 8), (4, 2, 5), (16, 1, 4), (3, 3, 7),
                                         (1, 1, 32), (1, 2, 40), (2, 1, 30), (1, 1, 64),
                                         (1, 1, 17), (11, 1, 3), (7, 2, 7)])
def test_verify_column_blocks(gpu_lib, group, hkv, T):
    """More than 16 query columns (up to 64): two 16-column tiles per wave up
    to 32, three up to 48 and four up to 64 (one wave per SIMD, 32-token
    spans), each at its lowest column count too (17, 33, 49); with one or two
    heads per group, nearly every column has its own causal limit, and q_len
    up to 64 puts limits deep into the last spans."""
    wcfg = dataclasses.replace(CONFIGS["tiny"], name=f"vb{group}x{T}", batch=6,
                               num_q_heads=group * hkv, num_kv_heads=hkv)
    case = build_case(wcfg, lengths=[1, 5, 64, 200, 777, 2100], num_workgroups=9, min_tiles=1,
                      q_len=T)
    q = make_q(case, T, seed=6)
    ref = oracle_verify_pairs(case, 0, all_pairs(case), q64_of(q))
    out = run(case, q)
    compare_verify(case, out, ref, f"verify blocks G={group} T={T}")
    compare_verify(case, run(case, q, lbp.lbp_attend_fused), ref,
                   f"verify blocks G={group} T={T} fused")
    assert torch.all(out[0, :T - 1] == 0)


def test_verify_six_rows_mixed_all_pairs(gpu_lib):
    """Six verification rows per request at the 8-query-head group (48
    columns): every pair of the mixed-length workload against the oracle."""
    case = build_case(CONFIGS["mixed"], q_len=6)
    q = make_q(case, 6, seed=7)
    t0 = time.time()
    ref = oracle_verify_layer(case, 0, q64_of(q))
    say(f"[verify] mixed T=6 oracle over {len(ref)} pairs: {time.time() - t0:.1f} s")
    compare_verify(case, run(case, q), ref, "verify mixed T=6 all pairs")


@pytest.mark.timeout(240)
def test_verify_six_rows_fp8_all_pairs(gpu_lib):
    """Six verification rows per request over the FP8-KV workload (128
    requests of 1K-256K tokens, 48 columns): every pair against the oracle."""
    case = build_case(CONFIGS["fp8"], q_len=6)
    q = make_q(case, 6, seed=11)
    t0 = time.time()
    ref = oracle_verify_layer(case, 0, q64_of(q))
    say(f"[verify] fp8 T=6 oracle over {len(ref)} pairs: {time.time() - t0:.1f} s")
    compare_verify(case, run(case, q), ref, "verify fp8 T=6 all pairs")


def test_verify_fully_masked_descriptor(gpu_lib):
    """L = 65 with one-tile bins: the descriptor [64, 65) is invisible to the
    first of two tokens, so its partial for those columns is empty."""
    wcfg = dataclasses.replace(CONFIGS["tiny"], name="v-masked", batch=3)
    case = build_case(wcfg, lengths=[65, 129, 64], num_workgroups=64, min_tiles=1, q_len=2)
    tm = lbp.read_taskmap(case.plan_ws, case.info)
    assert [64, 65] in tm["desc"][:, 2:].tolist()
    q = make_q(case, 2, seed=3)
    ref = oracle_verify_pairs(case, 0, all_pairs(case), q64_of(q))
    compare_verify(case, run(case, q), ref, "verify masked descriptor")
    compare_verify(case, run(case, q, lbp.lbp_attend_fused), ref, "verify masked descriptor fused")


def test_verify_static_plan(gpu_lib):
    case = build_case(CONFIGS["skewed"], policy=lbp.LBP_POLICY_STATIC_SPLITS, param=5, q_len=2)
    q = make_q(case, 2, seed=4)
    compare_verify(case, run(case, q), oracle_verify_pairs(case, 0, all_pairs(case), q64_of(q)),
                   "verify static")


@pytest.mark.parametrize("T", [2, 3, 4])
def test_verify_fp8_kv_and_query(gpu_lib, T):
    """FP8 KV with a BF16 and with an FP8 query: 16 columns (one MFMA column
    tile per wave), 24 and 32 (two tiles per wave)."""
    wcfg = dataclasses.replace(CONFIGS["fp8"], name="v-fp8", batch=5)
    case = build_case(wcfg, lengths=[1, 70, 700, 3000, 20000], q_len=T)
    q = make_q(case, T, seed=5)
    pairs = all_pairs(case)
    compare_verify(case, run(case, q), oracle_verify_pairs(case, 0, pairs, q64_of(q)),
                   "verify fp8 kv")
    codes, scale = quantize_query_e4m3(q)
    lay = case.wl.layers[0]
    out = torch.full_like(q, float("nan"))
    lbp.lbp_attend_fp8q(case.cfg, case.info, case.plan_ws, codes, scale, lay.k_cache,
                        lay.v_cache, lay.k_scale, lay.v_scale, case.split_ws, out)
    torch.cuda.synchronize()
    q8 = oracle.e4m3.dequantize(codes.cpu().numpy(), scale.cpu().numpy())
    compare_verify(case, out, oracle_verify_pairs(case, 0, pairs, q8), "verify fp8 q")


@pytest.mark.parametrize("T", [6, 8])
def test_verify_fp8_column_blocks(gpu_lib, T):
    """FP8 KV and FP8 query with 48 and 64 columns (three and four column
    tiles per wave at one wave per SIMD)."""
    wcfg = dataclasses.replace(CONFIGS["fp8"], name=f"vb-fp8-{T}", batch=4)
    case = build_case(wcfg, lengths=[3, 300, 4000, 9000], num_workgroups=20, q_len=T)
    q = make_q(case, T, seed=8)
    pairs = all_pairs(case)
    compare_verify(case, run(case, q), oracle_verify_pairs(case, 0, pairs, q64_of(q)),
                   f"verify blocks fp8 kv T={T}")
    compare_verify(case, run(case, q, lbp.lbp_attend_fused),
                   oracle_verify_pairs(case, 0, pairs, q64_of(q)),
                   f"verify blocks fp8 kv fused T={T}")
    codes, scale = quantize_query_e4m3(q)
    lay = case.wl.layers[0]
    out = torch.full_like(q, float("nan"))
    lbp.lbp_attend_fp8q(case.cfg, case.info, case.plan_ws, codes, scale, lay.k_cache,
                        lay.v_cache, lay.k_scale, lay.v_scale, case.split_ws, out)
    torch.cuda.synchronize()
    q8 = oracle.e4m3.dequantize(codes.cpu().numpy(), scale.cpu().numpy())
    compare_verify(case, out, oracle_verify_pairs(case, 0, pairs, q8), f"verify blocks fp8 q T={T}")


@pytest.mark.parametrize("T", [2, 6])
def test_verify_ticket_mode(gpu_lib, T):
    """More bins than CUs: workgroups take bins from the ticket counter, in
    the causal (T = 2) and three-tile (T = 6) instances, both merge forms."""
    wcfg = dataclasses.replace(CONFIGS["tiny"], name=f"v-ticket{T}", batch=4)
    case = build_case(wcfg, lengths=[3000, 50, 700, 9000], num_workgroups=1024, min_tiles=1,
                      q_len=T)
    q = make_q(case, T, seed=9)
    ref = oracle_verify_pairs(case, 0, all_pairs(case), q64_of(q))
    compare_verify(case, run(case, q), ref, f"verify ticket T={T}")
    compare_verify(case, run(case, q, lbp.lbp_attend_fused), ref, f"verify ticket T={T} fused")


def test_verify_zero_length_requests(gpu_lib):
    """A request with no tokens outputs zero rows for every query token."""
    wcfg = dataclasses.replace(CONFIGS["tiny"], name="v-zero", batch=4)
    case = build_case(wcfg, lengths=[0, 5, 0, 300], num_workgroups=3, min_tiles=1, q_len=4)
    q = make_q(case, 4, seed=10)
    out = run(case, q)
    assert torch.all(out[0] == 0) and torch.all(out[2] == 0)
    compare_verify(case, out, oracle_verify_pairs(case, 0, all_pairs(case), q64_of(q)),
                   "verify zero lengths")


def test_verify_fused_two_levels_blocks(gpu_lib):
    """A pair of more than 256 partials at 48 columns: the in-kernel merge runs
    both levels in column chunks."""
    wcfg = dataclasses.replace(CONFIGS["tiny"], name="v-two-level", batch=2)
    case = build_case(wcfg, lengths=[20000, 100], num_workgroups=1024, min_tiles=1, q_len=6)
    tm = lbp.read_taskmap(case.plan_ws, case.info)
    assert tm["pair_count"].max() > 256
    q = make_q(case, 6, seed=11)
    ref = oracle_verify_pairs(case, 0, all_pairs(case), q64_of(q))
    compare_verify(case, run(case, q, lbp.lbp_attend_fused), ref, "verify two-level fused")
    compare_verify(case, run(case, q), ref, "verify two-level two launches")


def test_verify_graph_replay_matches_eager(gpu_lib):
    """Plan and three-tile fused verification captured in a HIP graph: every
    replay equals eager, bit for bit."""
    T = 6
    wcfg = dataclasses.replace(CONFIGS["tiny"], name="v-graph", batch=4)
    case = build_case(wcfg, lengths=[3000, 50, 700, 9000], num_workgroups=64, min_tiles=1,
                      q_len=T)
    q = make_q(case, T, seed=12)
    eager = run(case, q, lbp.lbp_attend_fused).clone()
    out = torch.zeros_like(eager)
    lay = case.wl.layers[0]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            lbp.lbp_plan(case.cfg, case.seq_lens, case.page_table, case.plan_ws, stream=s)
            lbp.lbp_attend_fused(case.cfg, case.info, case.plan_ws, q, lay.k_cache, lay.v_cache,
                                 None, None, case.split_ws, out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        out.zero_()
        run(case, q)                       # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep


def test_verify_one_token_equals_decode(gpu_lib):
    """q_len = 1 in the [B, 1, Hq, D] layout is bit-identical to plain decode."""
    case = build_case(CONFIGS["skewed"])
    lay = case.wl.layers[0]
    a = run(case, lay.q[:, None].contiguous())
    b = torch.empty_like(lay.q)
    lbp.lbp_attend(case.cfg, case.info, case.plan_ws, lay.q, lay.k_cache, lay.v_cache, None, None,
                   case.split_ws, b)
    torch.cuda.synchronize()
    assert torch.equal(a[:, 0].view(torch.int16), b.view(torch.int16))
