"""CPU checks of the seeded workload definitions (no GPU, no oracle)."""

import collections

import numpy as np

from workloads import CONFIGS, TABLE3, draw_lengths, draw_page_table


def test_table3_mixes_are_the_pages_a_by_b_mixes():
    # vLLM x HPC-Ops page, Table 3: "A x B" = A requests at KV length B (K = 1024)
    expect = {
        "64x0.5K": {512: 64},
        "64x4K": {4096: 64},
        "32x0.125K+32x4K": {128: 32, 4096: 32},
        "2x32K+30x4K": {32768: 2, 4096: 30},
        "1x64K+15x4K": {65536: 1, 4096: 15},
        "1x128K+31x4K": {131072: 1, 4096: 31},
    }
    assert set(TABLE3) == set(expect)
    for name, cfg in TABLE3.items():
        lens = draw_lengths(cfg, np.random.default_rng(cfg.seed))
        assert dict(collections.Counter(lens.tolist())) == expect[name], name
        assert (cfg.num_q_heads, cfg.num_kv_heads, cfg.kv_dtype) == (8, 1, "fp8_e4m3")
        assert cfg.batch == len(lens)


def test_page_tables_are_permutations():
    for cfg in list(CONFIGS.values()) + list(TABLE3.values()):
        rng = np.random.default_rng(cfg.seed)
        lens = draw_lengths(cfg, rng)
        table, P = draw_page_table(lens, rng)
        n = (lens.astype(np.int64) + 63) // 64
        used = np.concatenate([table[r, :k] for r, k in enumerate(n)])
        assert sorted(used.tolist()) == list(range(P)), cfg.name


def test_fp8_query_recipe():
    import torch
    from oracle.e4m3 import dequantize
    from workloads import quantize_query_e4m3
    g = torch.Generator().manual_seed(7)
    q = torch.randn((3, 8, 128), generator=g).to(torch.bfloat16)
    q[1, 2] = 0
    codes, scale = quantize_query_e4m3(q)
    assert codes.dtype == torch.uint8 and scale.shape == (3, 8)
    vals = dequantize(codes.numpy(), scale.numpy())
    x = q.double().numpy()
    assert float(scale[1, 2]) == 1.0 and np.all(vals[1, 2] == 0)
    # the row maximum maps to +-448 exactly; every value within e4m3 rounding (2^-4 rel)
    amax = np.abs(x).max(-1)
    assert np.allclose(np.abs(vals).max(-1), amax, rtol=1e-6)
    assert np.all(np.abs(vals - x) <= np.abs(x) * 2.0 ** -4 + scale.numpy()[..., None] * 2.0 ** -9)
