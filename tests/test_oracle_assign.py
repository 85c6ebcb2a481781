"""CPU pins of the oracle's task-map builders."""

import numpy as np
import pytest

import oracle
import pins


def test_assign_pins():
    pins.pins_assign(oracle.assign)


@pytest.mark.parametrize("sec", pins.load_golden_taskmaps(),
                         ids=lambda s: f"{s['policy']}-" + "-".join(f"{k}{v}" for k, v in s["params"].items()))
def test_golden_taskmap(sec):
    tm = pins.build_from_golden(oracle.assign, sec)
    pins.assert_taskmap_equals(tm, sec["header"], sec["num_bins"][0], sec["bin_offset"],
                               sec["desc"], sec["pair_first"], sec["pair_count"])


def test_workload_maps_structure():
    """The five workloads' maps at W = 256, F = 4 satisfy every invariant."""
    from workloads import CONFIGS, draw_lengths
    for name, cfg in CONFIGS.items():
        L = draw_lengths(cfg, np.random.default_rng(cfg.seed))
        tm = oracle.assign.assign_dynamic(L, cfg.num_kv_heads, 256, 4)
        if name != "fp8":                       # fp8 is large; invariants are O(D * pairs)
            pins.check_taskmap_invariants(tm, L, cfg.num_kv_heads, "dynamic")
        assert tm.U <= 256
        assert tm.D <= cfg.num_kv_heads * cfg.batch + tm.U - 1
    L = draw_lengths(CONFIGS["uniform"], np.random.default_rng(1))
    tm = oracle.assign.assign_dynamic(L, 8, 256, 4)
    assert tm.header() == (16384, 64, 256, 256)


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.assign.assign_dynamic([10], 1, 0, 4)
    with pytest.raises(ValueError):
        oracle.assign.assign_dynamic([-1], 1, 4, 4)
    with pytest.raises(ValueError):
        oracle.assign.assign_static_chunk([1000], 1, 2, 3)


def test_descriptors_start_on_page_boundaries():
    """Every descriptor of every policy begins on a 64-token page boundary.
    The attention kernel relies on it: its spans of two 16-token slices start
    at multiples of 32 tokens inside a descriptor, so both slices of a span
    lie in one page.  (The GPU plans equal these maps bit for bit.)"""
    rng = np.random.default_rng(5)
    L = rng.integers(0, 5000, size=40)
    L[:3] = [0, 1, 64]
    maps = [oracle.assign.assign_dynamic(L, 3, 37, 1), oracle.assign.assign_dynamic(L, 3, 256, 4),
            oracle.assign.assign_static_splits(L, 3, 7),
            oracle.assign.assign_static_chunk(L, 3, 5, int(np.ceil(L.max() / 64)))]
    for tm in maps:
        assert tm.D > 0
        assert np.all(tm.desc[:tm.D, 2] % 64 == 0)
        assert np.all(tm.desc[:tm.D, 3] > tm.desc[:tm.D, 2])
