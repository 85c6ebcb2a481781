"""The parity gate of the GPU tests, checked on the CPU.

At unit-spread inputs an output row over L tokens has a spread of about
sqrt(e / L): at the FP8 workload's longest rows (L = 262144) that is about
3e-3, with row maxima near 1e-2, so the FP8 max-abs bound (3e-2) alone would
pass a kernel that lost those rows.  The per-pair relative bound must reject
it, and must still accept the output's own BF16 rounding.
"""

import numpy as np
import torch

import oracle
from gpu_support import FP8_MAX_ABS, PAIR_REL_RMS, BF16_REL_RMS, check_parity, parity_stats


def _long_row(L=262144, G=8, seed=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, 128))
    K = rng.standard_normal((L, 128))
    V = rng.standard_normal((L, 128))
    o, _ = oracle.attention.attend_range(q, K, V, 128 ** -0.5)
    return o


def _bf16(x):
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()


def test_zeroed_long_row_fails_only_the_pair_bound():
    ref = _long_row()[None]
    assert np.abs(ref).max() < FP8_MAX_ABS          # max-abs alone cannot see a lost row
    st = parity_stats(np.zeros_like(ref), ref, [262144])
    assert st["max_abs"] <= FP8_MAX_ABS
    assert st["pair_rel_max"] == 1.0
    try:
        check_parity("fp8_e4m3", st, "zeroed")
    except AssertionError:
        pass
    else:
        raise AssertionError("a zeroed 262144-token row passed the parity gate")


def test_bf16_rounded_output_passes_with_margin():
    ref = np.stack([_long_row(L, seed=L)[None][0] for L in (1, 3, 100, 5000, 262144)])
    st = parity_stats(_bf16(ref), ref, [1, 3, 100, 5000, 262144])
    check_parity("bf16", st, "bf16 rounding")
    # the relative error of the output's own rounding (about 1.6e-3 at every
    # length) stays far inside the relative bounds; its absolute error is
    # that of the largest values (a one-token row is v_0 itself)
    assert st["pair_rel_max"] < PAIR_REL_RMS / 4
    assert st["rel_rms"] < BF16_REL_RMS / 2


def test_pair_without_tokens_must_be_exact_zero():
    ref = np.zeros((1, 8, 128))
    assert parity_stats(np.zeros_like(ref), ref)["pair_rel_max"] == 0.0
    bad = np.zeros_like(ref)
    bad[0, 0, 0] = 1e-6
    assert parity_stats(bad, ref)["pair_rel_max"] == np.inf
