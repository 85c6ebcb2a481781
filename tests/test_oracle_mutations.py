"""Planted mistakes in copies of the oracle must fail at least one pin.

Each case edits the oracle's source text (a dropped term, a wrong sign,
index or operand), loads the edited copy as a fresh module on the CPU, and
runs the same pins the real oracle passes.  The real oracle files are not
touched.
"""

import importlib.util
import os
import sys

import pytest

import oracle
import pins

ORACLE_DIR = os.path.dirname(oracle.__file__)


def load_mutant(modname, old, new):
    src = open(os.path.join(ORACLE_DIR, modname + ".py")).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    spec = importlib.util.spec_from_loader(f"oracle._mutant_{modname}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    sys.modules[spec.name] = mod          # dataclasses look the module up by name
    exec(compile(src, f"<mutant {modname}>", "exec"), mod.__dict__)
    return mod


ASSIGN_MUTATIONS = [
    ("budget floor instead of ceiling", "max(-(-T // num_bins), min_tiles)", "max(T // num_bins, min_tiles)"),
    ("minimum-work floor dropped", "max(-(-T // num_bins), min_tiles)", "-(-T // num_bins)"),
    ("tile size 32", "TILE_TOKENS = 64", "TILE_TOKENS = 32"),
    ("partial tile dropped", "(L + TILE_TOKENS - 1) // TILE_TOKENS", "L // TILE_TOKENS"),
    ("token end not clipped", "min(TILE_TOKENS * t1, int(L[r]))", "TILE_TOKENS * t1"),
    ("early spill", "if fill == budget:", "if fill >= budget - 1:"),
    ("T counts one head", "T = int(n.sum()) * num_kv_heads", "T = int(n.sum())"),
    ("pair index batch-major", "pair_count[g * B + r] += 1", "pair_count[r * num_kv_heads + g] += 1"),
    ("static split width floor", "c = -(-int(n[r]) // splits)", "c = max(1, int(n[r]) // splits)"),
    ("static split bin index", "bins[p * splits + s]", "bins[s * num_kv_heads * B + p]"),
    ("static chunk grid floor", "S = -(-max_pages_per_seq // chunk_tiles)", "S = max(1, max_pages_per_seq // chunk_tiles)"),
]

ATTENTION_MUTATIONS = [
    ("slot off by one", "slots = t % PAGE_TOKENS", "slots = (t + 1) % PAGE_TOKENS"),
    ("page index off", "[t // PAGE_TOKENS]", "[(t + 1) // PAGE_TOKENS]"),
    ("GQA map interleaved", "o, l = attend_range(q[r, g * G:(g + 1) * G], K, V, sm_scale)",
     "o, l = attend_range(q[r, g::num_kv_heads], K, V, sm_scale)"),
    ("scale dropped", "s = sm_scale * (q_group @ K.T)", "s = (q_group @ K.T)"),
    ("softmax sign", "w = np.exp(s - m)", "w = np.exp(m - s)"),
    ("V replaced by K", "o = (w @ V) / l", "o = (w @ K) / l"),
    ("normaliser dropped", "o = (w @ V) / l", "o = (w @ V)"),
    ("lse max term dropped", "lse = (m + np.log(l))[:, 0]", "lse = (np.log(l))[:, 0]"),
    ("combine weight sign", "np.exp(lse_k - np.where", "np.exp(-lse_k + 0 * np.where"),
    ("combine not renormalised", "out[has] /= tot[has, None]", "pass"),
    ("fp8 scale divides", "return e4m3.decode(raw) * s[:, None]", "return e4m3.decode(raw) / s[:, None]"),
    ("bf16 widening shift", "astype(np.uint32) << 16", "astype(np.uint32) << 15"),
]

E4M3_MUTATIONS = [
    ("exponent bias 8", "2.0 ** (e - 7)", "2.0 ** (e - 8)"),
    ("subnormal scale", "m * 2.0 ** -9", "m * 2.0 ** -10"),
    ("mantissa step", "(1.0 + m / 8.0)", "(1.0 + m / 16.0)"),
    ("no NaN code", "if e == 0xF and m == 0x7:", "if False:"),
]


VERIFY_MUTATIONS = [
    ("causal limit off by one", "visible = np.clip(L - T + j + 1, 0, L)", "visible = np.clip(L - T + j, 0, L)"),
    ("tokens in reverse order", "visible = np.clip(L - T + j + 1, 0, L)", "visible = np.clip(L - j, 0, L)"),
    ("no causal limit", "visible = np.clip(L - T + j + 1, 0, L)", "visible = L"),
]

PROLOGUE_MUTATIONS = [
    ("eps outside the root", "np.sqrt(ms + eps)", "(np.sqrt(ms) + eps)"),
    ("sum for mean", "np.mean(x * x, axis=-1, keepdims=True)", "np.sum(x * x, axis=-1, keepdims=True)"),
    ("rope sine sign", "a * cos - b * sin", "a * cos + b * sin"),
    ("rope halves swapped", "[a * cos - b * sin, b * cos + a * sin]", "[b * cos + a * sin, a * cos - b * sin]"),
    ("ties away from even", "(_POS_CODES[hi] % 2 == 0)", "True"),
    ("scale max 240", "amax / E4M3_MAX", "amax / 240.0"),
    ("negative zero lost", "np.signbit(y)", "(y < 0)"),
    ("position is the length", "pos = L[:, None] - T + np.arange(T)[None, :]", "pos = L[:, None] - T + 1 + np.arange(T)[None, :]"),
    ("tokens in reverse", "pos = L[:, None] - T + np.arange(T)[None, :]", "pos = L[:, None] - 1 - np.arange(T)[None, :]"),
    ("key normed with query weight", "rms_norm(k, k_norm_w, eps)", "rms_norm(k, q_norm_w, eps)"),
    ("bf16 seven bits", "np.rint(np.ldexp(m, 8)), e - 8", "np.rint(np.ldexp(m, 7)), e - 7"),
]


@pytest.mark.parametrize("what,old,new", ASSIGN_MUTATIONS, ids=[m[0] for m in ASSIGN_MUTATIONS])
def test_assign_mutant_is_caught(what, old, new):
    mut = load_mutant("assign", old, new)
    with pytest.raises(Exception):
        pins.pins_assign(mut)


@pytest.mark.parametrize("what,old,new", ATTENTION_MUTATIONS, ids=[m[0] for m in ATTENTION_MUTATIONS])
def test_attention_mutant_is_caught(what, old, new):
    mut = load_mutant("attention", old, new)
    with pytest.raises(Exception):
        pins.pins_attention(mut, oracle.assign)
        pins.pins_attention_fp8(mut, oracle.e4m3)


@pytest.mark.parametrize("what,old,new", E4M3_MUTATIONS, ids=[m[0] for m in E4M3_MUTATIONS])
def test_e4m3_mutant_is_caught(what, old, new):
    mut = load_mutant("e4m3", old, new)
    with pytest.raises(Exception):
        pins.pins_e4m3(mut)


def test_prologue_pins_pass():
    pins.pins_prologue(oracle.prologue)


@pytest.mark.parametrize("what,old,new", PROLOGUE_MUTATIONS, ids=[m[0] for m in PROLOGUE_MUTATIONS])
def test_prologue_mutant_is_caught(what, old, new):
    mut = load_mutant("prologue", old, new)
    with pytest.raises(Exception):
        pins.pins_prologue(mut)


def test_verify_pins_pass():
    pins.pins_verify(oracle.attention)


@pytest.mark.parametrize("what,old,new", VERIFY_MUTATIONS, ids=[m[0] for m in VERIFY_MUTATIONS])
def test_verify_mutant_is_caught(what, old, new):
    mut = load_mutant("attention", old, new)
    with pytest.raises(Exception):
        pins.pins_verify(mut)
