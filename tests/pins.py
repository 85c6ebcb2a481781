"""Pins for the CPU oracle: facts fixed by the pages and by mathematics.

Every ``pins_*`` function takes the oracle module under test as an argument
and raises AssertionError when a pin fails, so the same pins run against the
real oracle (tests/test_oracle_*.py) and against copies with a planted
mistake (tests/test_oracle_mutations.py), which they must reject.

Nothing here re-types the oracle's formulas: task maps are pinned by
hand-worked maps, a tile-by-tile brute-force walk and structural invariants;
attention by pure-Python loops over unpaged arrays, torch's fp64 SDPA, split
invariance and closed forms; e4m3 by torch's float8_e4m3fn conversion.
"""

from __future__ import annotations

import math
import os
import struct

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# task maps
# --------------------------------------------------------------------------

def load_golden_taskmaps(path=os.path.join(GOLDEN, "taskmaps.txt")):
    sections, cur = [], None
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        if line.startswith("["):
            name = line.strip("[]").split()
            cur = {"policy": name[0], "params": dict(kv.split("=") for kv in name[1:]),
                   "desc": []}
            sections.append(cur)
            continue
        key, val = line.split(":", 1)
        toks = val.split()
        if key == "desc":
            cur["desc"].append([int(t) for t in toks])
        elif key == "bin_offset":
            cur["bin_offset"] = toks
        else:
            cur[key] = [int(t) for t in toks]
    for s in sections:
        D = s["header"][2]
        nb = s["num_bins"][0]
        toks = s["bin_offset"]
        if toks[-1] == "...":
            vals = [int(t) for t in toks[:-1]]
            vals += [D] * (nb + 1 - len(vals))
        else:
            vals = [int(t) for t in toks]
        assert len(vals) == nb + 1
        s["bin_offset"] = vals
    return sections


def build_from_golden(asg, sec):
    lens, H = sec["lengths"], sec["kv_heads"][0]
    p = sec["params"]
    if sec["policy"] == "dynamic":
        return asg.assign_dynamic(lens, H, int(p["W"]), int(p["F"]))
    if sec["policy"] == "static_splits":
        return asg.assign_static_splits(lens, H, int(p["S"]))
    if sec["policy"] == "static_chunk":
        return asg.assign_static_chunk(lens, H, int(p["C"]), int(p["max_pages"]))
    raise ValueError(sec["policy"])


def assert_taskmap_equals(tm, header, num_bins, bin_offset, desc, pair_first, pair_count):
    assert tuple(int(x) for x in tm.header()) == tuple(header), (tm.header(), header)
    assert tm.num_bins == num_bins
    assert np.array_equal(np.asarray(tm.bin_offset), np.asarray(bin_offset))
    assert np.array_equal(np.asarray(tm.desc).reshape(-1, 4), np.asarray(desc).reshape(-1, 4))
    assert np.array_equal(np.asarray(tm.pair_first), np.asarray(pair_first))
    assert np.array_equal(np.asarray(tm.pair_count), np.asarray(pair_count))


def tilewalk_dynamic(seq_lens, H, W, F):
    """Brute force: place every 64-token tile one at a time.

    The budget is found by search (the smallest value >= F with W bins of it
    holding every tile), and a new descriptor starts whenever the
    (bin, pair) of the next tile differs from the previous one's.
    """
    B = len(seq_lens)
    flat = []
    for g in range(H):
        for r in range(B):
            ntiles = 0
            while ntiles * 64 < seq_lens[r]:
                ntiles += 1
            flat += [(g, r, t) for t in range(ntiles)]
    T = len(flat)
    budget = F
    while budget * W < T:
        budget += 1
    desc, bins_of_desc = [], []
    for i, (g, r, t) in enumerate(flat):
        b = i // budget
        if desc and bins_of_desc[-1] == b and desc[-1][0] == g and desc[-1][1] == r:
            desc[-1][3] = min(64 * (t + 1), seq_lens[r])
        else:
            desc.append([g, r, 64 * t, min(64 * (t + 1), seq_lens[r])])
            bins_of_desc.append(b)
    D = len(desc)
    bin_offset = [sum(1 for bb in bins_of_desc if bb < b) for b in range(W + 1)]
    U = len(set(bins_of_desc))
    pair_count = [0] * (H * B)
    pair_first = [None] * (H * B)
    for d, (g, r, _, _) in enumerate(desc):
        p = g * B + r
        pair_count[p] += 1
        if pair_first[p] is None:
            pair_first[p] = d
    # pairs with no descriptor: first index of the next pair that has one
    nxt = D
    for p in reversed(range(H * B)):
        if pair_first[p] is None:
            pair_first[p] = nxt
        else:
            nxt = pair_first[p]
    return dict(header=(T, budget, D, U), num_bins=W, bin_offset=bin_offset, desc=desc,
                pair_first=pair_first, pair_count=pair_count)


def check_taskmap_invariants(tm, seq_lens, H, policy="dynamic"):
    """Structural invariants that any correct map of the stated policy has."""
    L = [int(x) for x in seq_lens]
    B = len(L)
    T, budget, D, U = tm.header()
    desc = np.asarray(tm.desc).reshape(-1, 4)
    bo = np.asarray(tm.bin_offset)
    assert desc.shape[0] == D
    assert bo[0] == 0 and bo[-1] == D and np.all(np.diff(bo) >= 0)
    assert T == H * sum((x + 63) // 64 for x in L)
    # every token of every pair covered exactly once, ranges tile-aligned
    cover = {}
    for g, r, a, b in desc:
        assert 0 <= g < H and 0 <= r < B
        assert a % 64 == 0 and a < b <= L[r]
        assert b == L[r] or b % 64 == 0
        cover.setdefault((g, r), []).append((a, b))
    for g in range(H):
        for r in range(B):
            rs = sorted(cover.get((g, r), []))
            pos = 0
            for a, b in rs:
                assert a == pos, "gap or overlap"
                pos = b
            assert pos == L[r]
    # per-bin tile counts
    bin_tiles = []
    for bidx in range(tm.num_bins):
        n = 0
        for g, r, a, b in desc[bo[bidx]:bo[bidx + 1]]:
            n += (b + 63) // 64 - a // 64
        bin_tiles.append(n)
    used = [i for i, n in enumerate(bin_tiles) if n > 0]
    assert U == len(used)
    if policy == "dynamic":
        assert U <= tm.num_bins                              # I7
        assert used == list(range(U))                         # bins fill from 0
        for i in range(U - 1):
            assert bin_tiles[i] == budget                     # I2
        if U:
            assert 0 < bin_tiles[U - 1] <= budget
        nonempty_pairs = H * sum(1 for x in L if x > 0)
        assert D <= nonempty_pairs + max(U - 1, 0)            # I4
        # I3: sorted by flat (head-major, batch-minor, tile) index
        flat = [(g * B + r, a) for g, r, a, b in desc]
        assert flat == sorted(flat)
    # I5 / I6: pair splits contiguous; count = distinct bins touched
    pf, pc = np.asarray(tm.pair_first), np.asarray(tm.pair_count)
    bin_of = np.searchsorted(bo, np.arange(D), side="right") - 1
    for g in range(H):
        for r in range(B):
            p = g * B + r
            idx = [d for d in range(D) if desc[d][0] == g and desc[d][1] == r]
            assert pc[p] == len(idx)
            if idx:
                assert idx == list(range(pf[p], pf[p] + pc[p]))
                assert len(set(bin_of[idx])) == pc[p]


def random_length_cases(seed, n_cases):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n_cases):
        B = int(rng.integers(1, 40))
        H = int(rng.choice([1, 2, 3, 8]))
        W = int(rng.choice([1, 2, 7, 16, 64, 256]))
        F = int(rng.choice([1, 4, 16]))
        kind = rng.integers(0, 4)
        if kind == 0:
            L = rng.integers(0, 3000, size=B)
        elif kind == 1:
            L = 64 * rng.integers(0, 20, size=B)             # exact multiples, zeros
        elif kind == 2:
            L = np.exp(rng.uniform(0, np.log(20000), size=B)).astype(int)
        else:
            L = rng.integers(1, 3, size=B)                    # L in {1, 2}
        cases.append(([int(x) for x in L], H, W, F))
    return cases


def pins_assign(asg):
    # hand-worked maps
    for sec in load_golden_taskmaps():
        tm = build_from_golden(asg, sec)
        assert_taskmap_equals(tm, sec["header"], sec["num_bins"][0], sec["bin_offset"],
                              sec["desc"], sec["pair_first"], sec["pair_count"])
    # brute-force tile walk and invariants
    for L, H, W, F in random_length_cases(1234, 60):
        tm = asg.assign_dynamic(L, H, W, F)
        ref = tilewalk_dynamic(L, H, W, F)
        assert_taskmap_equals(tm, **ref)
        check_taskmap_invariants(tm, L, H, "dynamic")
    # closed form: uniform 32 x 4096, 8 KV heads, W = 256 -> one pair per bin
    L = [4096] * 32
    tm = asg.assign_dynamic(L, 8, 256, 4)
    assert tm.header() == (16384, 64, 256, 256)
    for b in range(256):
        assert list(tm.desc[b]) == [b // 32, b % 32, 0, 4096]
    assert np.all(tm.pair_count == 1) and np.array_equal(tm.pair_first, np.arange(256))
    # ... and W = 512 gives two equal halves per pair
    tm = asg.assign_dynamic(L, 8, 512, 4)
    assert tm.header() == (16384, 32, 512, 512)
    assert np.all(tm.pair_count == 2)
    assert [list(x) for x in tm.desc[:2]] == [[0, 0, 0, 2048], [0, 0, 2048, 4096]]
    # T <= F: everything in bin 0
    tm = asg.assign_dynamic([10, 70, 0, 5], 1, 256, 16)
    assert tm.header() == (4, 16, 3, 1)
    assert np.array_equal(tm.pair_count, [1, 1, 0, 1])
    # empty batch of zero lengths
    tm = asg.assign_dynamic([0, 0], 2, 8, 4)
    assert tm.header() == (0, 4, 0, 0) and tm.desc.shape == (0, 4)
    # static maps: invariants on random inputs
    for L, H, W, F in random_length_cases(99, 25):
        for S in (1, 2, 5):
            tm = asg.assign_static_splits(L, H, S)
            check_taskmap_invariants(tm, L, H, "static")
            assert tm.num_bins == H * len(L) * S
            assert np.all(tm.pair_count <= S)
        mp = max(1, max((x + 63) // 64 for x in L))
        for C in (1, 3, 8):
            tm = asg.assign_static_chunk(L, H, C, mp + 2)
            check_taskmap_invariants(tm, L, H, "static")
            assert tm.num_bins == H * len(L) * (-(-(mp + 2) // C))
            for g, r, a, b in tm.desc:
                assert (b + 63) // 64 - a // 64 <= C and (a // 64) % C == 0


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def bf16_bits_to_float_struct(bits: int) -> float:
    """Independent bf16 widening: pack the 16 bits above 16 zero bits."""
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def to_bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_tiny_paged(seed, lengths, H, G, D, page=64, nan_tail=True):
    """Logical per-pair K/V (bf16 bits) and the same rows scattered into pages."""
    g = torch.Generator().manual_seed(seed)
    B = len(lengths)
    q = to_bf16_bits(torch.randn(B, H * G, D, generator=g))
    Klog = [[to_bf16_bits(torch.randn(L, D, generator=g)) for _ in range(H)] for L in lengths]
    Vlog = [[to_bf16_bits(torch.randn(L, D, generator=g)) for _ in range(H)] for L in lengths]
    npages = [(L + page - 1) // page for L in lengths]
    P = sum(npages)
    rng = np.random.default_rng(seed)
    perm = rng.permutation(P)
    table = np.zeros((B, max(1, max(npages))), dtype=np.int32)
    off = 0
    for r, n in enumerate(npages):
        table[r, :n] = perm[off:off + n]
        off += n
    fill = 0x7FC0 if nan_tail else 0
    kc = np.full((P, H, page, D), fill, dtype=np.uint16)
    vc = np.full((P, H, page, D), fill, dtype=np.uint16)
    for r, L in enumerate(lengths):
        for h in range(H):
            for t in range(L):
                kc[table[r, t // page], h, t % page] = Klog[r][h][t]
                vc[table[r, t // page], h, t % page] = Vlog[r][h][t]
    return q, Klog, Vlog, kc, vc, table


def brute_force_attention(q_bits, Klog, Vlog, lengths, H, G, sm_scale):
    """Pure-Python loops over the logical (unpaged) rows."""
    B, Hq, D = q_bits.shape
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for r in range(B):
        for h in range(Hq):
            kvh = h // G
            qv = [bf16_bits_to_float_struct(x) for x in q_bits[r, h]]
            scores = []
            for t in range(lengths[r]):
                kv = [bf16_bits_to_float_struct(x) for x in Klog[r][kvh][t]]
                scores.append(sm_scale * math.fsum(a * b for a, b in zip(qv, kv)))
            if not scores:
                lse[r, h] = -math.inf
                continue
            m = max(scores)
            ws = [math.exp(s - m) for s in scores]
            tot = math.fsum(ws)
            for d in range(D):
                acc = math.fsum(ws[t] * bf16_bits_to_float_struct(Vlog[r][kvh][t][d])
                                for t in range(lengths[r]))
                out[r, h, d] = acc / tot
            lse[r, h] = m + math.log(tot)
    return out, lse


def sdpa_reference(q, K, V, sm_scale):
    """torch's fp64 scaled-dot-product attention for one query row set."""
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, :, None, :]         # [1, G, 1, D]
    kt = torch.from_numpy(np.ascontiguousarray(K))[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(np.ascontiguousarray(V))[None, None].expand(1, q.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(),
                                                         scale=sm_scale)
    return o[0, :, 0, :].numpy()


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


def pins_attention(att, asg):
    sm = 1.0 / math.sqrt(16.0)
    # 1. paged oracle == unpaged pure-Python brute force (with NaN in unused slots)
    lengths, H, G, D = [1, 70, 130], 2, 2, 16
    q, Klog, Vlog, kc, vc, table = make_tiny_paged(7, lengths, H, G, D)
    out, lse = att.paged_decode_attention(att.bf16_bits_to_f64(q), kc, vc, table, lengths, H, sm)
    bo, bl = brute_force_attention(q, Klog, Vlog, lengths, H, G, sm)
    assert rel_err(out, bo) < 1e-12, rel_err(out, bo)
    assert np.max(np.abs(lse - bl)) < 1e-12
    # 2. against torch's fp64 SDPA at the real head_dim with GQA 8/2
    lengths, H, G, D = [300, 5, 64, 129], 2, 4, 128
    q, Klog, Vlog, kc, vc, table = make_tiny_paged(8, lengths, H, G, D)
    sm128 = 1.0 / math.sqrt(128.0)
    out, lse = att.paged_decode_attention(att.bf16_bits_to_f64(q), kc, vc, table, lengths, H,
                                          sm128)
    for r, L in enumerate(lengths):
        for g in range(H):
            ref = sdpa_reference(att.bf16_bits_to_f64(q[r, g * G:(g + 1) * G]),
                                 att.bf16_bits_to_f64(Klog[r][g]),
                                 att.bf16_bits_to_f64(Vlog[r][g]), sm128)
            assert rel_err(out[r, g * G:(g + 1) * G], ref) < 1e-12
    # 3. split invariance: random ranges, single tokens, and task-map splits
    qf = att.bf16_bits_to_f64(q)
    rng = np.random.default_rng(3)
    for r, L in enumerate(lengths):
        K = att.bf16_bits_to_f64(Klog[r][1])
        V = att.bf16_bits_to_f64(Vlog[r][1])
        full = att.attend_range(qf[r, G:2 * G], K, V, sm128)
        cuts = sorted(set([0, L] + list(rng.integers(0, L + 1, size=4))))
        parts = [att.attend_range(qf[r, G:2 * G], K[a:b], V[a:b], sm128)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        merged = att.combine(parts)
        assert rel_err(merged[0], full[0]) < 1e-12 and np.max(np.abs(merged[1] - full[1])) < 1e-12
        if L <= 130:
            singles = [att.attend_range(qf[r, G:2 * G], K[t:t + 1], V[t:t + 1], sm128)
                       for t in range(L)]
            assert rel_err(att.combine(singles)[0], full[0]) < 1e-12
    tm = asg.assign_dynamic(lengths, H, 5, 1)
    assert tm.D > len(lengths) * H          # some pairs really are split
    split = att.split_decode_attention(qf, kc, vc, table, lengths, H, sm128, tm.desc)
    assert rel_err(split, out) < 1e-12
    # 4. closed forms
    K = att.bf16_bits_to_f64(Klog[1][0])
    V = att.bf16_bits_to_f64(Vlog[1][0])
    o, l = att.attend_range(qf[1, :G], K[:1], V[:1], sm128)
    assert np.array_equal(o, np.repeat(V[:1], G, axis=0))                      # L = 1: v0
    assert np.allclose(l, sm128 * (qf[1, :G] @ K[0]), rtol=0, atol=1e-13)
    o, l = att.attend_range(np.zeros((G, 128)), K, V, sm128)
    assert rel_err(o, np.repeat(V.mean(0, keepdims=True), G, 0)) < 1e-12       # q = 0: mean
    assert np.allclose(l, np.log(K.shape[0]), atol=1e-13)
    o, _ = att.attend_range(qf[1, :G], np.repeat(K[:1], 5, 0), V, sm128)
    assert rel_err(o, np.repeat(V.mean(0, keepdims=True), G, 0)) < 1e-12       # equal keys
    Kp = K.copy()
    Kp[3] = 400.0 * qf[1, 0] / np.linalg.norm(qf[1, 0])                        # one dominant key
    o, _ = att.attend_range(qf[1, :1], Kp, V, sm128)
    assert rel_err(o[0], V[3]) < 1e-12
    u = rng.standard_normal(128)
    o1, l1 = att.attend_range(qf[1, :G], K, V, sm128)
    o2, l2 = att.attend_range(qf[1, :G], K + u, V, sm128)                     # shift keys
    assert rel_err(o2, o1) < 1e-12
    assert np.allclose(l2 - l1, sm128 * (qf[1, :G] @ u), atol=1e-12)
    # 5. zero-length request: zero output, no mass
    o, l = att.attend_range(qf[1, :G], K[:0], V[:0], sm128)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def pins_attention_fp8(att, e4m3_mod):
    """FP8 gather = torch's e4m3 decode times the per-(token, head) scale."""
    g = torch.Generator().manual_seed(11)
    P, H, D = 5, 2, 128
    x = torch.randn(P, H, 64, D, generator=g) * 30
    codes = torch.clamp(x, -448, 448).to(torch.float8_e4m3fn)
    scale = 0.01 + 0.09 * torch.rand(P, H, 64, generator=g)
    table = np.array([[3, 1], [0, 4]], dtype=np.int32)
    for r, L in ((0, 100), (1, 65)):
        for h in range(H):
            got = att.gather_pair_kv(codes.view(torch.uint8).numpy(), table[r], h, L,
                                     "fp8_e4m3", scale.numpy())
            t = np.arange(L)
            ref = (codes.to(torch.float64).numpy()[table[r][t // 64], h, t % 64]
                   * scale.double().numpy()[table[r][t // 64], h, t % 64][:, None])
            assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# e4m3
# --------------------------------------------------------------------------

def pins_e4m3(mod):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = mod.decode(np.arange(256, dtype=np.uint8))
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref)
    assert set(np.flatnonzero(nan_ref)) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan_ref], ref[~nan_ref])
    assert mod.decode(np.array([0x7E]))[0] == 448.0
    assert mod.decode(np.array([0x01]))[0] == 2.0 ** -9
    assert mod.decode(np.array([0x08]))[0] == 2.0 ** -6
    assert mod.decode(np.array([0x38]))[0] == 1.0
    assert mod.decode(np.array([0xB8]))[0] == -1.0


# --------------------------------------------------------------------------
# fused attention prologue
# --------------------------------------------------------------------------

def _brute_prologue(qkv, seq_lens, Hq, Hkv, qw, kw, eps, cos_sin):
    """Per-element loops with the math module: RMSNorm, then rotate-half RoPE."""
    B = len(qkv)
    D = len(cos_sin[0])
    h = D // 2
    out = {"q": [], "k": [], "v": []}
    for r in range(B):
        p = max(0, min(int(seq_lens[r]) - 1, len(cos_sin) - 1))
        for head in range(Hq + 2 * Hkv):
            x = [float(qkv[r][head * D + i]) for i in range(D)]
            if head >= Hq + Hkv:
                out["v"].append(x)
                continue
            w = qw if head < Hq else kw
            ms = sum(t * t for t in x) / D
            y = [x[i] / math.sqrt(ms + eps) * float(w[i]) for i in range(D)]
            z = [0.0] * D
            for i in range(h):
                c, s = float(cos_sin[p][i]), float(cos_sin[p][h + i])
                z[i] = y[i] * c - y[h + i] * s
                z[h + i] = y[h + i] * c + y[i] * s
            out["q" if head < Hq else "k"].append(z)
    return {k: np.array(v).reshape(B, -1, D) for k, v in out.items()}


def pins_prologue(pro):
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    rng = np.random.default_rng(5)
    # 1. RMSNorm is torch's rms_norm (fp64), eps inside the square root
    x = rng.normal(size=(3, 5, 128)) * 3
    w = 1 + 0.1 * rng.normal(size=128)
    for eps in (1e-6, 0.5):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w),
                                           eps).numpy()
        assert np.allclose(pro.rms_norm(x, w, eps), ref, rtol=1e-12, atol=1e-12)
    # 2. RoPE is the rotate-half convention of HF transformers' apply_rotary_pos_emb
    theta = rng.uniform(-10, 10, size=(3, 64))
    cos, sin = np.cos(theta), np.sin(theta)
    q = rng.normal(size=(3, 4, 128))
    c2 = torch.from_numpy(np.concatenate([cos, cos], -1))[:, None, :]
    s2 = torch.from_numpy(np.concatenate([sin, sin], -1))[:, None, :]
    qt = torch.from_numpy(q)[:, :, None, :]
    ref, _ = apply_rotary_pos_emb(qt, qt, c2, s2, unsqueeze_dim=1)
    got = pro.rope_rotate_half(q, cos[:, None, :], sin[:, None, :])
    assert np.allclose(got, ref[:, :, 0].numpy(), rtol=1e-12, atol=1e-12)
    # a quarter turn maps dim i onto dim i + 64; pair norms are kept
    e0 = np.zeros((1, 128))
    e0[0, 3] = 1.0
    qt_ = pro.rope_rotate_half(e0, np.zeros((1, 64)), np.ones((1, 64)))
    assert qt_[0, 67] == 1.0 and np.sum(np.abs(qt_)) == 1.0
    pn = got[..., :64] ** 2 + got[..., 64:] ** 2
    assert np.allclose(pn, q[..., :64] ** 2 + q[..., 64:] ** 2)
    # 3. e4m3 rounding: torch's float8_e4m3fn cast (nearest, ties to even) in range
    y = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(size=20000) * 0.01,
                        [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -(2.0 ** -10), 3 * 2.0 ** -10]])
    ref = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(pro.e4m3_round(y.astype(np.float32).astype(np.float64)), ref)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    from oracle.e4m3 import decode
    assert np.array_equal(pro.e4m3_round(decode(finite)), finite)      # every code round-trips
    # 4. row quantization: the row maximum maps to +-448 exactly; zero row -> scale 1, codes 0
    rows = rng.normal(size=(6, 128))
    rows[2] = 0
    codes, scale, _ = pro.quantize_rows_e4m3(rows)
    vals = decode(codes) * scale[:, None]
    assert np.allclose(np.abs(vals).max(1)[[0, 1, 3, 4, 5]], np.abs(rows).max(1)[[0, 1, 3, 4, 5]],
                       rtol=1e-15)
    assert scale[2] == 1.0 and not np.any(codes[2] & 0x7F)
    nz = [0, 1, 3, 4, 5]
    assert np.all(np.abs(decode(codes[nz])).max(1) == 448.0)      # the full e4m3 range is used
    assert np.all(np.abs(vals - rows) <= np.abs(rows) / 16 + scale[:, None] * 2.0 ** -9)
    # 5. BF16 rounding: torch's fp32 -> bf16 cast (nearest, ties to even)
    f = np.concatenate([rng.normal(size=5000).astype(np.float32),
                        np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)], np.float32)])
    ref = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(pro.bf16_round(f.astype(np.float64)), ref)
    # 6. the whole step against per-element loops on a tiny case (D = 8)
    D, Hq, Hkv = 8, 3, 1
    cs_t = rng.uniform(-3, 3, size=(5, D // 2))
    cos_sin = np.concatenate([np.cos(cs_t), np.sin(cs_t)], -1)
    qkv = rng.normal(size=(4, (Hq + 2 * Hkv) * D))
    L = [1, 3, 9, 0]                       # position 8 is past the table: its last row
    qw, kw = rng.normal(size=D), rng.normal(size=D)
    got = pro.prologue(qkv, L, Hq, Hkv, qw, kw, 1e-5, cos_sin)
    ref = _brute_prologue(qkv, L, Hq, Hkv, qw, kw, 1e-5, cos_sin)
    for key in ("q", "k", "v"):
        assert np.allclose(got[key], ref[key], rtol=1e-12, atol=1e-12), key
    assert list(got["pos"]) == [0, 2, 8, -1]
    # T = 3 new tokens per request at positions L - 3 + j
    qkv3 = rng.normal(size=(4, 3, (Hq + 2 * Hkv) * D))
    got3 = pro.prologue(qkv3, L, Hq, Hkv, qw, kw, 1e-5, cos_sin)
    for j in range(3):
        Lj = [x - 3 + j + 1 for x in L]        # a table row lookup at Lj - 1 = L - 3 + j
        ref = _brute_prologue(qkv3[:, j], Lj, Hq, Hkv, qw, kw, 1e-5, cos_sin)
        for key in ("q", "k", "v"):
            ok = np.array([x - 3 + j >= 0 for x in L])
            assert np.allclose(got3[key][ok, j], ref[key][ok], rtol=1e-12, atol=1e-12), (key, j)
    assert got3["pos"].tolist() == [[-1, -1, 0], [0, 1, 2], [6, 7, 8], [-1, -1, -1]]


# --------------------------------------------------------------------------
# multi-token verification (causal attention of T query tokens per request)
# --------------------------------------------------------------------------

def pins_verify(att):
    """Against torch's fp64 SDPA with an explicit causal mask over unpaged rows."""
    H, G, D, T = 2, 3, 16, 4
    lengths = [1, 3, 4, 70, 129, 200]
    q1, Klog, Vlog, kc, vc, table = make_tiny_paged(21, lengths, H, G, D)
    g = torch.Generator().manual_seed(22)
    qb = to_bf16_bits(torch.randn(len(lengths), T, H * G, D, generator=g))
    q = att.bf16_bits_to_f64(qb)
    sm = 1.0 / math.sqrt(D)
    out, lse = att.paged_verify_attention(q, kc, vc, table, lengths, H, sm)
    for r, L in enumerate(lengths):
        for h in range(H):
            K = att.bf16_bits_to_f64(np.asarray(Klog[r][h]))
            V = att.bf16_bits_to_f64(np.asarray(Vlog[r][h]))
            qr = q[r, :, h * G:(h + 1) * G]                        # [T, G, D]
            qt = torch.from_numpy(np.ascontiguousarray(qr.transpose(1, 0, 2)))[None]   # [1,G,T,D]
            kt = torch.from_numpy(K)[None, None].expand(1, G, -1, -1).contiguous()
            vt = torch.from_numpy(V)[None, None].expand(1, G, -1, -1).contiguous()
            pos = np.arange(T)[:, None] + L - T                    # query positions
            mask = torch.from_numpy(np.arange(L)[None, :] <= pos)  # [T, L]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qt, kt, vt, attn_mask=mask, scale=sm)[0].numpy().transpose(1, 0, 2)
            for j in range(T):
                got = out[r, j, h * G:(h + 1) * G]
                if L - T + j < 0:                                  # no visible position
                    assert np.all(got == 0) and np.all(np.isneginf(lse[r, j, h * G:(h + 1) * G]))
                else:
                    assert rel_err(got, ref[j]) < 1e-12, (r, h, j)
    # one query token is plain decode
    o1, l1 = att.paged_verify_attention(q[:, :1], kc, vc, table, lengths, H, sm)
    o0, l0 = att.paged_decode_attention(q[:, 0], kc, vc, table, lengths, H, sm)
    assert np.array_equal(o1[:, 0], o0) and np.array_equal(l1[:, 0], l0)
