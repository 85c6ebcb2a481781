"""Reference task-map builders (oracle; test infrastructure only).

Dynamic assigner, following the SGLang x HPC-Ops page, section "Scheduling
around live KV work", and the vLLM x HPC-Ops page, section "Solution:
per-step load-balanced decode scheduler", bullet "Assign":

1. every sequence is cut into uniform 64-token tiles; a partial last tile is
   one whole unit of work (ceil(L / 64) tiles);
2. the tile count is summed over all (KV head, request) pairs;
3. the total is divided by the number of persistent workgroups to get each
   bin's tile budget (rounded up, so every tile has a bin), and a
   minimum-work floor keeps the budget from dropping below ``min_tiles``;
4. pairs are walked head-major, batch-minor, and their tiles fill the current
   bin up to the budget before spilling into the next bin;
5. each maximal run of one pair inside one bin is one task descriptor.

Static split-KV policies, following the SGLang x HPC-Ops page, section
"Attention: load balancing for mixed-length decode" (and the "Challenge"
paragraph of the vLLM x HPC-Ops page): one fixed grid over (KV head, request,
split), with either a fixed split count or a fixed chunk size for every
request.

Task-map contract (all int32):

* header  ``T`` (total tiles), ``budget``, ``D`` (descriptors), ``U`` (bins
  that hold work);
* ``bin_offset[num_bins + 1]``: descriptors of bin b are
  ``desc[bin_offset[b] : bin_offset[b + 1]]``;
* ``desc[D][4]`` = (kv_head, request, token_begin, token_end);
* ``pair_first[H_kv * B]``, ``pair_count[H_kv * B]`` with pair index
  ``p = kv_head * B + request``: the descriptors of a pair are contiguous.
"""

from __future__ import annotations

import dataclasses

import numpy as np

TILE_TOKENS = 64


@dataclasses.dataclass
class TaskMap:
    T: int
    budget: int
    D: int
    U: int
    num_bins: int
    bin_offset: np.ndarray   # int32 [num_bins + 1]
    desc: np.ndarray         # int32 [D, 4]
    pair_first: np.ndarray   # int32 [H_kv * B]
    pair_count: np.ndarray   # int32 [H_kv * B]

    def header(self):
        return (self.T, self.budget, self.D, self.U)


def tiles_per_request(seq_lens) -> np.ndarray:
    """ceil(L / 64) for every request: the partial last tile counts as a whole one."""
    L = np.asarray(seq_lens, dtype=np.int64)
    if np.any(L < 0):
        raise ValueError("negative sequence length")
    return (L + TILE_TOKENS - 1) // TILE_TOKENS


def _finish(seq_lens, num_kv_heads, bins, T, budget):
    """Flatten per-bin lists of (kv_head, request, tile_lo, tile_hi) into the contract."""
    L = np.asarray(seq_lens, dtype=np.int64)
    B = len(L)
    num_bins = len(bins)
    bin_offset = np.zeros(num_bins + 1, dtype=np.int64)
    rows = []
    for b, items in enumerate(bins):
        bin_offset[b + 1] = bin_offset[b] + len(items)
        for (g, r, t0, t1) in items:
            rows.append((g, r, TILE_TOKENS * t0, min(TILE_TOKENS * t1, int(L[r]))))
    D = len(rows)
    desc = np.asarray(rows, dtype=np.int64).reshape(D, 4)
    npairs = num_kv_heads * B
    pair_count = np.zeros(npairs, dtype=np.int64)
    for (g, r, _, _) in rows:
        pair_count[g * B + r] += 1
    pair_first = np.concatenate([[0], np.cumsum(pair_count)[:-1]]) if npairs else np.zeros(0)
    # a pair's descriptors must be contiguous and start at pair_first
    for d, (g, r, _, _) in enumerate(rows):
        p = g * B + r
        assert pair_first[p] <= d < pair_first[p] + pair_count[p], "pair split is not contiguous"
    U = sum(1 for items in bins if items)
    return TaskMap(T=int(T), budget=int(budget), D=D, U=U, num_bins=num_bins,
                   bin_offset=bin_offset.astype(np.int32), desc=desc.astype(np.int32),
                   pair_first=np.asarray(pair_first, dtype=np.int32),
                   pair_count=pair_count.astype(np.int32))


def assign_dynamic(seq_lens, num_kv_heads: int, num_bins: int, min_tiles: int) -> TaskMap:
    """Budgeted greedy fill of ``num_bins`` bins in head-major, batch-minor order."""
    if num_bins < 1 or min_tiles < 1 or num_kv_heads < 1:
        raise ValueError("num_bins, min_tiles and num_kv_heads must be >= 1")
    n = tiles_per_request(seq_lens)
    B = len(n)
    T = int(n.sum()) * num_kv_heads                    # step 2: tiles of all pairs
    budget = max(-(-T // num_bins), min_tiles)         # step 3: ceil, then the floor
    bins = [[] for _ in range(num_bins)]
    b, fill = 0, 0
    for g in range(num_kv_heads):                      # step 4: head-major ...
        for r in range(B):                             # ... batch-minor
            tile, left = 0, int(n[r])
            while left > 0:
                if fill == budget:                     # bin full: spill to the next
                    b, fill = b + 1, 0
                take = min(left, budget - fill)
                bins[b].append((g, r, tile, tile + take))   # step 5: one run = one descriptor
                tile, left, fill = tile + take, left - take, fill + take
    assert b < num_bins
    return _finish(seq_lens, num_kv_heads, bins, T, budget)


def assign_static_splits(seq_lens, num_kv_heads: int, splits: int) -> TaskMap:
    """Fixed split count S: a grid of H_kv * B * S bins, one per (pair, split).

    Pair p's n tiles are cut into S ranges of ceil(n / S) tiles; range s goes
    to bin ``p * S + s``; empty ranges produce no descriptor.  ``budget``
    records S.
    """
    if splits < 1:
        raise ValueError("splits must be >= 1")
    n = tiles_per_request(seq_lens)
    B = len(n)
    bins = [[] for _ in range(num_kv_heads * B * splits)]
    for g in range(num_kv_heads):
        for r in range(B):
            p = g * B + r
            c = -(-int(n[r]) // splits)
            for s in range(splits):
                lo, hi = s * c, min((s + 1) * c, int(n[r]))
                if lo < hi:
                    bins[p * splits + s].append((g, r, lo, hi))
    return _finish(seq_lens, num_kv_heads, bins, int(n.sum()) * num_kv_heads, splits)


def assign_static_chunk(seq_lens, num_kv_heads: int, chunk_tiles: int,
                        max_pages_per_seq: int) -> TaskMap:
    """Fixed chunk size C tiles: every pair gets ceil(max_pages_per_seq / C) bins.

    The grid is sized for the longest request the cache admits, so short
    requests leave trailing bins empty.  Bin ``p * S + s`` holds tiles
    ``[s*C, min((s+1)*C, n))`` when that range is nonempty.  ``budget``
    records C.
    """
    if chunk_tiles < 1 or max_pages_per_seq < 1:
        raise ValueError("chunk_tiles and max_pages_per_seq must be >= 1")
    n = tiles_per_request(seq_lens)
    if len(n) and n.max() > max_pages_per_seq:
        raise ValueError("a request is longer than max_pages_per_seq pages")
    B = len(n)
    S = -(-max_pages_per_seq // chunk_tiles)
    bins = [[] for _ in range(num_kv_heads * B * S)]
    for g in range(num_kv_heads):
        for r in range(B):
            p = g * B + r
            for s in range(S):
                lo, hi = s * chunk_tiles, min((s + 1) * chunk_tiles, int(n[r]))
                if lo < hi:
                    bins[p * S + s].append((g, r, lo, hi))
    return _finish(seq_lens, num_kv_heads, bins, int(n.sum()) * num_kv_heads, chunk_tiles)
