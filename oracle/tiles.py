"""Oracle: classification of (query-tile, key-tile) pairs from subtree ends.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Key j is visible to query i iff j <= i < se[j] (ancestor-or-self in preorder:
the descendants of j are exactly the packed indices in (j, se[j]); the
"Trie packing" page Step 2 and "Tree Training" §3.2). Tiles are BQ query rows
by BK key columns. Key columns at or past T are padding with se = 0 (never
visible). Query tile rows are clipped to T.

For a causal tile (first key <= last query row) with i0 = first row,
i1 = one past its last real row, j0 = first key, j1 = j0 + BK:
  empty    if max se over the tile's keys <= i0      (no query in any subtree)
  full     if j1 - 1 <= i0 and min se >= i1          (every pair visible)
  partial  otherwise
Non-causal tiles (j0 > i1 - 1) are not counted at all. The rule is
conservative: an empty tile has no visible pair and a full tile has only
visible pairs; a partial tile may have any number.
"""
from __future__ import annotations

import numpy as np


def tile_stats(se, T, BQ, BK):
    se = np.asarray(se, dtype=np.int64)
    nq = -(-T // BQ)
    nk = -(-T // BK)
    pad = np.zeros(nk * BK, dtype=np.int64)
    pad[:T] = se[:T]
    full = partial = empty = causal = 0
    for qt in range(nq):
        i0 = qt * BQ
        i1 = min(i0 + BQ, T)
        for kt in range(nk):
            j0 = kt * BK
            j1 = j0 + BK
            if j0 > i1 - 1:
                continue
            causal += 1
            blk = pad[j0:j1]
            if blk.max() <= i0:
                empty += 1
            elif j1 - 1 <= i0 and blk.min() >= i1:
                full += 1
            else:
                partial += 1
    return full, partial, empty, causal


def tile_visible_counts(vis, BQ, BK):
    """Brute force: number of visible pairs in every tile of a dense mask."""
    T = vis.shape[0]
    nq, nk = -(-T // BQ), -(-T // BK)
    out = np.zeros((nq, nk), dtype=np.int64)
    for qt in range(nq):
        for kt in range(nk):
            out[qt, kt] = vis[qt * BQ:(qt + 1) * BQ, kt * BK:(kt + 1) * BK].sum()
    return out


def tile_counts_per_qtile(se, T, BQ, BK):
    """Per query tile (rows [qt*BQ, min(qt*BQ+BQ, T))): the number of causal
    key tiles that are non-empty and the number that are full, under the
    rule of tile_stats. Returns two int64 arrays of length ceil(T / BQ)."""
    se = np.asarray(se, dtype=np.int64)
    nq = -(-T // BQ)
    nk = -(-T // BK)
    pad = np.zeros(nk * BK, dtype=np.int64)
    pad[:T] = se[:T]
    nonempty = np.zeros(nq, dtype=np.int64)
    full = np.zeros(nq, dtype=np.int64)
    for qt in range(nq):
        i0 = qt * BQ
        i1 = min(i0 + BQ, T)
        for kt in range(nk):
            j0 = kt * BK
            j1 = j0 + BK
            if j0 > i1 - 1:
                continue
            blk = pad[j0:j1]
            if blk.max() <= i0:
                continue
            nonempty[qt] += 1
            if j1 - 1 <= i0 and blk.min() >= i1:
                full[qt] += 1
    return nonempty, full
