"""Pins of the tile classification against brute force over dense masks."""
import numpy as np
import pytest

import workloads
from oracle import pack as OP
from oracle import tiles as OT


@pytest.mark.parametrize("BQ,BK", [(4, 2), (2, 4), (8, 8), (3, 5)])
def test_classification_is_conservative_and_complete(BQ, BK):
    rng = np.random.default_rng(BQ * 100 + BK)
    for _ in range(150):
        seqs, groups = workloads.random_small_forest(rng, n_seqs_max=7, len_max=9, vocab=3)
        p = OP.pack(seqs, groups)
        T, se = p["T"], p["se"]
        vis = OP.visibility_dense(p["par"])
        cnt = OT.tile_visible_counts(vis, BQ, BK)
        nq, nk = cnt.shape
        full = partial = empty = causal = 0
        for qt in range(nq):
            i0, i1 = qt * BQ, min(qt * BQ + BQ, T)
            for kt in range(nk):
                j0 = kt * BK
                if j0 > i1 - 1:
                    assert cnt[qt, kt] == 0  # nothing above the diagonal
                    continue
                causal += 1
                real_k = min(j0 + BK, T) - j0
                blk = np.zeros(BK, dtype=np.int64)
                blk[:real_k] = se[j0:j0 + real_k]
                if blk.max() <= i0:
                    empty += 1
                    assert cnt[qt, kt] == 0
                elif j0 + BK - 1 <= i0 and blk.min() >= i1:
                    full += 1
                    assert cnt[qt, kt] == (i1 - i0) * BK
                else:
                    partial += 1
        assert OT.tile_stats(se, T, BQ, BK) == (full, partial, empty, causal)
        assert causal == sum(min(nk, -(-min(qt * BQ + BQ, T) // BK)) for qt in range(nq))


@pytest.mark.parametrize("BQ,BK", [(4, 2), (8, 4), (3, 5)])
def test_per_query_tile_counts_brute_force(BQ, BK):
    """Per query tile: a key tile is counted non-empty iff it holds a visible
    pair, and full iff every one of its BQ' x BK pairs is visible (key columns
    past T count as not visible)."""
    rng = np.random.default_rng(7 * BQ + BK)
    for _ in range(120):
        seqs, groups = workloads.random_small_forest(rng, n_seqs_max=7, len_max=9, vocab=3, n_groups_max=3)
        p = OP.pack(seqs, groups)
        T = p["T"]
        cnt = OT.tile_visible_counts(OP.visibility_dense(p["par"]), BQ, BK)
        ne, fu = OT.tile_counts_per_qtile(p["se"], T, BQ, BK)
        for qt in range(cnt.shape[0]):
            rows = min(qt * BQ + BQ, T) - qt * BQ
            assert ne[qt] == int((cnt[qt] > 0).sum())
            assert fu[qt] == int((cnt[qt] == rows * BK).sum())
        f, pa, e, c = OT.tile_stats(p["se"], T, BQ, BK)
        assert (int(ne.sum()), int(fu.sum())) == (f + pa, f)
