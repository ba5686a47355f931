"""Pins of the partition planner oracle: optimality of the cut stage by brute
force on tiny trees, the single-parent and capacity invariants, closed-form
special cases. CPU only."""
import numpy as np
import pytest

import workloads
from oracle import pack as OP
from oracle import partition as OPT


def _tiny_tree(rng, n):
    par = [-1] + [int(rng.integers(0, v)) for v in range(1, n)]
    # relabel to preorder so that parents come first and subtrees are contiguous
    children = [[] for _ in range(n)]
    for v in range(1, n):
        children[par[v]].append(v)
    order, stack = [], [0]
    while stack:
        v = stack.pop()
        order.append(v)
        stack.extend(reversed(children[v]))
    new = {v: i for i, v in enumerate(order)}
    npar = [-1] * n
    for v in range(1, n):
        npar[new[v]] = new[par[v]]
    lens = [int(x) for x in rng.integers(1, 9, n)]
    return lens, npar


@pytest.mark.parametrize("seed", range(40))
def test_cut_stage_is_optimal_for_connected_pieces(seed):
    rng = np.random.default_rng(seed)
    lens, par = _tiny_tree(rng, int(rng.integers(2, 10)))
    C = int(rng.integers(max(lens), sum(lens) + 1))
    _, tokens = OPT.cut(lens, par, C)
    assert len(tokens) == OPT.min_connected_pieces_brute(lens, par, C)


def _check_plan(lens, par, C, r):
    n = len(lens)
    part = r["node_part"]
    P = len(r["part_tokens"])
    assert sorted(set(part.tolist())) == list(range(P))
    for b in range(P):
        assert r["part_tokens"][b] == sum(lens[v] for v in range(n) if part[v] == b) <= C
    for v in range(n):
        p = par[v]
        if p < 0:
            assert r["part_parent"][part[v]] == -1
        elif part[p] != part[v]:
            assert r["part_parent"][part[v]] == part[p]      # exactly one parent partition
            assert r["part_cut"][part[v]] == p               # and one cut node (one gateway)
        piece = r["piece"][v]
        assert piece == v or r["piece"][p] == piece            # pieces are connected
    assert P >= -(-sum(lens) // C)


@pytest.mark.parametrize("seed", range(30))
def test_plan_invariants_random_forests(seed):
    seqs, groups = workloads.random_forest(seed, [300, 120, 45], max_depth=5, seg_lo=1, seg_hi=60)
    po = OP.pack(seqs, groups)
    lens = (po["node_end"] - po["node_start"]).tolist()
    par = po["node_parent"].tolist()
    for C in (max(lens), 2 * max(lens), 150, 10 ** 6):
        if C < max(lens):
            continue
        _check_plan(lens, par, C, OPT.plan(lens, par, C))


def test_special_cases():
    # everything fits: one partition holding all trees
    r = OPT.plan([5, 3, 4, 6], [-1, 0, 0, -1], 100)
    assert r["part_tokens"].tolist() == [18] and r["part_parent"].tolist() == [-1]
    # a chain at capacity = node length: one node per partition, each the parent of the next
    r = OPT.plan([4, 4, 4], [-1, 0, 1], 4)
    assert r["part_tokens"].tolist() == [4, 4, 4] and r["part_parent"].tolist() == [-1, 0, 1]
    # root 10 with children 6, 5, 4 at C = 16: cut the heaviest child (6); the
    # remaining root piece is 19 > 16, so 5 goes too; root piece 14; the two cut
    # pieces (6, 5) hang from the same node and pack together (11)
    r = OPT.plan([10, 6, 5, 4], [-1, 0, 0, 0], 16)
    assert r["part_tokens"].tolist() == [14, 11] and r["part_parent"].tolist() == [-1, 0]
    assert r["node_part"].tolist() == [0, 1, 1, 0] and r["part_cut"].tolist() == [-1, 0]
    # r(1) with children a(3) -> a1(2) and b(3) -> b1(2), C = 4. Cut: a
    # (3 + 2 > 4) drops a1, b drops b1, r (1 + 3 + 3 > 4) drops a (tie: the
    # earlier child): pieces {r, b} 4, {a} 3, {a1} 2, {b1} 2. Pack: {r, b};
    # then the pieces hanging from its nodes in preorder: from r: {a}; from
    # b: {b1}; then from a (in the second partition): {a1}.
    r = OPT.plan([1, 3, 2, 3, 2], [-1, 0, 1, 0, 3], 4)
    assert r["part_tokens"].tolist() == [4, 3, 2, 2] and r["part_cut"].tolist() == [-1, 0, 3, 1]
    assert r["part_parent"].tolist() == [-1, 0, 0, 1] and r["node_part"].tolist() == [0, 1, 3, 0, 2]


def test_token_counts_worked_case():
    """Root 10 with two children of 6 at C = 10: three partitions. Flattened
    (two sequences of 16) = 32 tokens; standard partitioning re-reads the root
    for each child partition: 22 + 10 = 32 (the children pack together: 22);
    with boundaries: 22."""
    lens, par = [10, 6, 6], [-1, 0, 0]
    r = OPT.plan(lens, par, 12)
    assert r["part_tokens"].tolist() == [10, 12]
    c = OPT.token_counts(lens, par, r["node_part"], seq_total=32)
    assert c == {"flattened": 32, "standard_partitioning": 32, "with_boundaries": 22}
