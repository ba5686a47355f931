"""Oracle: partition planner for trees larger than one pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows: "Tree Training" §3.3, Partitioning. Cuts fall on node
boundaries; a partition's backward must keep exactly one parent partition's
graph alive (so peak memory stays at one root-to-leaf path); the goal is the
fewest partitions of at most C tokens -- a bin packing of subtrees that the
pages hand to a general solver.

Reading taken (the pages leave the algorithm open):
1. Cut. Split the tree into the fewest connected pieces of <= C tokens, whole
   nodes only. Bottom-up, a node's residual is its own length plus its
   uncut children's residuals; while that exceeds C, the child with the
   largest residual is cut off (ties: the earlier child). This greedy is
   optimal for connected pieces (Kundu and Misra, "A linear tree partitioning
   algorithm", SIAM J. Comput. 1977); pinned here by brute force.
2. Pack. Pieces cut from the same node (or tree roots) share every ancestor,
   so they may share a partition with one parent partition and one gateway
   of cached ancestor rows (App. B.2 keeps one gateway per cut node). Groups
   are taken in order: tree roots first, then, partition by partition in
   creation order, the nodes of that partition in preorder; inside a group,
   first-fit decreasing by tokens (ties: preorder).
A node longer than C cannot be placed (a cut inside a node is not a node
boundary): the planner rejects it.
"""
from __future__ import annotations

import itertools

import numpy as np


def cut(node_len, node_parent, C):
    """Stage 1. Returns (piece_root_of_node [n], piece_tokens dict root -> tokens)."""
    n = len(node_len)
    assert max(node_len) <= C
    children = [[] for _ in range(n)]
    for v in range(n):
        if node_parent[v] >= 0:
            children[node_parent[v]].append(v)
    resid = [0] * n
    is_cut = [False] * n
    for v in range(n - 1, -1, -1):                 # children come after parents in preorder
        kids = list(children[v])
        total = node_len[v] + sum(resid[c] for c in kids)
        while total > C:
            heaviest = max(kids, key=lambda c: (resid[c], -c))
            is_cut[heaviest] = True
            kids.remove(heaviest)
            total -= resid[heaviest]
        resid[v] = total
    piece = [-1] * n
    for v in range(n):
        p = node_parent[v]
        piece[v] = v if (p < 0 or is_cut[v]) else piece[p]
    tokens = {}
    for v in range(n):
        tokens[piece[v]] = tokens.get(piece[v], 0) + int(node_len[v])
    return piece, tokens


def plan(node_len, node_parent, C):
    """Both stages. Returns dict: node_part [n], part_tokens [P], part_parent
    [P] (-1: no parent partition), part_cut [P] (the node the partition's
    pieces hang from, -1 for tree roots), piece [n] (piece root of each node)."""
    piece, tokens = cut(node_len, node_parent, C)
    roots = sorted(tokens)                            # piece roots in preorder
    part_of_piece = {}
    part_tokens, part_parent, part_cut = [], [], []
    queue = [-1]                                      # -1: the tree roots, then partitions in creation order
    while queue:
        gp = queue.pop(0)
        if gp == -1:
            cut_nodes = [-1]
        else:                                         # nodes of partition gp with pieces hanging from them
            cut_nodes = sorted({node_parent[r] for r in roots
                                if node_parent[r] >= 0 and part_of_piece.get(piece[node_parent[r]]) == gp})
        for u in cut_nodes:
            members = [r for r in roots if node_parent[r] == u]
            members.sort(key=lambda r: (-tokens[r], r))
            mine = []
            for r in members:
                for b in mine:
                    if part_tokens[b] + tokens[r] <= C:
                        part_of_piece[r] = b
                        part_tokens[b] += tokens[r]
                        break
                else:
                    b = len(part_tokens)
                    part_tokens.append(tokens[r])
                    part_parent.append(gp)
                    part_cut.append(u)
                    part_of_piece[r] = b
                    mine.append(b)
                    queue.append(b)
    node_part = [part_of_piece[piece[v]] for v in range(len(node_len))]
    return {"node_part": np.array(node_part), "part_tokens": np.array(part_tokens),
            "part_parent": np.array(part_parent), "part_cut": np.array(part_cut), "piece": np.array(piece)}


def min_connected_pieces_brute(node_len, node_parent, C):
    """Fewest connected pieces of <= C tokens, by trying every set of cut
    edges (tiny trees only)."""
    n = len(node_len)
    edges = [v for v in range(n) if node_parent[v] >= 0]
    best = None
    for k in range(len(edges) + 1):
        for cutset in itertools.combinations(edges, k):
            cs = set(cutset)
            piece = [-1] * n
            for v in range(n):
                p = node_parent[v]
                piece[v] = v if (p < 0 or v in cs) else piece[p]
            tok = {}
            for v in range(n):
                tok[piece[v]] = tok.get(piece[v], 0) + node_len[v]
            if max(tok.values()) <= C:
                best = len(tok)
                break
        if best is not None:
            break
    return best


def token_counts(node_len, node_parent, node_part, seq_total):
    """Tokens one pass over the data processes under three schemes ("Tree
    Training" Fig. 5): flattening every sequence (seq_total), partitions that
    re-include the ancestors of their pieces (no differentiable boundaries),
    and partitions with boundaries (every token once)."""
    n = len(node_len)
    unique = int(sum(node_len))
    recompute = unique
    for b in set(int(x) for x in node_part):
        anc = set()
        for v in range(n):
            if node_part[v] == b and (node_parent[v] < 0 or node_part[node_parent[v]] != b):
                u = node_parent[v]
                while u >= 0:
                    anc.add(u)
                    u = node_parent[u]
        recompute += sum(node_len[u] for u in anc if node_part[u] != b)
    return {"flattened": int(seq_total), "standard_partitioning": recompute, "with_boundaries": unique}
