"""Oracle: trie packing of token sequences into one DFS-serialized stream.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What it follows
---------------
* "Trie packing" page, "Three sequences, one shared tree" and "Step 1 - Store
  each node once": identical prefixes become one set of token nodes; a token
  is shared only when its whole preceding context is identical; the position
  ID of a token is its depth on its own path, not its packed index.
* "Tree Training" §3.1, Eq. 7-8: the DFS serialization visits every tree token
  once (parent before children, children one after another); Eq. 9: the
  position of a token is the summed length of its ancestors' segments plus
  its offset inside its own segment; §3.1 Eq. 2-4: g_t counts the paths
  through t, the per-token weight is g_t / K.
* Claw-R1 "Prefix Tree Merge" page, section 1 (build and compress): insert
  every sequence into a plain trie, merge single-child chains into one node,
  then give every node its (start, end) range in preorder.

Readings taken where the pages are silent:
* children are visited in first-insertion order;
* a node boundary falls at a fork and also right after a token where some
  input sequence ends (the Prefix Tree Merge example keeps [6,7] and [8,9]
  apart although [6,7] has one child, because seq1 ends at 7);
* K is the number of input sequences of the group and g_t the number of input
  sequences that contain t (duplicates count);
* one trie per group; groups are laid out one after another in order of
  first appearance; positions restart at 0 in every tree;
* node and subtree ends are exclusive.
"""
from __future__ import annotations

import numpy as np


class _TrieNode:
    __slots__ = ("token", "children", "passes", "ends", "parent")

    def __init__(self, token, parent):
        self.token = token
        self.parent = parent
        self.children = {}  # token -> node; dict keeps first-insertion order
        self.passes = 0     # sequences whose path goes through this token
        self.ends = 0       # sequences whose last token is this one


def _group_order(groups):
    order, seen = [], set()
    for gid in groups:
        if gid not in seen:
            seen.add(gid)
            order.append(gid)
    return order


def pack(seqs, groups=None):
    """Pack token sequences; returns a dict of NumPy arrays.

    seqs   : list of sequences (lists / arrays of ints), each non-empty
    groups : optional list, one group label per sequence (None = one tree)

    Keys of the result:
      ids, pos, se (subtree end, exclusive), par (-1 at a tree root), g,
      weight (float32 g/K), K_of_token, occ (list of int arrays, one per input
      sequence: packed index of each of its tokens), node_start, node_end
      (exclusive), node_parent (-1 at a root), node_se, node_seqs (sorted
      list of sequence indices per node), tree_start (n_trees + 1), T,
      n_nodes, n_trees.
    """
    n = len(seqs)
    if n == 0:
        raise ValueError("no sequences")
    for s in seqs:
        if len(s) == 0:
            raise ValueError("empty sequence")
    if groups is None:
        groups = [0] * n
    if len(groups) != n:
        raise ValueError("groups length mismatch")

    ids, pos, se, par, g, weight, kot = [], [], [], [], [], [], []
    occ = [None] * n
    node_start, node_end, node_parent, node_se, node_seqs = [], [], [], [], []
    tree_start = [0]

    for gid in _group_order(groups):
        members = [k for k in range(n) if groups[k] == gid]
        K = len(members)
        root = _TrieNode(None, None)
        # trie insert (Prefix Tree Merge, "insert"): one node per distinct prefix
        seq_nodes = {}
        for k in members:
            cur = root
            path = []
            for tok in seqs[k]:
                tok = int(tok)
                nxt = cur.children.get(tok)
                if nxt is None:
                    nxt = _TrieNode(tok, cur)
                    cur.children[tok] = nxt
                nxt.passes += 1
                path.append(nxt)
                cur = nxt
            cur.ends += 1
            seq_nodes[k] = path

        # preorder DFS, children in first-insertion order (Eq. 8)
        base = len(ids)
        index_of = {}
        order = []
        stack = list(reversed(list(root.children.values())))
        while stack:
            node = stack.pop()
            index_of[id(node)] = base + len(order)
            order.append(node)
            stack.extend(reversed(list(node.children.values())))

        depth_of = {}
        for node in order:
            i = index_of[id(node)]
            p = node.parent
            if p is root:
                parent_index = -1
                depth = 0
            else:
                parent_index = index_of[id(p)]
                depth = depth_of[id(p)] + 1
            depth_of[id(node)] = depth
            ids.append(node.token)
            pos.append(depth)          # depth on the token's own path (Eq. 9)
            par.append(parent_index)
            g.append(node.passes)
            weight.append(np.float32(node.passes) / np.float32(K))
            kot.append(K)

        # subtree end: one past the last packed index below the token
        T_tree = len(order)
        size = [1] * T_tree
        for local in range(T_tree - 1, -1, -1):
            p = par[base + local]
            if p >= 0:
                size[p - base] += size[local]
        for local in range(T_tree):
            se.append(base + local + size[local])

        # chunk (node) formation: a new chunk starts at a tree root, below a
        # fork, or after a token where an input sequence ends
        node_of = {}
        for node in order:
            i = index_of[id(node)]
            p = node.parent
            starts = (p is root) or len(p.children) >= 2 or p.ends > 0
            if starts:
                c = len(node_start)
                node_start.append(i)
                node_end.append(i + 1)
                node_parent.append(-1 if p is root else node_of[id(p)])
                node_se.append(se[i])
                node_seqs.append(set())
            else:
                c = node_of[id(p)]
                if node_end[c] != i:
                    raise AssertionError("chain not contiguous in DFS order")
                node_end[c] = i + 1
            node_of[id(node)] = c

        for k in members:
            path = seq_nodes[k]
            occ[k] = np.array([index_of[id(nd)] for nd in path], dtype=np.int64)
            for nd in path:
                node_seqs[node_of[id(nd)]].add(k)

        tree_start.append(len(ids))

    out = dict(
        ids=np.array(ids, dtype=np.int64),
        pos=np.array(pos, dtype=np.int64),
        se=np.array(se, dtype=np.int64),
        par=np.array(par, dtype=np.int64),
        g=np.array(g, dtype=np.int64),
        weight=np.array(weight, dtype=np.float32),
        K_of_token=np.array(kot, dtype=np.int64),
        occ=occ,
        node_start=np.array(node_start, dtype=np.int64),
        node_end=np.array(node_end, dtype=np.int64),
        node_parent=np.array(node_parent, dtype=np.int64),
        node_se=np.array(node_se, dtype=np.int64),
        node_seqs=[sorted(s) for s in node_seqs],
        tree_start=np.array(tree_start, dtype=np.int64),
    )
    out["T"] = len(ids)
    out["n_nodes"] = len(node_start)
    out["n_trees"] = len(tree_start) - 1
    return out


def children_lists(par):
    """Children of every packed token, in packed (preorder) order."""
    T = len(par)
    ch = [[] for _ in range(T)]
    for i in range(T):
        if par[i] >= 0:
            ch[par[i]].append(i)
    return ch


def leaf_paths(par):
    """Root-to-leaf index paths: walk parents up from every token with no child."""
    T = len(par)
    has_child = np.zeros(T, dtype=bool)
    for i in range(T):
        if par[i] >= 0:
            has_child[par[i]] = True
    paths = []
    for leaf in range(T):
        if has_child[leaf]:
            continue
        p = []
        j = leaf
        while j >= 0:
            p.append(j)
            j = par[j]
        paths.append(np.array(p[::-1], dtype=np.int64))
    return paths


def ancestors_or_self(par, i):
    """Packed indices on the root-to-i path, root first."""
    chain = []
    j = i
    while j >= 0:
        chain.append(j)
        j = par[j]
    return np.array(chain[::-1], dtype=np.int64)


def visibility_dense(par):
    """Brute-force (T, T) visibility: vis[i, j] iff j is i or one of i's ancestors.

    The "Trie packing" page, Step 2 ("allow only ancestors and self"), and
    "Tree Training" §3.2 (attend iff j <= i and both lie on one root-to-leaf
    path). Tiny inputs only.
    """
    T = len(par)
    vis = np.zeros((T, T), dtype=bool)
    for i in range(T):
        j = i
        while j >= 0:
            vis[i, j] = True
            j = par[j]
    return vis


def visibility_chunks(p):
    """(T, T) visibility from the chunk view: every token of every ancestor
    chunk, plus causal order inside the token's own chunk ("Tree Training"
    App. A.1, the chunk-boundary mask construction). Tiny inputs only."""
    T = p["T"]
    ns, ne, npar = p["node_start"], p["node_end"], p["node_parent"]
    chunk_of = np.empty(T, dtype=np.int64)
    for c in range(len(ns)):
        chunk_of[ns[c]:ne[c]] = c
    vis = np.zeros((T, T), dtype=bool)
    for i in range(T):
        c = chunk_of[i]
        vis[i, ns[c]:i + 1] = True
        a = npar[c]
        while a >= 0:
            vis[i, ns[a]:ne[a]] = True
            a = npar[a]
    return vis


def path_counts_through(par):
    """c_i: number of root-to-leaf paths (leaves) through token i."""
    c = np.zeros(len(par), dtype=np.int64)
    for path in leaf_paths(par):
        c[path] += 1
    return c
