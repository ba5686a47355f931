"""Pins of the packing oracle against the pages' printed facts, invariants and
brute force. CPU only."""
import json
import os

import numpy as np
import pytest

import workloads
from oracle import pack as OP


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_trie_packing_example(golden_dir):
    gd = _load(golden_dir, "trie_packing_example.json")
    tok = gd["tokens"]
    seqs = [[tok[c] for c in s] for s in gd["sequences"]]
    p = OP.pack(seqs)
    assert p["ids"].tolist() == [tok[c] for c in gd["packed_tokens"]]
    assert p["pos"].tolist() == gd["position_ids"]
    assert p["T"] == gd["ffn_rows_packed"]
    assert sum(len(s) for s in seqs) == gd["ffn_rows_unpacked"]
    vis = OP.visibility_dense(p["par"])
    name = {v: k for k, v in tok.items()}
    idx = {name[int(t)]: i for i, t in enumerate(p["ids"])}
    for q, keys in gd["sees"].items():
        assert sorted(name[int(p["ids"][j])] for j in np.nonzero(vis[idx[q]])[0]) == sorted(keys)
    for q, keys in gd["never_sees"].items():
        for kk in keys:
            assert not vis[idx[q], idx[kk]]
    assert vis.sum() == gd["allowed_pairs_packed"]
    assert sum(len(s) * (len(s) + 1) // 2 for s in seqs) == gd["allowed_pairs_unpacked"]
    assert p["T"] ** 2 == gd["dense_score_entries_packed"]
    assert sum(len(s) ** 2 for s in seqs) == gd["dense_score_entries_unpacked"]
    # shared logit rows: one entry per original prediction occurrence
    src = [int(p["occ"][k][a]) for k, s in enumerate(seqs) for a in range(len(s) - 1)]
    tgt = [name[s[a + 1]] for s in seqs for a in range(len(s) - 1)]
    assert src == gd["source_rows"]
    assert tgt == gd["targets"]
    assert len(src) == gd["prediction_occurrences"]
    assert len(set(src)) == gd["distinct_logit_rows"]


def test_prefix_tree_merge_example(golden_dir):
    gd = _load(golden_dir, "prefix_tree_merge_example.json")
    seqs = gd["sequences"]
    p = OP.pack(seqs)
    assert p["ids"].tolist() == gd["packed_sequence"]
    assert p["T"] == gd["packed_tokens"]
    assert sum(len(s) for s in seqs) == gd["original_tokens"]
    assert round(100.0 * p["T"] / gd["original_tokens"], 1) == gd["token_ratio_percent"]
    assert p["n_nodes"] == len(gd["nodes"])
    for c, nd in enumerate(gd["nodes"]):
        s, e = int(p["node_start"][c]), int(p["node_end"][c])
        assert [s, e - 1] == nd["range_inclusive"]
        assert p["ids"][s:e].tolist() == nd["tokens"]
        assert p["node_seqs"][c] == nd["seqs"]
        want_parent = -1 if nd["parent"] is None else nd["parent"]
        assert int(p["node_parent"][c]) == want_parent
    assert [o.tolist() for o in p["occ"]] == gd["paths"]
    vis = OP.visibility_dense(p["par"])
    for k, row in enumerate(gd["mask_rows"]):
        assert vis[p["occ"][k][-1]].astype(int).tolist() == row


def _check_invariants(seqs, groups, p):
    T = p["T"]
    par, pos, se, g = p["par"], p["pos"], p["se"], p["g"]
    # parents precede children, depth grows by one
    for i in range(T):
        if par[i] >= 0:
            assert par[i] < i
            assert pos[i] == pos[par[i]] + 1
        else:
            assert pos[i] == 0
    # subtree intervals are laminar and contain exactly the descendants
    for i in range(T):
        assert i < se[i] <= T
        if par[i] >= 0:
            assert se[i] <= se[par[i]]
    # path counts: sum of g equals the total input length
    assert int(g.sum()) == sum(len(s) for s in seqs)
    # T equals the number of distinct (group, prefix) pairs
    prefixes = set()
    for s, gr in zip(seqs, groups):
        for a in range(1, len(s) + 1):
            prefixes.add((gr, tuple(int(x) for x in s[:a])))
    assert T == len(prefixes)
    # every sequence is recovered by walking parents from its last token
    for k, s in enumerate(seqs):
        occ = p["occ"][k]
        assert occ.shape[0] == len(s)
        chain = OP.ancestors_or_self(par, int(occ[-1]))
        assert chain.tolist() == occ.tolist()
        assert p["ids"][occ].tolist() == [int(x) for x in s]
    # three independent visibility constructions agree
    vis = OP.visibility_dense(par)
    ii, jj = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
    rule = (jj <= ii) & (ii < se[jj])
    assert np.array_equal(vis, rule)
    assert np.array_equal(vis, OP.visibility_chunks(p))
    assert vis.sum() == int((pos + 1).sum())
    # nodes partition the stream; tokens of a node share their sequence set
    cover = np.zeros(T, dtype=int)
    for c in range(p["n_nodes"]):
        s0, e0 = p["node_start"][c], p["node_end"][c]
        cover[s0:e0] += 1
        assert len(set(g[s0:e0].tolist())) == 1
        assert p["node_se"][c] == se[s0]
    assert (cover == 1).all()
    # weights: g / K in float32, K = sequences of the token's tree
    for i in range(T):
        assert p["weight"][i] == np.float32(g[i]) / np.float32(p["K_of_token"][i])


def test_invariants_random_forests():
    rng = np.random.default_rng(1234)
    for _ in range(400):
        seqs, groups = workloads.random_small_forest(rng)
        p = OP.pack(seqs, groups)
        _check_invariants(seqs, groups, p)


def test_single_sequence_is_causal():
    p = OP.pack([[5, 1, 5, 1, 9, 9]])
    T = p["T"]
    assert T == 6
    assert (p["se"] == T).all()
    vis = OP.visibility_dense(p["par"])
    assert np.array_equal(vis, np.tril(np.ones((T, T), dtype=bool)))
    assert p["n_nodes"] == 1


def test_disjoint_sequences_block_diagonal():
    # distinct first tokens: plain sequence packing ("Tree Training" §2: a plain
    # sequence is a special case of a prefix tree)
    seqs = [[0, 1, 2], [1, 1], [2, 0, 0, 0]]
    p = OP.pack(seqs)
    vis = OP.visibility_dense(p["par"])
    want = np.zeros((9, 9), dtype=bool)
    o = 0
    for s in seqs:
        L = len(s)
        want[o:o + L, o:o + L] = np.tril(np.ones((L, L), dtype=bool))
        o += L
    assert np.array_equal(vis, want)


def test_groups_make_separate_trees():
    seqs = [[1, 2, 3], [1, 2, 4], [1, 2, 3]]
    p = OP.pack(seqs, [7, 3, 7])
    # group 7 first (first appearance), duplicates count in g and K
    assert p["tree_start"].tolist() == [0, 3, 6]
    assert p["g"].tolist() == [2, 2, 2, 1, 1, 1]
    assert p["weight"].tolist() == [1.0, 1.0, 1.0, 1.0, 1.0, 1.0]
    assert p["pos"].tolist() == [0, 1, 2, 0, 1, 2]
    assert p["se"].tolist() == [3, 3, 3, 6, 6, 6]


def test_empty_sequence_rejected():
    with pytest.raises(ValueError):
        OP.pack([[1, 2], []])


@pytest.mark.parametrize("name", ["short", "multistep", "agentic"])
def test_generator_trees_come_back(name):
    seqs, groups = workloads.sequences(name)
    p = OP.pack(seqs, groups)
    if name == "short":
        assert p["T"] == 8 * (256 + 4 * 128)
        assert p["n_nodes"] == 8 * 5
        assert (p["K_of_token"] == 4).all()
    elif name == "multistep":
        assert p["T"] == 4 * (1024 + 8 * (256 + 512))
        assert p["n_nodes"] == 4 * (1 + 8 + 8)
        assert (p["K_of_token"] == 16).all()
    else:
        children, lengths, _ = workloads.random_tree_structure(4, 6, 32768)
        assert p["T"] == sum(lengths) == 32768
        # chains of single children fold into one node
        single_edges = sum(1 for ch in children if len(ch) == 1)
        assert p["n_nodes"] == len(lengths) - single_edges
        leaves = sum(1 for ch in children if not ch)
        assert len(seqs) == leaves and (p["K_of_token"] == leaves).all()
