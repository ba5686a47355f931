"""Seeded synthetic workloads: token trees and dense inputs.

This module only draws inputs. It holds none of the method's arithmetic (no
packing, masking, attention or loss), so both the oracle-based tests and the
HIP path can take their inputs from it.

Tree workloads (token sequences plus a group label per sequence):

  ex_a      the worked example of the "Trie packing" page: ABCD, ABCE, ABFG
            with A..G = 0..6
  ex_b      the worked example of the Claw-R1 "Prefix Tree Merge" page:
            [1..5], [1,2,3,6,7], [1,2,3,6,7,8,9]
  short     8 trees, each a 256-token shared prompt plus 4 branches of 128
            tokens (the "short prompt, few branches" scenario of the Prefix
            Tree Merge page's token-ratio table)
  multistep 4 trees, each a 1024-token prompt and 8 trajectories of 2 steps:
            step 0 = prompt + 256-token response, step 1 = step 0 + 256-token
            tool output + 256-token response (the multi-step agent layout of
            the Prefix Tree Merge page, "Why prefix tree merge")
  agentic   one random agentic tree: depth <= 6 turns, 1-3 children per turn,
            segments of 64-1024 tokens, grown breadth-first until exactly
            32768 tokens
  agentic_l the same generator with depth <= 10 and 131072 tokens

Token ids are uniform in [0, 32000); the first tokens of sibling segments are
forced pairwise distinct so that the trie keeps the generated branching.
Sequences are emitted in depth-first leaf order, so insertion order
reproduces the generated layout.

Dense inputs are float32 N(0, 1) from a seeded torch generator, rounded to
bf16 (round to nearest even) where the workload is bf16.
"""
from __future__ import annotations

import numpy as np

VOCAB_TOKENS = 32000

WORKLOADS = {
    "ex_a": dict(Hq=1, Hkv=1, d=16, dtype="f32", vocab=32, seed=1),
    "ex_b": dict(Hq=1, Hkv=1, d=16, dtype="f32", vocab=32, seed=1),
    "short": dict(Hq=32, Hkv=8, d=128, dtype="bf16", seed=2),
    "multistep": dict(Hq=32, Hkv=8, d=128, dtype="bf16", seed=3),
    "agentic": dict(Hq=64, Hkv=8, d=128, dtype="bf16", seed=4, max_depth=6, budget=32768),
    "agentic_l": dict(Hq=64, Hkv=8, d=128, dtype="bf16", seed=5, max_depth=10, budget=131072),
}


def _segment(rng, n, avoid_first=None):
    seg = rng.integers(0, VOCAB_TOKENS, size=n)
    if avoid_first is not None:
        while int(seg[0]) in avoid_first:
            seg[0] = rng.integers(0, VOCAB_TOKENS)
    return seg


def _shared_prefix_trees(rng, n_trees, prefix_len, branch_lens):
    """n_trees trees; each = prefix + one branch per entry of branch_lens."""
    seqs, groups = [], []
    for t in range(n_trees):
        prefix = _segment(rng, prefix_len)
        firsts = set()
        for bl in branch_lens:
            br = _segment(rng, bl, firsts)
            firsts.add(int(br[0]))
            seqs.append(np.concatenate([prefix, br]))
            groups.append(t)
    return seqs, groups


def _multistep_trees(rng, n_trees, prompt_len, n_traj, resp0, tool, resp1):
    seqs, groups = [], []
    for t in range(n_trees):
        prompt = _segment(rng, prompt_len)
        firsts = set()
        for _ in range(n_traj):
            r0 = _segment(rng, resp0, firsts)
            firsts.add(int(r0[0]))
            step0 = np.concatenate([prompt, r0])
            step1 = np.concatenate([step0, _segment(rng, tool), _segment(rng, resp1)])
            seqs += [step0, step1]
            groups += [t, t]
    return seqs, groups


def random_tree_structure(seed, max_depth, budget, seg_lo=64, seg_hi=1024, max_tries=1000):
    """Breadth-first random tree with exactly `budget` tokens.

    Root segment length U{seg_lo..seg_hi}; nodes are expanded in BFS order;
    a node at max_depth is not expanded; otherwise it gets U{1,2,3} children
    of length U{seg_lo..seg_hi}. The child that reaches the budget is cut to
    fit and all growth stops. A tree that stops growing short of the budget
    is rejected and the next seed is tried. Returns (children, lengths,
    accepted_seed); node 0 is the root.
    """
    for attempt in range(max_tries):
        s = seed + attempt
        rng = np.random.default_rng(s)
        lengths = [int(rng.integers(seg_lo, seg_hi + 1))]
        children = [[]]
        total = lengths[0]
        queue = [(0, 1)]
        head = 0
        done = total >= budget
        while head < len(queue) and not done:
            node, depth = queue[head]
            head += 1
            if depth >= max_depth:
                continue
            b = int(rng.integers(1, 4))
            for _ in range(b):
                L = int(rng.integers(seg_lo, seg_hi + 1))
                cid = len(lengths)
                if total + L >= budget:
                    L = budget - total
                    lengths.append(L)
                    children.append([])
                    children[node].append(cid)
                    total += L
                    done = True
                    break
                lengths.append(L)
                children.append([])
                children[node].append(cid)
                total += L
                queue.append((cid, depth + 1))
        if total == budget:
            return children, lengths, s
    raise RuntimeError("no tree reached the budget")


def random_tree(seed, max_depth, budget, seg_lo=64, seg_hi=1024):
    """Sequences of one random tree from random_tree_structure (DFS leaf order)."""
    seqs, groups, _ = _random_tree_sequences(seed, max_depth, budget, seg_lo, seg_hi)
    return seqs, groups


def random_forest(seed, budgets, max_depth=4, seg_lo=8, seg_hi=120):
    """Several random trees, one group each, for multi-tile tests."""
    seqs, groups = [], []
    for t, b in enumerate(budgets):
        s, _ = random_tree(seed * 101 + t, max_depth, b, seg_lo, seg_hi)
        seqs += s
        groups += [t] * len(s)
    return seqs, groups


def _random_tree_sequences(seed, max_depth, budget, seg_lo=64, seg_hi=1024):
    children, lengths, accepted = random_tree_structure(seed, max_depth, budget, seg_lo, seg_hi)
    rng = np.random.default_rng(accepted + 7919)
    segs = [None] * len(lengths)
    segs[0] = _segment(rng, lengths[0])
    order = [0]
    for node in order:  # BFS over the structure, siblings drawn together
        firsts = set()
        for c in children[node]:
            segs[c] = _segment(rng, lengths[c], firsts)
            firsts.add(int(segs[c][0]))
            order.append(c)
    seqs = []

    def dfs(node, prefix):
        cur = np.concatenate([prefix, segs[node]])
        if not children[node]:
            seqs.append(cur)
        for c in children[node]:
            dfs(c, cur)

    import sys
    old = sys.getrecursionlimit()
    sys.setrecursionlimit(max(old, 10000))
    try:
        dfs(0, np.zeros(0, dtype=np.int64))
    finally:
        sys.setrecursionlimit(old)
    return seqs, [0] * len(seqs), accepted


def sequences(name):
    """Token sequences and group labels of a named tree workload."""
    if name == "ex_a":
        A, B, C, D, E, F, G = range(7)
        return [[A, B, C, D], [A, B, C, E], [A, B, F, G]], [0, 0, 0]
    if name == "ex_b":
        return [[1, 2, 3, 4, 5], [1, 2, 3, 6, 7], [1, 2, 3, 6, 7, 8, 9]], [0, 0, 0]
    cfg = WORKLOADS[name]
    rng = np.random.default_rng(cfg["seed"])
    if name == "short":
        return _shared_prefix_trees(rng, 8, 256, [128] * 4)
    if name == "multistep":
        return _multistep_trees(rng, 4, 1024, 8, 256, 256, 256)
    if name in ("agentic", "agentic_l"):
        seqs, groups, _ = _random_tree_sequences(cfg["seed"], cfg["max_depth"], cfg["budget"])
        return seqs, groups
    raise KeyError(name)


def random_small_forest(rng, n_seqs_max=6, len_max=8, vocab=4, n_groups_max=3):
    """Tiny random sequence sets for brute-force checks: a small vocabulary
    makes shared prefixes, duplicates and prefix-of-another cases common."""
    n = int(rng.integers(1, n_seqs_max + 1))
    seqs = [list(rng.integers(0, vocab, size=int(rng.integers(1, len_max + 1)))) for _ in range(n)]
    groups = [int(x) for x in rng.integers(0, int(rng.integers(1, n_groups_max + 1)), size=n)]
    return seqs, groups


def dense_inputs(T, Hq, Hkv, d, dtype, seed, device="cpu", with_grad_out=True):
    """q [T,Hq,d], k, v [T,Hkv,d] and dO [T,Hq,d]: N(0,1) float32 draws from
    a torch generator seeded with seed + 1000, rounded to bf16 if asked."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 1000)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def draw(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32).to(tdt)

    q = draw(T, Hq, d)
    k = draw(T, Hkv, d)
    v = draw(T, Hkv, d)
    do = draw(T, Hq, d) if with_grad_out else None
    return q, k, v, do


def logits_input(R, V, dtype, seed, device="cpu"):
    """[R, V] N(0,1) logits from a torch generator seeded with seed + 2000."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 2000)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.randn(R, V, generator=gen, device=device, dtype=torch.float32).to(tdt)


def repeated_rows_entries(R, V, repeats, seed):
    """Entries that reference every row exactly `repeats` times, in a seeded
    random order, with uniform targets in [0, V) and weight 1/repeats."""
    rng = np.random.default_rng(seed + 3000)
    src = rng.permutation(np.repeat(np.arange(R, dtype=np.int64), repeats))
    tgt = rng.integers(0, V, size=R * repeats)
    w = np.full(R * repeats, 1.0 / repeats, dtype=np.float32)
    return src.astype(np.int32), tgt.astype(np.int32), w


# ratios r = exp(logp - old_logp) for policy-loss inputs: below, inside and
# above the default clip range [0.8, 1.2], each at least 0.05 from its edges
POLICY_RATIOS = np.array([0.5, 0.7, 0.9, 1.0, 1.1, 1.3, 1.6])


def policy_inputs(M, seed, mask_frac=0.1):
    """Per-entry advantages N(0, 1), a ratio drawn from POLICY_RATIOS (the
    caller sets old_logp = logp - ln r from its own logp) and a mask with
    about mask_frac of the entries off."""
    rng = np.random.default_rng(seed + 4000)
    adv = rng.standard_normal(M).astype(np.float32)
    ratio = POLICY_RATIOS[rng.integers(0, len(POLICY_RATIOS), M)]
    mask = (rng.random(M) >= mask_frac).astype(np.uint8)
    return adv, ratio, mask


def gdn_inputs(T, H, Hv, dk, dv, dtype, seed, device="cpu"):
    """Gated-delta-rule inputs: q, k rows of unit length (the caller-side
    normalisation GDN layers apply), v N(0, 1), log decays g = -softplus(x)
    with x ~ N(-2, 1) (decay factors mostly 0.8-0.95), beta = sigmoid(N(0, 1))."""
    import torch

    gen = torch.Generator().manual_seed(seed + 5000)
    q = torch.randn(T, H, dk, generator=gen)
    k = torch.randn(T, H, dk, generator=gen)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn(T, Hv, dv, generator=gen)
    g = -torch.nn.functional.softplus(torch.randn(T, Hv, generator=gen) - 2.0)
    beta = torch.sigmoid(torch.randn(T, Hv, generator=gen))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return (q.to(dt).to(device), k.to(dt).to(device), v.to(dt).to(device), g.to(device), beta.to(device))


def gdn_dout(T, Hv, dv, dtype, seed, device="cpu"):
    """Output gradient for the gated delta rule backward: N(0, 1) [T, Hv, dv]."""
    import torch

    gen = torch.Generator().manual_seed(seed + 5500)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.randn(T, Hv, dv, generator=gen).to(dt).to(device)


def conv_inputs(T, C, K, dtype, seed, device="cpu"):
    """Tree conv inputs: x and dy N(0, 1) [T, C], weight N(0, 0.25) [C, K],
    bias N(0, 0.01) [C]."""
    import torch

    gen = torch.Generator().manual_seed(seed + 6000)
    x = torch.randn(T, C, generator=gen)
    dy = torch.randn(T, C, generator=gen)
    w = torch.randn(C, K, generator=gen) * 0.5
    b = torch.randn(C, generator=gen) * 0.1
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return x.to(dt).to(device), dy.to(dt).to(device), w.to(device), b.to(device)
