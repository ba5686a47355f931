"""Oracle: tree-masked attention, forward and backward, with RoPE at depth positions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method computes exactly (up to rounding order) a result with a plain
definition: "Tree Training" §3.1 Eq. 6 (forward equivalence) and the "Trie
packing" page ("identical initial representations plus identical visible
contexts produce identical layer outputs") say that every packed token's
attention output equals the one it gets in an ordinary causal forward pass
over any single root-to-leaf sequence that contains it. So the main oracle
here unpacks every root-to-leaf path, runs textbook causal attention on it
(S = QK^T / sqrt(d) with a causal mask, the "Trie packing" page, Step 3), and
maps the rows back. RoPE is applied to q and k at each token's position on
its path ("Trie packing" Step 1, "Tree Training" §3.2 Eq. 9), in the
rotate-half convention with base theta (the pages name RoPE but fix neither
convention nor base, so this is a reading).

Everything is float64. bf16 inputs are widened exactly.

Conventions: q [T, Hq, d], k and v [T, Hkv, d]; query head h uses kv head
h // (Hq // Hkv); LSE is the natural-log row log-sum-exp of the scaled scores,
laid out [Hq, T].

Other formulations kept for cross-checks and for sampled checks at full size:
  forward_dense   packed formulation with a brute-force dense visibility mask
  forward_rows    one query row at a time over its ancestor chain
  backward_rows_dq, backward_keys   gradients for sampled rows / keys
"""
from __future__ import annotations

import numpy as np

from .pack import leaf_paths, path_counts_through, ancestors_or_self, children_lists


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def rope_angles(positions, d, theta):
    """angle[n, k] = position_n * theta^(-2k/d), k < d/2, in float64.
    theta <= 0 means no rotation (all angles 0), the library's convention
    for switching RoPE off."""
    if theta <= 0:
        return np.zeros((len(positions), d // 2))
    k = np.arange(d // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * k / d)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(x, positions, theta):
    """Rotate-half RoPE. x [L, H, d] (float64); positions [L]."""
    d = x.shape[-1]
    ang = rope_angles(positions, d, theta)
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_transpose(g, positions, theta):
    """Gradient through RoPE: apply the inverse (= transposed) rotation."""
    d = g.shape[-1]
    ang = rope_angles(positions, d, theta)
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    g1, g2 = g[..., : d // 2], g[..., d // 2:]
    return np.concatenate([g1 * c + g2 * s, g2 * c - g1 * s], axis=-1)


def _causal_fwd(qr, kr, vv, scale):
    """Textbook causal attention on one sequence, one head. qr, kr, vv [L, d]."""
    L = qr.shape[0]
    S = (qr @ kr.T) * scale
    S[np.triu_indices(L, 1)] = -np.inf
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    return P @ vv, (m + np.log(l))[:, 0], P


def forward_branches(q, k, v, par, pos, scale=None, theta=10000.0, check_agree=True):
    """Per-branch forward. Returns (O [T,Hq,d], LSE [Hq,T]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    O = np.full((T, Hq, d), np.nan)
    LSE = np.full((Hq, T), np.nan)
    seen = np.zeros(T, dtype=bool)
    for p in leaf_paths(par):
        L = len(p)
        if not np.array_equal(np.asarray(pos)[p], np.arange(L)):
            raise AssertionError("depth positions differ from path offsets")
        qr = rope(q[p], np.arange(L), theta)
        kr = rope(k[p], np.arange(L), theta)
        for h in range(Hq):
            o, lse, _ = _causal_fwd(qr[:, h], kr[:, h // G], v[p, h // G], scale)
            new = ~seen[p]
            if check_agree and (~new).any():
                old = O[p[~new], h]
                if np.max(np.abs(old - o[~new])) > 1e-9:
                    raise AssertionError("branches disagree on a shared token")
            O[p[new], h] = o[new]
            LSE[h, p[new]] = lse[new]
        seen[p] = True
    return O, LSE


def backward_branches(q, k, v, do, par, pos, scale=None, theta=10000.0):
    """Per-branch backward of sum_i <dO_i, O_i>. Returns dq, dk, dv (float64).

    The upstream gradient of a token is split evenly over the c_i leaf paths
    through it; any split that sums to dO_i gives the same total, because
    every path through i contains all of i's visible keys. Per path the
    textbook attention backward runs (the "Trie packing" page, "Same chain
    rule": ordinary matrix backward, masked edges contribute zero), then the
    inverse RoPE rotation, then a scatter-add back to the packed rows, which
    also sums dK and dV over the query heads of a kv group.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    c = path_counts_through(par).astype(np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for p in leaf_paths(par):
        L = len(p)
        ar = np.arange(L)
        qr = rope(q[p], ar, theta)
        kr = rope(k[p], ar, theta)
        dqr = np.zeros((L, Hq, d))
        dkr = np.zeros((L, Hkv, d))
        for h in range(Hq):
            hk = h // G
            o, _, P = _causal_fwd(qr[:, h], kr[:, hk], v[p, hk], scale)
            dop = do[p, h] / c[p][:, None]
            dv[p, hk] += P.T @ dop
            dP = dop @ v[p, hk].T
            D = np.sum(dop * o, axis=1, keepdims=True)
            dS = P * (dP - D)
            dqr[:, h] += (dS @ kr[:, hk]) * scale
            dkr[:, hk] += (dS.T @ qr[:, h]) * scale
        dq[p] += rope_transpose(dqr, ar, theta)
        dk[p] += rope_transpose(dkr, ar, theta)
    return dq, dk, dv


def forward_dense(q, k, v, vis, pos, scale=None, theta=10000.0):
    """Packed formulation: S = QK^T * scale + M with M = 0 where vis, -inf
    elsewhere ("Trie packing" Step 3). Tiny inputs only."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hq, d = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    qr = rope(q, pos, theta)
    kr = rope(k, pos, theta)
    O = np.zeros((T, Hq, d))
    LSE = np.zeros((Hq, T))
    for h in range(Hq):
        S = (qr[:, h] @ kr[:, h // G].T) * scale
        S = np.where(vis, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        l = E.sum(axis=1, keepdims=True)
        O[:, h] = (E / l) @ v[:, h // G]
        LSE[h] = (m + np.log(l))[:, 0]
    return O, LSE


def _row(qi, kc, vc, scale):
    """One query row against its visible keys (already rotated)."""
    s = (kc @ qi) * scale
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    p = e / l
    return p @ vc, m + np.log(l), p


def forward_rows(q, k, v, par, rows, heads=None, scale=None, theta=10000.0):
    """Attention for selected query rows, each over its ancestor-or-self chain.

    Positions are the offsets along the chain (the token's depth). Returns
    O [len(rows), len(heads), d] and LSE [len(heads), len(rows)].
    """
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    heads = list(range(Hq)) if heads is None else list(heads)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    O = np.zeros((len(rows), len(heads), d))
    LSE = np.zeros((len(heads), len(rows)))
    for a, i in enumerate(rows):
        chain = ancestors_or_self(par, int(i))
        L = len(chain)
        qi = rope(_f64(q[i:i + 1]), [L - 1], theta)[0]
        kc = rope(_f64(k[chain]), np.arange(L), theta)
        vc = _f64(v[chain])
        for b, h in enumerate(heads):
            o, lse, _ = _row(qi[h], kc[:, h // G], vc[:, h // G], scale)
            O[a, b] = o
            LSE[b, a] = lse
    return O, LSE


def backward_rows_dq(q, k, v, do, par, rows, heads=None, scale=None, theta=10000.0):
    """dQ for selected rows: it depends only on the row's own chain.

    dq'_i = scale * sum_j dS_ij k'_j with dS_ij = P_ij (dO_i.v_j - dO_i.O_i),
    then the inverse rotation at the row's depth.
    """
    T, Hq, d = q.shape
    G = Hq // k.shape[1]
    heads = list(range(Hq)) if heads is None else list(heads)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((len(rows), len(heads), d))
    for a, i in enumerate(rows):
        chain = ancestors_or_self(par, int(i))
        L = len(chain)
        qi = rope(_f64(q[i:i + 1]), [L - 1], theta)[0]
        kc = rope(_f64(k[chain]), np.arange(L), theta)
        vc = _f64(v[chain])
        for b, h in enumerate(heads):
            hk = h // G
            o, _, p = _row(qi[h], kc[:, hk], vc[:, hk], scale)
            doi = _f64(do[i, h])
            ds = p * (vc[:, hk] @ doi - doi @ o)
            g = (ds @ kc[:, hk]) * scale
            out[a, b] = rope_transpose(g[None, None, :], [L - 1], theta)[0, 0]
    return out


def subtree_rows(par, j):
    """Token j and all its descendants, from the parent links alone."""
    ch = children_lists(par)
    out, stack = [], [int(j)]
    while stack:
        x = stack.pop()
        out.append(x)
        stack.extend(ch[x])
    return np.array(sorted(out), dtype=np.int64)


def backward_keys(q, k, v, do, par, keys, kv_heads=None, scale=None, theta=10000.0):
    """dK and dV for selected keys: sums over the key's descendants-or-self.

    dV_j = sum_{h in group} sum_i P_ij dO_i ;  dk'_j = scale * sum dS_ij q'_i,
    then the inverse rotation at the key's depth. Every row's softmax runs
    over its own ancestor chain. Returns (dk, dv) of shape
    [len(keys), len(kv_heads), d].
    """
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    kv_heads = list(range(Hkv)) if kv_heads is None else list(kv_heads)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    dk = np.zeros((len(keys), len(kv_heads), d))
    dv = np.zeros((len(keys), len(kv_heads), d))
    for a, j in enumerate(keys):
        j = int(j)
        above = ancestors_or_self(par, j)          # root .. j
        depth_j = len(above) - 1
        sub = subtree_rows(par, j)                 # j and its descendants
        # rotate every row that any chain below j uses, once
        rows = np.concatenate([above[:-1], sub])
        depth = {int(x): n for n, x in enumerate(above)}
        for x in sub:
            x = int(x)
            if x != j:
                depth[x] = depth[int(par[x])] + 1
        dpos = np.array([depth[int(x)] for x in rows], dtype=np.float64)
        slot = {int(x): n for n, x in enumerate(rows)}
        kr = rope(_f64(k[rows]), dpos, theta)
        vv = _f64(v[rows])
        acc_k = np.zeros((len(kv_heads), d))
        for i in sub:
            i = int(i)
            chain = [slot[int(x)] for x in ancestors_or_self(par, i)]
            qi = rope(_f64(q[i:i + 1]), [depth[i]], theta)[0]
            kc, vc = kr[chain], vv[chain]
            for b, hk in enumerate(kv_heads):
                for h in range(hk * G, (hk + 1) * G):
                    o, _, p = _row(qi[h], kc[:, hk], vc[:, hk], scale)
                    doi = _f64(do[i, h])
                    dv[a, b] += p[depth_j] * doi
                    ds_ij = p[depth_j] * (vc[depth_j, hk] @ doi - doi @ o)
                    acc_k[b] += ds_ij * qi[h] * scale
        dk[a] = rope_transpose(acc_k[None], [depth_j], theta)[0]
    return dk, dv


# ----------------------------------------------------------------------------
# Whole-tree ancestor-chain formulation (for element-wise checks at full size)
#
# Every packed query row attends to exactly its ancestor-or-self chain (the
# "Trie packing" page, Step 2; "Tree Training" §3.2, Attention Mask), with
# RoPE at its depth. The rows of a chain segment (a run of consecutive tokens
# each of whose parent is the token before it; in preorder the first child of
# a token directly follows it) share the ancestors of the segment's first
# token, so one textbook causal attention over [those ancestors ; the
# segment] with the segment's rows as queries computes them all. Gradients
# are the textbook ones, scatter-added to the keys of every chain they belong
# to ("Trie packing", "Same chain rule", Step 3). No path splitting is needed:
# each packed row is a query exactly once. A long segment is taken in blocks
# of at most `block` query rows, each over the segment's context plus the
# segment rows before and in the block, which bounds the masked part.


def chain_segments(par):
    """(start, end) of the maximal runs t with par[t] == t - 1, in order."""
    par = np.asarray(par)
    starts = [t for t in range(len(par)) if t == 0 or par[t] != t - 1]
    return list(zip(starts, starts[1:] + [len(par)]))


def chain_blocks(par, block):
    """(segment start, block start, block end): every chain segment cut into
    consecutive blocks of at most `block` rows."""
    return [(s, b, min(b + block, e)) for s, e in chain_segments(par) for b in range(s, e, block)]


def depths(par):
    """Depth of every token (0 at a root), from the parent links."""
    par = np.asarray(par)
    dep = np.zeros(len(par), dtype=np.int64)
    for t in range(len(par)):
        if par[t] >= 0:
            dep[t] = dep[par[t]] + 1
    return dep


def _block_keys(par, s, b, e):
    """Keys of query rows [b, e) of the segment starting at s: the ancestors
    of s (root first), then rows s .. e - 1; and the number before row b."""
    ctx = ancestors_or_self(par, int(par[s])) if par[s] >= 0 else np.zeros(0, dtype=np.int64)
    return np.concatenate([np.asarray(ctx, dtype=np.int64), np.arange(s, e, dtype=np.int64)]), len(ctx) + b - s


def _segment_probs(qr_h, kr_h, n_ctx, scale):
    """Causal softmax of one segment's rows over [context ; segment]."""
    S = (qr_h @ kr_h.T) * scale
    R, L = S.shape
    # row r sees key columns 0 .. n_ctx + r
    S[np.arange(L)[None, :] > (n_ctx + np.arange(R))[:, None]] = -np.inf
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return E / l, (m + np.log(l))[:, 0]


def _chain_heads(Hq, Hkv, kv_heads, q_heads):
    G = Hq // Hkv
    kv_heads = list(range(Hkv)) if kv_heads is None else list(kv_heads)
    heads = [h for hk in kv_heads for h in range(hk * G, (hk + 1) * G)]
    if q_heads is not None:
        heads = [h for h in heads if h in set(q_heads)]
    return kv_heads, heads, [kv_heads.index(h // G) for h in heads]


def forward_chains(q, k, v, par, kv_heads=None, scale=None, theta=10000.0, block=256, q_heads=None):
    """O and LSE of every row for the q heads of the given kv groups (or
    only those of them listed in q_heads). Returns O [T, n_heads, d] and
    LSE [n_heads, T], heads in increasing order."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    kv_heads, heads, slot = _chain_heads(Hq, Hkv, kv_heads, q_heads)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    dep = depths(par)
    qr = rope(_f64(q[:, heads]), dep, theta)
    kr = rope(_f64(k[:, kv_heads]), dep, theta)
    vv = _f64(v[:, kv_heads])
    O = np.zeros((T, len(heads), d))
    LSE = np.zeros((len(heads), T))
    for s, b0, e in chain_blocks(par, block):
        idx, n_ctx = _block_keys(par, s, b0, e)
        for a, b in enumerate(slot):
            P, lse = _segment_probs(qr[b0:e, a], kr[idx, b], n_ctx, scale)
            O[b0:e, a] = P @ vv[idx, b]
            LSE[a, b0:e] = lse
    return O, LSE


def backward_chains(q, k, v, do, par, kv_heads=None, scale=None, theta=10000.0, block=256, q_heads=None):
    """dQ of every row (the q heads of the given kv groups) and dK, dV of
    every key (those kv groups), for the upstream gradient do. With q_heads,
    only those heads are taken: the caller's do must be zero on the other
    heads of the groups, which then contribute nothing to dK and dV.
    Returns dq [T, n_heads, d], dk and dv [T, len(kv_heads), d]."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    kv_heads, heads, slot = _chain_heads(Hq, Hkv, kv_heads, q_heads)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    dep = depths(par)
    qr = rope(_f64(q[:, heads]), dep, theta)
    kr = rope(_f64(k[:, kv_heads]), dep, theta)
    vv = _f64(v[:, kv_heads])
    dov = _f64(do[:, heads])
    dqr = np.zeros((T, len(heads), d))
    dkr = np.zeros((T, len(kv_heads), d))
    dv = np.zeros((T, len(kv_heads), d))
    for s, b0, e in chain_blocks(par, block):
        idx, n_ctx = _block_keys(par, s, b0, e)
        for a, b in enumerate(slot):
            P, _ = _segment_probs(qr[b0:e, a], kr[idx, b], n_ctx, scale)
            o = P @ vv[idx, b]
            dOr = dov[b0:e, a]
            D = np.sum(dOr * o, axis=1, keepdims=True)
            dS = P * (dOr @ vv[idx, b].T - D)
            dqr[b0:e, a] = (dS @ kr[idx, b]) * scale
            dkr[idx, b] += (dS.T @ qr[b0:e, a]) * scale
            dv[idx, b] += P.T @ dOr
    return rope_transpose(dqr, dep, theta), rope_transpose(dkr, dep, theta), dv
