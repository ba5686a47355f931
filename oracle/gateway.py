"""Oracle: tree attention across a partition boundary (a "gateway").

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Tree Training" §3.3 and App. B.2-B.5: when a tree is split into partitions
at node boundaries, a child partition does not re-run its ancestors. It
attends to the parent partition's cached, already rotated keys and values
(past_len rows, App. B.2), masked by an additive bias that is 0 on the
ancestors of the cut node and -inf on every other cached row (Eq. 15-16),
followed by its own packed subtree under the ordinary tree mask (Eq. 14).
Its own tokens take RoPE at pos_offset + depth inside the subtree (Eq. 17).
The gradients of the cached rows leave in float32 and are summed over all
child partitions of the cut node before they are relayed into the parent
partition's backward (Eq. 18).

The oracle below is that definition written out one query row at a time
(the heads of one kv group as one batched product), in float64: row i of the child sees the
visible cached rows (given post-RoPE) plus its own ancestors-or-self, with q
and the own keys rotated at pos_offset + depth.

Conventions as in oracle.attention: q [T, Hq, d], k and v [T, Hkv, d];
k_past and v_past [past_len, Hkv, d] (k_past post-RoPE); visible [past_len]
booleans; LSE [Hq, T].
"""
from __future__ import annotations

import numpy as np

from .attention import rope, rope_transpose, _f64
from .pack import ancestors_or_self


def _depths(par):
    d = np.zeros(len(par), dtype=np.int64)
    for i, p in enumerate(par):
        d[i] = 0 if p < 0 else d[p] + 1
    return d


def _row_keys(k, v, kp, vp, chain, depth_chain, pos_offset, theta):
    """Visible cached rows followed by the own chain, rotated where needed."""
    kc = rope(_f64(k[chain]), pos_offset + depth_chain, theta)
    return np.concatenate([kp, kc], axis=0), np.concatenate([vp, _f64(v[chain])], axis=0)


def forward(q, k, v, par, k_past, v_past, visible, pos_offset, scale=None, theta=10000.0):
    """O [T, Hq, d] and LSE [Hq, T] of the child partition (float64)."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    vis = np.asarray(visible, dtype=bool)
    kp, vp = _f64(k_past)[vis], _f64(v_past)[vis]
    depth = _depths(par)
    O = np.zeros((T, Hq, d))
    LSE = np.zeros((Hq, T))
    for i in range(T):
        chain = ancestors_or_self(par, i)
        kc, vc = _row_keys(k, v, kp, vp, chain, depth[chain], pos_offset, theta)  # [L, Hkv, d]
        qi = rope(_f64(q[i:i + 1]), [pos_offset + depth[i]], theta)[0]            # [Hq, d]
        s = (qi.reshape(Hkv, G, d) @ kc.transpose(1, 2, 0)) * scale              # [Hkv, G, L]
        m = s.max(axis=2, keepdims=True)
        e = np.exp(s - m)
        O[i] = ((e / e.sum(axis=2, keepdims=True)) @ vc.transpose(1, 0, 2)).reshape(Hq, d)
        LSE[:, i] = (m + np.log(e.sum(axis=2, keepdims=True))).reshape(Hq)
    return O, LSE


def backward(q, k, v, do, par, k_past, v_past, visible, pos_offset, scale=None, theta=10000.0):
    """Gradients of sum_i <dO_i, O_i>: dq, dk, dv of the child's own rows
    (through their RoPE) and dk_past, dv_past of the cached rows (with
    respect to the given post-RoPE keys; zero on rows the bias masks)."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    Lp = k_past.shape[0]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    vis = np.asarray(visible, dtype=bool)
    vidx = np.nonzero(vis)[0]
    kp, vp = _f64(k_past)[vis], _f64(v_past)[vis]
    nv = len(vidx)
    depth = _depths(par)
    dq = np.zeros((T, Hq, d))
    dkr = np.zeros((T, Hkv, d))  # gradient w.r.t. the rotated own keys
    dv = np.zeros((T, Hkv, d))
    dk_past = np.zeros((Lp, Hkv, d))
    dv_past = np.zeros((Lp, Hkv, d))
    for i in range(T):
        chain = ancestors_or_self(par, i)
        kc, vc = _row_keys(k, v, kp, vp, chain, depth[chain], pos_offset, theta)  # [L, Hkv, d]
        kh, vh = kc.transpose(1, 0, 2), vc.transpose(1, 0, 2)                    # [Hkv, L, d]
        qi = rope(_f64(q[i:i + 1]), [pos_offset + depth[i]], theta)[0]
        qg = qi.reshape(Hkv, G, d)
        s = (qg @ kh.transpose(0, 2, 1)) * scale                                  # [Hkv, G, L]
        e = np.exp(s - s.max(axis=2, keepdims=True))
        p = e / e.sum(axis=2, keepdims=True)
        o = p @ vh                                                                # [Hkv, G, d]
        dg = _f64(do[i]).reshape(Hkv, G, d)
        ds = p * ((dg @ vh.transpose(0, 2, 1)) - np.sum(dg * o, axis=2, keepdims=True))
        gq = (ds @ kh).reshape(Hq, d) * scale
        dq[i] = rope_transpose(gq[None], [pos_offset + depth[i]], theta)[0]
        # per key and kv head, summed over the G query heads of the group
        gk = ((ds.transpose(0, 2, 1) @ qg) * scale).transpose(1, 0, 2)           # [L, Hkv, d]
        gv = (p.transpose(0, 2, 1) @ dg).transpose(1, 0, 2)
        dk_past[vidx] += gk[:nv]
        dv_past[vidx] += gv[:nv]
        dkr[chain] += gk[nv:]
        dv[chain] += gv[nv:]
    dk = rope_transpose(dkr, pos_offset + depth, theta)
    return dq, dk, dv, dk_past, dv_past


def split_at(par, children):
    """Split a packed tree at the edges (cut, c) for c in `children`, which
    must share one parent token `cut` (App. B.2-B.5).

    Each child partition is the subtree of one child; the parent partition is
    everything else, in the same preorder. Returns a dict with
      parent_rows, parent_par   packed indices of the parent partition and its
                                parent links remapped to it
      child_rows, child_par     lists, one entry per child partition
      past_len                  e: the parent rows up to and including the
                                cut token (the gateway slice)
      visible                   [past_len] bool, Eq. 15-16: the cut token and
                                its ancestors
      pos_offset                Eq. 17: depth of the cut token + 1
    """
    par = np.asarray(par)
    T = len(par)
    children = [int(children)] if np.isscalar(children) else [int(c) for c in children]
    cut = int(par[children[0]])
    if cut < 0 or any(int(par[c]) != cut for c in children):
        raise ValueError("the children must share one parent token")
    ch = [[] for _ in range(T)]
    for i, p in enumerate(par):
        if p >= 0:
            ch[p].append(i)
    owner = -np.ones(T, dtype=np.int64)  # child partition of each token, -1 = parent
    for n, c in enumerate(children):
        stack = [c]
        while stack:
            x = stack.pop()
            owner[x] = n
            stack.extend(ch[x])
    parent_rows = np.nonzero(owner < 0)[0]
    pmap = -np.ones(T, dtype=np.int64)
    pmap[parent_rows] = np.arange(len(parent_rows))
    parent_par = np.array([pmap[par[i]] if par[i] >= 0 else -1 for i in parent_rows], dtype=np.int64)
    child_rows, child_par = [], []
    for n in range(len(children)):
        rows = np.nonzero(owner == n)[0]
        cmap = -np.ones(T, dtype=np.int64)
        cmap[rows] = np.arange(len(rows))
        child_rows.append(rows)
        child_par.append(np.array([cmap[par[i]] if par[i] >= 0 and owner[par[i]] == n else -1 for i in rows],
                                  dtype=np.int64))
    past_len = int(pmap[cut]) + 1
    anc = set(int(x) for x in ancestors_or_self(par, cut))
    visible = np.array([int(parent_rows[n]) in anc for n in range(past_len)], dtype=bool)
    depth = _depths(par)
    return dict(parent_rows=parent_rows, child_rows=child_rows, parent_par=parent_par, child_par=child_par,
                past_len=past_len, visible=visible, pos_offset=int(depth[cut]) + 1)
