"""Oracle: tree-routed Gated DeltaNet state and tree-correct causal conv1d.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows
---------------
* "Tree Training" §3.2, "SSM Layers (GDN)", Eq. 10: every tree chunk starts
  from the end state of its parent chunk (zero at a root), never from the
  DFS-preceding sibling; App. A.2 gives the chunked delta-rule computation
  with that routing.
* Same section, Eq. 11 and App. A.3: the causal conv1d of a chunk takes its
  left context from the parent's last K-1 effective input tokens (which reach
  into older ancestors when the parent is short), so every token sees the
  window an independent per-branch pass would give it.

Both fixes exist to make the packed tree reproduce an independent forward
pass of every root-to-leaf branch, so the plain definition is per token:
the recurrence and the conv window follow the parent chain par[t].

Gated delta rule (per v-head; state h is [dk, dv], alpha_t = exp(g_t)):
  h_t = alpha_t (I - beta_t k_t k_t^T) h_{par(t)} + beta_t k_t v_t^T,  h_{-1} = 0
  o_t = h_t^T q_t
q/k head of v-head j: j // (Hv / H). q and k are taken as given (any
normalisation or scaling is the caller's). The backward (gdn_tree_backward)
is reverse mode of this recurrence; the pages give no backward of their own
(training differentiates their forward), and it is pinned by finite
differences.

Tree conv (depthwise, kernel K, weight w [C, K], bias b [C]):
  a_t = b + sum_{n=0}^{K-1} w[:, K-1-n] * x_{anc_n(t)}   (anc_0 = t, zero past a root)
  y_t = act(a_t),  act = SiLU or identity
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------- helpers


def _ancestor(par, t, n):
    for _ in range(n):
        if t < 0:
            return -1
        t = int(par[t])
    return t


def _silu(a):
    return a / (1.0 + np.exp(-a))


def _silu_grad(a):
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def leaf_paths(par):
    """Root-to-leaf token paths of a packed forest (a leaf has no child)."""
    par = np.asarray(par)
    T = len(par)
    has_child = np.zeros(T, bool)
    has_child[par[par >= 0]] = True
    paths = []
    for t in range(T):
        if not has_child[t]:
            p = [t]
            while par[p[-1]] >= 0:
                p.append(int(par[p[-1]]))
            paths.append(p[::-1])
    return paths


# ----------------------------------------------------------------- conv


def tree_conv(x, w, b, par, activation="silu"):
    """Forward of the tree conv, per token along its ancestor chain. x [T, C];
    returns (y [T, C], a [T, C] the pre-activation)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    T, C = x.shape
    K = w.shape[1]
    a = np.tile(np.asarray(b, np.float64), (T, 1))
    for t in range(T):
        for n in range(K):
            s = _ancestor(par, t, n)
            if s < 0:
                break
            a[t] += w[:, K - 1 - n] * x[s]
    y = _silu(a) if activation == "silu" else a.copy()
    return y, a


def tree_conv_backward(x, w, b, par, dy, activation="silu"):
    """Gradients (dx, dw, db) of sum(dy * y) by the chain rule: every
    (token, ancestor) pair of the forward sum sends its product back."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    _, a = tree_conv(x, w, b, par, activation)
    gy = np.asarray(dy, np.float64) * (_silu_grad(a) if activation == "silu" else 1.0)
    T, C = x.shape
    K = w.shape[1]
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    for t in range(T):
        for n in range(K):
            s = _ancestor(par, t, n)
            if s < 0:
                break
            dx[s] += w[:, K - 1 - n] * gy[t]
            dw[:, K - 1 - n] += gy[t] * x[s]
    return dx, dw, gy.sum(axis=0)


def _causal_conv_plain(x, w, b, activation):
    """Ordinary causal depthwise conv of one [L, C] sequence with zero left
    padding (the per-chunk primitive App. A.3 calls)."""
    L, C = x.shape
    K = w.shape[1]
    xp = np.vstack([np.zeros((K - 1, C)), x])
    a = np.tile(b, (L, 1)).astype(np.float64)
    for i in range(K):
        a += w[:, i] * xp[i:i + L]
    return _silu(a) if activation == "silu" else a


def conv_chunks(x, w, b, node_start, node_end, node_parent, activation="silu"):
    """App. A.3 as described: chunks in DFS order; a chunk with a parent
    prepends the parent's saved K-1 effective input tokens, runs the plain
    causal conv on the extended chunk and drops the prepended outputs; it
    saves the last K-1 tokens of its extended input for its children (a root
    chunk saves its own tail, zero-padded on the left)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    b = np.asarray(b, np.float64)
    K = w.shape[1]
    C = x.shape[1]
    y = np.zeros_like(x)
    saved = {}
    for c in range(len(node_start)):
        s, e = int(node_start[c]), int(node_end[c])
        chunk = x[s:e]
        p = int(node_parent[c])
        if p >= 0:
            ext = np.vstack([saved[p], chunk])
            y[s:e] = _causal_conv_plain(ext, w, b, activation)[K - 1:]
        else:
            ext = np.vstack([np.zeros((K - 1, C)), chunk])
            y[s:e] = _causal_conv_plain(chunk, w, b, activation)
        saved[c] = ext[-(K - 1):].copy() if K > 1 else np.zeros((0, C))
    return y


# ----------------------------------------------------------------- gated delta rule


def _heads(q, k, v, g, beta):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    H, Hv = q.shape[1], v.shape[1]
    assert Hv % H == 0
    r = Hv // H
    # q/k of every v-head (v-head j reads q/k head j // r)
    return np.repeat(q, r, axis=1), np.repeat(k, r, axis=1), v, g, beta


def gdn_tree(q, k, v, g, beta, par, return_states=False):
    """Per-token recurrence in DFS order with the state routed through
    par[t] (Eq. 10 at token granularity). q, k [T, H, dk]; v [T, Hv, dv];
    g, beta [T, Hv]. Returns o [T, Hv, dv] (and the end state after every
    token when return_states)."""
    q, k, v, g, beta = _heads(q, k, v, g, beta)
    T, Hv, dk = k.shape
    dv = v.shape[2]
    par = np.asarray(par)
    nchild = np.zeros(T, np.int64)
    np.add.at(nchild, par[par >= 0], 1)
    keep = {}
    states = np.zeros((T, Hv, dk, dv)) if return_states else None
    o = np.zeros((T, Hv, dv))
    h = np.zeros((Hv, dk, dv))
    for t in range(T):
        p = int(par[t])
        if p < 0:
            h = np.zeros((Hv, dk, dv))
        elif p != t - 1:
            h = keep[p]
        h = h * np.exp(g[t])[:, None, None]
        kv = np.einsum("hk,hkv->hv", k[t], h)                  # what the state recalls for k_t
        delta = beta[t][:, None] * (v[t] - kv)
        h = h + k[t][:, :, None] * delta[:, None, :]
        o[t] = np.einsum("hk,hkv->hv", q[t], h)
        if nchild[t] >= 2:
            keep[t] = h
        if return_states:
            states[t] = h
    return (o, states) if return_states else o


def gdn_tree_backward(q, k, v, g, beta, par, do):
    """Gradients (dq, dk, dv, dg, dbeta) of sum(do * o) for gdn_tree, by
    reverse mode of the same per-token recurrence. Tokens are visited in
    reverse DFS order, so every child has already sent the gradient of its
    start state h_{par(t)} back to its parent (siblings add theirs, which is
    how a state shared by several branches collects its gradient). Per token,
    with hh = alpha h_par, delta = beta (v - hh^T k), h = hh + k delta^T and
    o = h^T q:
      dh     = (sum of the children's dh_par) + q do^T,   dq = h do
      ddelta = dh^T k,   dk = dh delta + hh (-beta ddelta),
      dv     = beta ddelta,   dbeta = ddelta . (v - hh^T k)
      dhh    = dh + k (-beta ddelta)^T,   dg = <dhh, hh>,   dh_par = alpha dhh
    dq and dk of a q/k head sum over the v-heads that read it."""
    H = np.asarray(q).shape[1]
    qr, kr, vv, gg, bb = _heads(q, k, v, g, beta)
    T, Hv, dk = kr.shape
    dv = vv.shape[2]
    do = np.asarray(do, np.float64)
    par = np.asarray(par)
    _, states = gdn_tree(q, k, v, g, beta, par, return_states=True)
    dH = np.zeros((T, Hv, dk, dv))
    dqr = np.zeros((T, Hv, dk))
    dkr = np.zeros((T, Hv, dk))
    dvv = np.zeros((T, Hv, dv))
    dg = np.zeros((T, Hv))
    dbeta = np.zeros((T, Hv))
    for t in range(T - 1, -1, -1):
        p = int(par[t])
        hp = states[p] if p >= 0 else np.zeros((Hv, dk, dv))
        a = np.exp(gg[t])
        hh = hp * a[:, None, None]
        resid = vv[t] - np.einsum("hk,hkv->hv", kr[t], hh)
        delta = bb[t][:, None] * resid
        h = states[t]
        dh = dH[t] + qr[t][:, :, None] * do[t][:, None, :]
        dqr[t] = np.einsum("hkv,hv->hk", h, do[t])
        ddelta = np.einsum("hkv,hk->hv", dh, kr[t])
        dkv = -bb[t][:, None] * ddelta
        dkr[t] = np.einsum("hkv,hv->hk", dh, delta) + np.einsum("hkv,hv->hk", hh, dkv)
        dvv[t] = bb[t][:, None] * ddelta
        dbeta[t] = np.sum(ddelta * resid, axis=1)
        dhh = dh + kr[t][:, :, None] * dkv[:, None, :]
        dg[t] = np.sum(dhh * hh, axis=(1, 2))
        if p >= 0:
            dH[p] += dhh * a[:, None, None]
    r = Hv // H
    dq = dqr.reshape(T, H, r, dk).sum(axis=2)
    dk_ = dkr.reshape(T, H, r, dk).sum(axis=2)
    return dq, dk_, dvv, dg, dbeta


def gdn_branches(q, k, v, g, beta, par):
    """The per-branch definition: run every root-to-leaf path on its own from
    a zero state, with the matrix form of the update, and map each packed
    token back (all paths through a token must agree)."""
    q, k, v, g, beta = _heads(q, k, v, g, beta)
    T, Hv, dk = k.shape
    dv = v.shape[2]
    o = np.full((T, Hv, dv), np.nan)
    eye = np.eye(dk)
    for path in leaf_paths(par):
        for hh in range(Hv):
            h = np.zeros((dk, dv))
            for t in path:
                kk = k[t, hh]
                A = np.exp(g[t, hh]) * (eye - beta[t, hh] * np.outer(kk, kk))
                h = A @ h + beta[t, hh] * np.outer(kk, v[t, hh])
                ot = h.T @ q[t, hh]
                if np.isnan(o[t, hh, 0]):
                    o[t, hh] = ot
                else:
                    assert np.max(np.abs(o[t, hh] - ot)) <= 1e-9 * (1.0 + np.max(np.abs(ot)))
    return o


def gdn_chunks(q, k, v, g, beta, node_start, node_end, node_parent):
    """App. A.2 as described: each tree node is one chunk; within a chunk
    the delta rule is solved in WY form, and the chunk starts from its parent
    node's end state. With gc the in-chunk cumulative log decay and
    Gam[i, j] = exp(gc_i - gc_j) (i >= j):
      M    = strictly-lower part of (beta k) k^T * Gam
      u    = (I + M)^-1 (beta v),   w = (I + M)^-1 (beta k * exp(gc))
      vn   = u - w h0
      o    = (q * exp(gc)) h0 + (lower-incl-diagonal part of q k^T * Gam) vn
      hend = exp(gc_last) h0 + (k * exp(gc_last - gc))^T vn
    """
    q, k, v, g, beta = _heads(q, k, v, g, beta)
    T, Hv, dk = k.shape
    dv = v.shape[2]
    o = np.zeros((T, Hv, dv))
    hend = {}
    for c in range(len(node_start)):
        s, e = int(node_start[c]), int(node_end[c])
        L = e - s
        p = int(node_parent[c])
        for hh in range(Hv):
            h0 = hend[(p, hh)] if p >= 0 else np.zeros((dk, dv))
            qc, kc, vc = q[s:e, hh], k[s:e, hh], v[s:e, hh]
            bc = beta[s:e, hh]
            gc = np.cumsum(g[s:e, hh])
            low = np.tril(np.ones((L, L)), -1)
            lowd = np.tril(np.ones((L, L)))
            Gam = np.exp(np.where(lowd > 0, gc[:, None] - gc[None, :], -np.inf))  # 0 above the diagonal
            M = (bc[:, None] * kc) @ kc.T * Gam * low
            IM = np.eye(L) + M
            u = np.linalg.solve(IM, bc[:, None] * vc)
            w = np.linalg.solve(IM, bc[:, None] * kc * np.exp(gc)[:, None])
            vn = u - w @ h0
            o[s:e, hh] = (qc * np.exp(gc)[:, None]) @ h0 + ((qc @ kc.T) * Gam * lowd) @ vn
            hend[(c, hh)] = np.exp(gc[-1]) * h0 + (kc * np.exp(gc[-1] - gc)[:, None]).T @ vn
    return o
