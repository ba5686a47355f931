"""Pins of the tree SSM oracle (GDN state routing, tree conv1d): closed forms
of the delta rule, decayed linear attention under the tree mask for
orthonormal keys, the per-branch definition, the pages' chunked forms, a
library convolution, and finite differences. CPU only, float64."""
import numpy as np
import pytest

import workloads
from oracle import pack as OP
from oracle import ssm as OS


def _forest(seed, budgets=(40, 23), max_depth=4, lo=1, hi=9):
    seqs, groups = workloads.random_forest(seed, list(budgets), max_depth=max_depth, seg_lo=lo, seg_hi=hi)
    return OP.pack(seqs, groups)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _gdn_inputs(T, H, Hv, dk, dv, seed):
    rng = np.random.default_rng(seed)
    q = _unit(rng.standard_normal((T, H, dk)))
    k = _unit(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, Hv, dv))
    g = -np.log1p(np.exp(rng.standard_normal((T, Hv))))       # log sigmoid(-x): decays in (0, 1)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, Hv))))
    return q, k, v, g, beta


# ----------------------------------------------------------------- gated delta rule


def test_delta_rule_reads_back_what_it_wrote():
    """beta = 1, no decay, unit keys, q = k: the delta rule overwrites the
    value stored under k_t, so reading with k_t returns v_t exactly."""
    p = _forest(1)
    T = p["T"]
    q, k, v, g, beta = _gdn_inputs(T, 2, 2, 8, 5, 1)
    o = OS.gdn_tree(k, k, v, np.zeros_like(g), np.ones_like(beta), p["par"])
    assert np.max(np.abs(o - v)) < 1e-12


def test_full_forgetting_keeps_only_the_current_token():
    """alpha = 0 (g = -inf): h_t = beta k_t v_t^T, so o_t = beta (q.k) v_t."""
    p = _forest(2)
    q, k, v, g, beta = _gdn_inputs(p["T"], 2, 4, 8, 5, 2)
    o = OS.gdn_tree(q, k, v, np.full_like(g, -np.inf), beta, p["par"])
    qk = np.einsum("thk,thk->th", np.repeat(q, 2, 1), np.repeat(k, 2, 1))
    assert np.max(np.abs(o - (beta * qk)[:, :, None] * v)) < 1e-12


def test_orthonormal_keys_give_decayed_linear_attention_on_the_tree():
    """beta = 1 and keys that are distinct basis vectors along every path:
    nothing is ever overwritten, so o_t = sum over ancestors-or-self s of
    (q_t . k_s) exp(G_t - G_s) v_s with G the cumulative log decay along the
    path -- a dense masked product with the tree visibility mask."""
    p = _forest(3, budgets=(30, 17))
    par, pos, T = p["par"], p["pos"], p["T"]
    dk, dv = int(pos.max()) + 1, 6
    rng = np.random.default_rng(3)
    k = np.zeros((T, 1, dk))
    k[np.arange(T), 0, pos] = 1.0                       # depth-indexed basis vector
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    g = -rng.random((T, 1))
    o = OS.gdn_tree(q, k, v, g, np.ones((T, 1)), par)
    G = np.zeros(T)
    vis = np.zeros((T, T), bool)
    for t in range(T):
        G[t] = g[t, 0] + (G[par[t]] if par[t] >= 0 else 0.0)
        s = t
        while s >= 0:
            vis[t, s] = True
            s = par[s]
    scores = (q[:, 0] @ k[:, 0].T) * np.exp(np.where(vis, G[:, None] - G[None, :], -np.inf))
    assert np.max(np.abs(o[:, 0] - scores @ v[:, 0])) < 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_tree_routing_equals_every_branch_run_alone(seed):
    p = _forest(10 + seed)
    q, k, v, g, beta = _gdn_inputs(p["T"], 2, 4, 6, 5, seed)
    o = OS.gdn_tree(q, k, v, g, beta, p["par"])
    ob = OS.gdn_branches(q, k, v, g, beta, p["par"])
    assert np.max(np.abs(o - ob)) < 1e-11


def test_sequential_routing_differs_on_a_fork():
    """Carrying the state from the DFS-preceding sibling (what the pages warn
    about) changes the outputs of a second child."""
    p = OP.pack([[1, 2, 3], [1, 2, 4]])
    q, k, v, g, beta = _gdn_inputs(p["T"], 1, 1, 4, 3, 5)
    o = OS.gdn_tree(q, k, v, g, beta, p["par"])
    chain = np.arange(p["T"]) - 1                        # par of a single sequence in DFS order
    o_seq = OS.gdn_tree(q, k, v, g, beta, chain)
    assert np.allclose(o[:3], o_seq[:3]) and not np.allclose(o[3], o_seq[3])


@pytest.mark.parametrize("seed", range(4))
def test_pages_chunk_form_equals_the_recurrence(seed):
    p = _forest(20 + seed, budgets=(60, 41), lo=1, hi=14)
    q, k, v, g, beta = _gdn_inputs(p["T"], 2, 2, 6, 4, seed)
    o = OS.gdn_tree(q, k, v, g, beta, p["par"])
    oc = OS.gdn_chunks(q, k, v, g, beta, p["node_start"], p["node_end"], p["node_parent"])
    assert np.max(np.abs(o - oc)) < 1e-10


def _gdn_loss(ins, par, do):
    return float(np.sum(OS.gdn_tree(*ins, par) * do))


def test_gdn_backward_finite_differences_every_entry():
    """Central differences of sum(do * o) against every gradient entry, on a
    small forest with forks and two v-heads sharing one q/k head (their dq and
    dk add up)."""
    seqs, groups = workloads.random_forest(5, [12, 7], max_depth=3, seg_lo=1, seg_hi=4)
    p = OP.pack(seqs, groups)
    T = p["T"]
    rng = np.random.default_rng(0)
    q, k, v, g, beta = _gdn_inputs(T, 1, 2, 3, 2, 9)
    q = q * 1.3
    do = rng.standard_normal((T, 2, 2))
    grads = OS.gdn_tree_backward(q, k, v, g, beta, p["par"], do)
    ins = [q, k, v, g, beta]
    eps = 1e-6
    for n, (x, gx) in enumerate(zip(ins, grads)):
        assert gx.shape == x.shape
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp = [a.copy() for a in ins]
            xm = [a.copy() for a in ins]
            xp[n][idx] += eps
            xm[n][idx] -= eps
            fd[idx] = (_gdn_loss(xp, p["par"], do) - _gdn_loss(xm, p["par"], do)) / (2 * eps)
        assert np.max(np.abs(fd - gx)) < 1e-7 * (1 + np.max(np.abs(gx))), n


@pytest.mark.parametrize("seed", [0, 1])
def test_gdn_backward_directional_derivative(seed):
    """One random direction per input at a larger size (dk 8, dv 6, four
    v-heads on two q/k heads, deeper forest): <grad, dir> equals the central
    difference of the loss along dir."""
    p = _forest(30 + seed, budgets=(45, 30), lo=1, hi=9)
    T = p["T"]
    q, k, v, g, beta = _gdn_inputs(T, 2, 4, 8, 6, 40 + seed)
    rng = np.random.default_rng(seed)
    do = rng.standard_normal((T, 4, 6))
    grads = OS.gdn_tree_backward(q, k, v, g, beta, p["par"], do)
    ins = [q, k, v, g, beta]
    eps = 1e-5
    for n, gx in enumerate(grads):
        d = rng.standard_normal(ins[n].shape)
        xp = [a.copy() for a in ins]
        xm = [a.copy() for a in ins]
        xp[n] = xp[n] + eps * d
        xm[n] = xm[n] - eps * d
        fd = (_gdn_loss(xp, p["par"], do) - _gdn_loss(xm, p["par"], do)) / (2 * eps)
        assert abs(fd - np.sum(gx * d)) < 1e-7 * (1 + abs(fd)), n


def test_gdn_backward_full_forgetting_closed_form():
    """alpha = 0: o_t = beta_t (q_t . k_t) v_t, so dv_t = beta_t (q_t . k_t)
    do_t, dq_t = beta_t (v_t . do_t) k_t, dbeta_t = (q_t . k_t)(v_t . do_t),
    and nothing flows to the parent (dg = 0 because the state before the
    decay is multiplied by zero)."""
    p = _forest(4)
    T = p["T"]
    q, k, v, g, beta = _gdn_inputs(T, 1, 1, 5, 3, 4)
    do = np.random.default_rng(1).standard_normal((T, 1, 3))
    dq, dk, dv, dg, db = OS.gdn_tree_backward(q, k, v, np.full_like(g, -np.inf), beta, p["par"], do)
    qk = np.sum(q[:, 0] * k[:, 0], axis=1)
    vd = np.sum(v[:, 0] * do[:, 0], axis=1)
    assert np.max(np.abs(dv[:, 0] - (beta[:, 0] * qk)[:, None] * do[:, 0])) < 1e-12
    assert np.max(np.abs(dq[:, 0] - (beta[:, 0] * vd)[:, None] * k[:, 0])) < 1e-12
    assert np.max(np.abs(db[:, 0] - qk * vd)) < 1e-12
    assert np.max(np.abs(dg)) == 0.0


# ----------------------------------------------------------------- conv


def _conv_inputs(T, C, K, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, C)), rng.standard_normal((C, K)) * 0.5, rng.standard_normal(C) * 0.1


@pytest.mark.parametrize("act", ["silu", None])
def test_conv_chain_is_numpy_convolve(act):
    T, C, K = 23, 5, 4
    x, w, b = _conv_inputs(T, C, K, 1)
    y, _ = OS.tree_conv(x, w, b, np.arange(T) - 1, act)
    for c in range(C):
        a = np.convolve(x[:, c], w[c, ::-1])[:T] + b[c]  # causal: output t uses x[t-K+1..t]
        want = a / (1 + np.exp(-a)) if act == "silu" else a
        assert np.allclose(y[:, c], want, atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_conv_equals_every_branch_run_alone(seed):
    p = _forest(30 + seed)
    T, C, K = p["T"], 4, 4
    x, w, b = _conv_inputs(T, C, K, seed)
    y, _ = OS.tree_conv(x, w, b, p["par"])
    for path in OS.leaf_paths(p["par"]):
        for c in range(C):
            a = np.convolve(x[path, c], w[c, ::-1])[:len(path)] + b[c]
            assert np.allclose(y[path, c], a / (1 + np.exp(-a)), atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_conv_pages_chunk_form_with_short_parents(seed):
    """Nodes of 1-2 tokens make the saved context reach the grandparent."""
    p = _forest(40 + seed, lo=1, hi=3)
    assert np.min(p["node_end"] - p["node_start"]) < 3
    T, C, K = p["T"], 3, 4
    x, w, b = _conv_inputs(T, C, K, seed)
    y, _ = OS.tree_conv(x, w, b, p["par"])
    yc = OS.conv_chunks(x, w, b, p["node_start"], p["node_end"], p["node_parent"])
    assert np.max(np.abs(y - yc)) < 1e-13


@pytest.mark.parametrize("act", ["silu", None])
def test_conv_backward_finite_differences(act):
    p = _forest(50, budgets=(14, 9))
    T, C, K = p["T"], 3, 4
    x, w, b = _conv_inputs(T, C, K, 5)
    dy = np.random.default_rng(6).standard_normal((T, C))
    dx, dw, db = OS.tree_conv_backward(x, w, b, p["par"], dy, act)
    f = lambda x_, w_, b_: np.sum(dy * OS.tree_conv(x_, w_, b_, p["par"], act)[0])
    h = 1e-6
    for arr, grad in ((x, dx), (w, dw), (b, db)):
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = arr[i]
            arr[i] = old + h
            fp = f(x, w, b)
            arr[i] = old - h
            fm = f(x, w, b)
            arr[i] = old
            fd[i] = (fp - fm) / (2 * h)
        assert np.max(np.abs(fd - grad)) < 1e-7
