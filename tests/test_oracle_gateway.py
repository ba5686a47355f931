"""Pins for the gateway oracle (oracle/gateway.py).

The pages' claim for differentiable partition boundaries ("Tree Training"
§3.3, App. B.2-B.6) is that splitting a tree at a node boundary and running
the child partition against the parent's cached keys/values loses nothing:
every token is computed exactly once and the result equals the unsplit tree.
The main pin checks exactly that against the full-tree oracle (itself pinned
in test_oracle_attention.py): parent partition by plain tree attention, child
partitions through the gateway, gradients of the cached rows relayed into the
parent (Eq. 18 sums them over the children). Further pins: an empty gateway
reduces to plain tree attention, and with nothing visible in the gateway the
result does not depend on pos_offset (RoPE is relative).
"""
import numpy as np
import pytest

import workloads
from oracle import attention as OA
from oracle import gateway as GW
from oracle import pack as OP

TOL = 1e-9


def _tree(seed, budget=70):
    seqs, groups = workloads.random_forest(seed, [budget], max_depth=4, seg_lo=3, seg_hi=12)
    po = OP.pack(seqs, groups)
    return np.asarray(po["par"]), np.asarray(po["pos"])


def _inputs(T, Hq, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    do = rng.standard_normal((T, Hq, d))
    return q, k, v, do


def _cuts(par, rng, n):
    """Non-root tokens; prefer ones whose cut token is not the last row
    before them in preorder (then past_len differs from pos_offset)."""
    cand = [i for i in range(len(par)) if par[i] >= 0]
    far = [i for i in cand if par[i] != i - 1]
    pick = list(rng.choice(far, size=min(n, len(far)), replace=False)) if far else []
    pick += list(rng.choice(cand, size=n, replace=False))
    return [int(x) for x in pick]


def _partitioned(q, k, v, do, par, pos, children, theta=10000.0):
    sp = GW.split_at(par, children)
    P = sp["parent_rows"]
    e = sp["past_len"]
    # parent partition: plain tree attention on its own rows
    Op, Lp = OA.forward_branches(q[P], k[P], v[P], sp["parent_par"], pos[P], theta=theta)
    dqp, dkp, dvp = OA.backward_branches(q[P], k[P], v[P], do[P], sp["parent_par"], pos[P], theta=theta)
    k_past = OA.rope(k[P[:e]], pos[P[:e]], theta)
    v_past = v[P[:e]]
    T, Hq, d = q.shape
    O = np.zeros_like(q)
    LSE = np.zeros((Hq, T))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    O[P], LSE[:, P] = Op, Lp
    dq[P], dk[P], dv[P] = dqp, dkp, dvp
    acc_k = np.zeros_like(k_past)
    acc_v = np.zeros_like(v_past)
    for C, cpar in zip(sp["child_rows"], sp["child_par"]):
        Oc, Lc = GW.forward(q[C], k[C], v[C], cpar, k_past, v_past, sp["visible"], sp["pos_offset"], theta=theta)
        gq, gk, gv, gkp, gvp = GW.backward(q[C], k[C], v[C], do[C], cpar, k_past, v_past, sp["visible"],
                                           sp["pos_offset"], theta=theta)
        O[C], LSE[:, C] = Oc, Lc
        dq[C], dk[C], dv[C] = gq, gk, gv
        acc_k += gkp
        acc_v += gvp
    # relay: the cached keys were rotated at the parent's depths
    dk[P[:e]] += OA.rope_transpose(acc_k, pos[P[:e]], theta)
    dv[P[:e]] += acc_v
    return sp, O, LSE, dq, dk, dv


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_partition_equals_full_tree(seed):
    par, pos = _tree(seed)
    T = len(par)
    q, k, v, do = _inputs(T, 4, 2, 8, seed)
    O, LSE = OA.forward_branches(q, k, v, par, pos)
    dq, dk, dv = OA.backward_branches(q, k, v, do, par, pos)
    rng = np.random.default_rng(seed)
    n_offset_differs = 0
    for c in _cuts(par, rng, 3):
        sp, O2, L2, dq2, dk2, dv2 = _partitioned(q, k, v, do, par, pos, c)
        n_offset_differs += int(sp["past_len"] != sp["pos_offset"])
        assert np.max(np.abs(O2 - O)) < TOL and np.max(np.abs(L2 - LSE)) < TOL
        for a, b in ((dq2, dq), (dk2, dk), (dv2, dv)):
            assert np.max(np.abs(a - b)) < TOL
    assert n_offset_differs > 0  # Eq. 17: pos_offset != past_len when siblings precede the cut


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_two_child_partitions_sum_into_the_gateway(seed):
    """Eq. 18: children of one cut node accumulate into the same cached rows."""
    par, pos = _tree(seed, budget=90)
    T = len(par)
    kids = {}
    for i, p in enumerate(par):
        if p >= 0:
            kids.setdefault(int(p), []).append(i)
    forks = [v for v in kids.values() if len(v) >= 2]
    assert forks
    q, k, v, do = _inputs(T, 2, 1, 8, seed + 10)
    O, LSE = OA.forward_branches(q, k, v, par, pos)
    dq, dk, dv = OA.backward_branches(q, k, v, do, par, pos)
    sp, O2, L2, dq2, dk2, dv2 = _partitioned(q, k, v, do, par, pos, forks[0][:2])
    assert len(sp["child_rows"]) == 2
    assert np.max(np.abs(O2 - O)) < TOL and np.max(np.abs(L2 - LSE)) < TOL
    for a, b in ((dq2, dq), (dk2, dk), (dv2, dv)):
        assert np.max(np.abs(a - b)) < TOL


def test_empty_gateway_is_plain_tree_attention():
    par, pos = _tree(8, budget=40)
    T = len(par)
    q, k, v, do = _inputs(T, 2, 2, 8, 8)
    O, LSE = OA.forward_branches(q, k, v, par, pos)
    dq, dk, dv = OA.backward_branches(q, k, v, do, par, pos)
    z = np.zeros((0, 2, 8))
    O2, L2 = GW.forward(q, k, v, par, z, z, np.zeros(0, bool), 0)
    g = GW.backward(q, k, v, do, par, z, z, np.zeros(0, bool), 0)
    assert np.max(np.abs(O2 - O)) < TOL and np.max(np.abs(L2 - LSE)) < TOL
    for a, b in zip(g[:3], (dq, dk, dv)):
        assert np.max(np.abs(a - b)) < TOL
    assert g[3].shape == (0, 2, 8) and g[4].shape == (0, 2, 8)


def test_masked_gateway_ignores_pos_offset():
    """Nothing visible in the gateway: the child is plain tree attention and,
    RoPE being relative, independent of pos_offset; masked cached rows get
    zero gradient."""
    par, pos = _tree(9, budget=40)
    T = len(par)
    q, k, v, do = _inputs(T, 2, 1, 8, 9)
    rng = np.random.default_rng(9)
    kp, vp = rng.standard_normal((5, 1, 8)), rng.standard_normal((5, 1, 8))
    vis = np.zeros(5, bool)
    O, LSE = OA.forward_branches(q, k, v, par, pos)
    dq, dk, dv = OA.backward_branches(q, k, v, do, par, pos)
    for off in (0, 7, 123):
        O2, L2 = GW.forward(q, k, v, par, kp, vp, vis, off)
        g = GW.backward(q, k, v, do, par, kp, vp, vis, off)
        assert np.max(np.abs(O2 - O)) < TOL and np.max(np.abs(L2 - LSE)) < TOL
        for a, b in zip(g[:3], (dq, dk, dv)):
            assert np.max(np.abs(a - b)) < TOL
        assert not g[3].any() and not g[4].any()


def test_split_metadata_on_a_hand_tree():
    """Eq. 15-17 on the App. B.3 shape: DFS [a, b, c1, c2] with c1, c2
    siblings and the cut at c2: the gateway slice holds c1 but masks it, and
    pos_offset counts only the ancestor path."""
    # tokens: 0 a, 1 b, 2 c1, 3 c2, 4 child of c2
    par = np.array([-1, 0, 1, 1, 3])
    sp = GW.split_at(par, 4)
    assert list(sp["parent_rows"]) == [0, 1, 2, 3] and [list(r) for r in sp["child_rows"]] == [[4]]
    assert sp["past_len"] == 4
    assert list(sp["visible"]) == [True, True, False, True]
    assert sp["pos_offset"] == 3  # depth(c2) + 1 = 2 + 1, while past_len = 4
