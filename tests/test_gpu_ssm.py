"""GPU parity of the tree SSM kernels against the float64 oracle.

tree_conv_fwd / tree_conv_bwd against oracle.ssm.tree_conv(_backward);
tree_gdn_fwd against oracle.ssm.gdn_tree (the per-token recurrence routed
through par); tree_gdn_bwd against oracle.ssm.gdn_tree_backward (reverse
mode of that recurrence). Inputs are the bf16 / fp32 values the kernels
receive.

Tolerances (none are stated for these kernels; they follow the attention
ones): outputs max |err| / max(1, |ref|) <= 2e-2, gradients relative L2 <=
5e-2. The scaling by max(1, |ref|) is there because a bf16 output is rounded
once, with a relative error up to 2^-9, so values above 1 carry an
absolute rounding error that grows with them (a conv output near 8 rounds by
up to 0.03). The GDN output is O(1) for unit-length q, k; its products round
operands to bf16 (relative 2^-9) with float32 accumulation.
"""
import numpy as np
import pytest
import torch

import tree_packed_attention_amd as ta
import workloads
from oracle import pack as OP
from oracle import ssm as OS

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-2
GRAD_TOL = 5e-2


def host(t):
    return t.detach().double().cpu().numpy()


def out_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b)))) if b.size else 0.0


def rel_l2(a, b):
    """Relative L2 error; the absolute one where the reference is all zero
    (a single token's decay gradient is exactly zero)."""
    nb = np.linalg.norm(np.asarray(b))
    d = np.linalg.norm(np.asarray(a) - np.asarray(b))
    return float(d / nb) if nb > 0 else float(d)


def _pack(seqs, groups):
    p = ta.tree_pack(seqs, groups)
    po = OP.pack(seqs, groups)
    assert np.array_equal(p["parent"], po["par"])
    return p, po


# ----------------------------------------------------------------- conv

CONV_CASES = {
    "forest_short_nodes_bf16": (lambda: workloads.random_forest(3, [200, 131], max_depth=40, seg_lo=1, seg_hi=4), 64, 4,
                                "bf16", 1),
    "forest_f32_no_act": (lambda: workloads.random_forest(4, [150, 77]), 40, 4, "f32", 0),
    "forest_k2_f32": (lambda: workloads.random_forest(5, [90]), 24, 2, "f32", 1),
    "forest_k1_bf16": (lambda: workloads.random_forest(7, [150, 60]), 48, 1, "bf16", 1),
    "chain_k8_bf16": (lambda: ([list(range(300))], [0]), 2056, 8, "bf16", 1),
    "single_token": (lambda: ([[7]], None), 8, 4, "f32", 1),
    "deep_tree": (lambda: workloads.random_tree(11, 6, 1500, 16, 200), 128, 4, "bf16", 1),
}


@pytest.mark.parametrize("case", list(CONV_CASES))
def test_conv_matches_oracle(case):
    make, C, K, dtype, act = CONV_CASES[case]
    seqs, groups = make()
    print(f"\n[case] conv {case}", flush=True)
    p, po = _pack(seqs, groups)
    T = p["T"]
    x, dy, w, b = workloads.conv_inputs(T, C, K, dtype, 7)
    dev = "cuda"
    par = torch.from_numpy(p["parent"]).to(dev)
    pos = torch.from_numpy(p["pos"]).to(dev)
    se = torch.from_numpy(p["subtree_end"]).to(dev)
    y = ta.tree_conv_fwd(x.to(dev), w.to(dev), b.to(dev), par, act)
    dx, dw, db = ta.tree_conv_bwd(x.to(dev), dy.to(dev), w.to(dev), b.to(dev), par, pos, se, act)
    torch.cuda.synchronize()
    a = "silu" if act else None
    ry, _ = OS.tree_conv(host(x), host(w), host(b), po["par"], a)
    rdx, rdw, rdb = OS.tree_conv_backward(host(x), host(w), host(b), po["par"], host(dy), a)
    tol_y = OUT_TOL if dtype == "bf16" else 1e-5
    tol_g = GRAD_TOL if dtype == "bf16" else 1e-5
    assert out_err(host(y), ry) <= tol_y
    assert rel_l2(host(dx), rdx) <= tol_g
    assert rel_l2(host(dw), rdw) <= 1e-5
    assert rel_l2(host(db), rdb) <= 1e-5


def test_conv_multistep_full_size_channel_slice():
    """The multistep batch (T = 28672) at 8192 channels (the conv width of a
    16 q/k-head x 32 v-head x 128 layer), K = 4, bf16, SiLU. The conv is
    depthwise, so a channel slice of the oracle is exact for those channels:
    every token on 256 channels."""
    seqs, groups = workloads.sequences("multistep")
    p, po = _pack(seqs, groups)
    T, C, K = p["T"], 8192, 4
    x, dy, w, b = workloads.conv_inputs(T, C, K, "bf16", 3, device="cuda")
    par = torch.from_numpy(p["parent"]).cuda()
    y = ta.tree_conv_fwd(x, w, b, par, 1)
    dx, dw, db = ta.tree_conv_bwd(x, dy, w, b, par, torch.from_numpy(p["pos"]).cuda(),
                                  torch.from_numpy(p["subtree_end"]).cuda(), 1)
    torch.cuda.synchronize()
    cs = np.r_[0:128, C - 128:C]
    ry, _ = OS.tree_conv(host(x[:, cs]), host(w[cs]), host(b[cs]), po["par"])
    rdx, rdw, rdb = OS.tree_conv_backward(host(x[:, cs]), host(w[cs]), host(b[cs]), po["par"], host(dy[:, cs]))
    assert out_err(host(y[:, cs]), ry) <= OUT_TOL
    assert rel_l2(host(dx[:, cs]), rdx) <= GRAD_TOL
    assert rel_l2(host(dw[cs]), rdw) <= 1e-4 and rel_l2(host(db[cs]), rdb) <= 1e-4


def test_conv_max_size_tree():
    """The largest tree (agentic_l: 131072 tokens, depth up to 5842, forks at
    every level) at 256 channels, K = 4, bf16, SiLU: every token against the
    oracle."""
    seqs, groups = workloads.sequences("agentic_l")
    p, po = _pack(seqs, groups)
    T, C, K = p["T"], 256, 4
    x, dy, w, b = workloads.conv_inputs(T, C, K, "bf16", 4, device="cuda")
    par = torch.from_numpy(p["parent"]).cuda()
    y = ta.tree_conv_fwd(x, w, b, par, 1)
    dx, dw, db = ta.tree_conv_bwd(x, dy, w, b, par, torch.from_numpy(p["pos"]).cuda(),
                                  torch.from_numpy(p["subtree_end"]).cuda(), 1)
    torch.cuda.synchronize()
    print(f"\n[case] conv agentic_l T={T}", flush=True)
    ry, _ = OS.tree_conv(host(x), host(w), host(b), po["par"])
    rdx, rdw, rdb = OS.tree_conv_backward(host(x), host(w), host(b), po["par"], host(dy))
    assert out_err(host(y), ry) <= OUT_TOL
    assert rel_l2(host(dx), rdx) <= GRAD_TOL
    assert rel_l2(host(dw), rdw) <= 1e-4 and rel_l2(host(db), rdb) <= 1e-4


def test_conv_bwd_deterministic():
    seqs, groups = workloads.random_forest(8, [400, 300])
    p, _ = _pack(seqs, groups)
    x, dy, w, b = workloads.conv_inputs(p["T"], 64, 4, "bf16", 2, device="cuda")
    args = (x, dy, w, b, torch.from_numpy(p["parent"]).cuda(), torch.from_numpy(p["pos"]).cuda(),
            torch.from_numpy(p["subtree_end"]).cuda(), 1)
    r1 = ta.tree_conv_bwd(*args)
    r2 = ta.tree_conv_bwd(*args)
    for a, c in zip(r1, r2):
        assert torch.equal(a, c)


# ----------------------------------------------------------------- gated delta rule

GDN_CASES = {
    # name: (sequences, H, Hv, dk, dv, dtype, chunk)
    "forest_gva_d64": (lambda: workloads.random_forest(3, [333, 250, 97]), 2, 4, 64, 64, "bf16", 64),
    "forest_short_nodes_chunk16": (lambda: workloads.random_forest(4, [200, 190], max_depth=12, seg_lo=1, seg_hi=40),
                                   1, 2, 128, 128, "bf16", 16),
    "forest_f32_dk128_dv64": (lambda: workloads.random_forest(6, [260, 41]), 2, 2, 128, 64, "f32", 64),
    "chain_d128": (lambda: ([list(range(500))], [0]), 1, 1, 128, 128, "bf16", 64),
    "varlen_disjoint": (lambda: ([[1000 + i] + list(range(40 + 23 * i)) for i in range(5)], None), 1, 2, 64, 128,
                        "bf16", 64),
    "single_token": (lambda: ([[5]], None), 1, 1, 64, 64, "bf16", 64),
    "deep_tree_chunk7": (lambda: workloads.random_tree(11, 6, 1500, 16, 200), 1, 2, 64, 64, "bf16", 7),
}


def _gdn_case(seqs, groups, H, Hv, dk, dv, dtype, chunk, seed=17):
    p, po = _pack(seqs, groups)
    plan = ta.tree_gdn_plan(p["node_start"], p["node_end"], p["node_parent"], chunk)
    q, k, v, g, beta = workloads.gdn_inputs(p["T"], H, Hv, dk, dv, dtype, seed, device="cuda")
    o = ta.tree_gdn_fwd(q, k, v, g, beta, plan)
    torch.cuda.synchronize()
    return p, po, plan, (q, k, v, g, beta), o


@pytest.mark.parametrize("case", list(GDN_CASES))
def test_gdn_matches_oracle(case):
    make, H, Hv, dk, dv, dtype, chunk = GDN_CASES[case]
    seqs, groups = make()
    print(f"\n[case] gdn {case}", flush=True)
    p, po, plan, (q, k, v, g, beta), o = _gdn_case(seqs, groups, H, Hv, dk, dv, dtype, chunk)
    ro = OS.gdn_tree(host(q), host(k), host(v), host(g), host(beta), po["par"])
    err = out_err(host(o), ro)
    print(case, f"max-abs {err:.2e} rel-l2 {rel_l2(host(o), ro):.2e} levels {plan[2]}", flush=True)
    assert err <= OUT_TOL
    assert rel_l2(host(o), ro) <= 1e-2


def test_gdn_chunk_size_does_not_change_the_result_beyond_rounding():
    seqs, groups = workloads.random_forest(9, [300, 200])
    outs = []
    for chunk in (64, 32, 5):
        *_, o = _gdn_case(seqs, groups, 1, 2, 64, 64, "bf16", chunk)
        outs.append(host(o))
    assert out_err(outs[1], outs[0]) <= OUT_TOL and out_err(outs[2], outs[0]) <= OUT_TOL


def test_gdn_multistep_full_size_trees():
    """The multistep batch (T = 28672, 4 trees) with 16 q/k heads, 32 v heads,
    dk = dv = 128, bf16. Trees are independent, so the oracle runs whole trees
    0 and 3 on v-heads 0 and 31 (with their q/k heads)."""
    seqs, groups = workloads.sequences("multistep")
    H, Hv, d = 16, 32, 128
    p, po, plan, (q, k, v, g, beta), o = _gdn_case(seqs, groups, H, Hv, d, d, "bf16", 64, seed=3)
    for t in (0, 3):
        ts, te = int(po["tree_start"][t]), int(po["tree_start"][t + 1])
        par = po["par"][ts:te].copy()
        par[par >= 0] -= ts
        for hv in (0, Hv - 1):
            hk = hv // (Hv // H)
            ro = OS.gdn_tree(host(q[ts:te, hk:hk + 1]), host(k[ts:te, hk:hk + 1]), host(v[ts:te, hv:hv + 1]),
                             host(g[ts:te, hv:hv + 1]), host(beta[ts:te, hv:hv + 1]), par)
            got = host(o[ts:te, hv:hv + 1])
            print(f"tree {t} v-head {hv}: err {out_err(got, ro):.2e}", flush=True)
            assert out_err(got, ro) <= OUT_TOL
            assert rel_l2(got, ro) <= 1e-2


def test_gdn_deterministic():
    seqs, groups = workloads.random_forest(12, [500, 300])
    *_, inp, o1 = _gdn_case(seqs, groups, 2, 4, 128, 128, "bf16", 64)
    *_, o2 = _gdn_case(seqs, groups, 2, 4, 128, 128, "bf16", 64)
    assert torch.equal(o1, o2)


# ----------------------------------------------------------------- gated delta rule, backward

GRAD_NAMES = ("dq", "dk", "dv", "dg", "dbeta")


def _gdn_bwd_case(seqs, groups, H, Hv, dk, dv, dtype, chunk, seed=17):
    p, po = _pack(seqs, groups)
    plan = ta.tree_gdn_plan(p["node_start"], p["node_end"], p["node_parent"], chunk)
    q, k, v, g, beta = workloads.gdn_inputs(p["T"], H, Hv, dk, dv, dtype, seed, device="cuda")
    do = workloads.gdn_dout(p["T"], Hv, dv, dtype, seed, device="cuda")
    ws = ta.gdn_workspace(q, v, plan, backward=True)
    ta.tree_gdn_fwd(q, k, v, g, beta, plan, workspace=ws)
    grads = ta.tree_gdn_bwd(q, k, v, g, beta, do, plan, ws)
    torch.cuda.synchronize()
    return po, plan, (q, k, v, g, beta, do), grads


def _check_grads(tag, got, ref):
    for name, a, b in zip(GRAD_NAMES, got, ref):
        a = host(a) if isinstance(a, torch.Tensor) else np.asarray(a)
        rl = rel_l2(a, b)
        mx = float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1.0 if not np.any(b) else 1e-30))
        print(f"{tag} {name}: rel-l2 {rl:.2e} max-err/max-ref {mx:.2e}", flush=True)
        assert rl <= GRAD_TOL, name
        assert mx <= 2 * GRAD_TOL, name


@pytest.mark.parametrize("case", list(GDN_CASES))
def test_gdn_bwd_matches_oracle(case):
    make, H, Hv, dk, dv, dtype, chunk = GDN_CASES[case]
    seqs, groups = make()
    print(f"\n[case] gdn bwd {case}", flush=True)
    po, plan, (q, k, v, g, beta, do), grads = _gdn_bwd_case(seqs, groups, H, Hv, dk, dv, dtype, chunk)
    ref = OS.gdn_tree_backward(host(q), host(k), host(v), host(g), host(beta), po["par"], host(do))
    _check_grads(case, grads, ref)


def test_gdn_bwd_multistep_full_size_tree():
    """The multistep batch (T = 28672) with 16 q/k and 32 v heads of 128,
    bf16. The oracle runs whole tree 3 on q/k head 7 and the two v-heads that
    read it (14, 15), which gives that head's dq and dk in full."""
    seqs, groups = workloads.sequences("multistep")
    H, Hv, d = 16, 32, 128
    po, plan, (q, k, v, g, beta, do), grads = _gdn_bwd_case(seqs, groups, H, Hv, d, d, "bf16", 64, seed=3)
    ts, te = int(po["tree_start"][3]), int(po["tree_start"][4])
    par = po["par"][ts:te].copy()
    par[par >= 0] -= ts
    hk, hvs = 7, slice(14, 16)
    ref = OS.gdn_tree_backward(host(q[ts:te, hk:hk + 1]), host(k[ts:te, hk:hk + 1]), host(v[ts:te, hvs]),
                               host(g[ts:te, hvs]), host(beta[ts:te, hvs]), par, host(do[ts:te, hvs]))
    dq, dk_, dv_, dg, db = grads
    got = (dq[ts:te, hk:hk + 1], dk_[ts:te, hk:hk + 1], dv_[ts:te, hvs], dg[ts:te, hvs], db[ts:te, hvs])
    _check_grads(f"tree 3 ({te - ts} tokens), q/k head {hk}", got, ref)


def test_gdn_bwd_deterministic():
    seqs, groups = workloads.random_forest(12, [500, 300])
    *_, g1 = _gdn_bwd_case(seqs, groups, 2, 4, 128, 128, "bf16", 16)
    *_, g2 = _gdn_bwd_case(seqs, groups, 2, 4, 128, 128, "bf16", 16)
    for name, a, b in zip(GRAD_NAMES, g1, g2):
        assert torch.equal(a, b), name


def _leaf_path(par, leaf):
    path = [int(leaf)]
    while par[path[-1]] >= 0:
        path.append(int(par[path[-1]]))
    return np.array(path[::-1])


@pytest.mark.parametrize("chunk", [64, 16])
def test_gdn_max_size_tree_one_path(chunk):
    """The largest tree (agentic_l: 131072 tokens, 204 nodes, 124 chains on 7
    levels) with dO nonzero on one root-to-leaf path only. The outputs of the
    path and every gradient are then those of that path run alone as one
    sequence (the oracle's per-token recurrence on it); every token off the
    path gets exactly zero gradient, since no output it reaches has a
    gradient (no leakage between sibling branches)."""
    seqs, groups = workloads.sequences("agentic_l")
    p, po = _pack(seqs, groups)
    par = po["par"]
    T, H, Hv, d = p["T"], 2, 4, 64
    plan = ta.tree_gdn_plan(p["node_start"], p["node_end"], p["node_parent"], chunk)
    q, k, v, g, beta = workloads.gdn_inputs(T, H, Hv, d, d, "bf16", 5, device="cuda")
    has_child = np.zeros(T, bool)
    has_child[par[par >= 0]] = True
    leaves = np.nonzero(~has_child)[0]
    path = _leaf_path(par, leaves[len(leaves) // 3])
    on = torch.zeros(T, dtype=torch.bool)
    on[torch.from_numpy(path)] = True
    do = workloads.gdn_dout(T, Hv, d, "bf16", 5, device="cuda")
    do[~on.cuda()] = 0
    ws = ta.gdn_workspace(q, v, plan, backward=True)
    o = ta.tree_gdn_fwd(q, k, v, g, beta, plan, workspace=ws)
    grads = ta.tree_gdn_bwd(q, k, v, g, beta, do, plan, ws)
    torch.cuda.synchronize()
    print(f"\n[case] agentic_l chunk {chunk}: {int(plan[0])} chunks, {int(plan[1])} chains, {int(plan[2])} levels, "
          f"path of {len(path)} tokens", flush=True)
    chain = np.arange(len(path)) - 1
    sel = lambda t: host(t[torch.from_numpy(path).cuda()])
    ro = OS.gdn_tree(sel(q), sel(k), sel(v), sel(g), sel(beta), chain)
    assert out_err(sel(o), ro) <= OUT_TOL and rel_l2(sel(o), ro) <= 1e-2
    ref = OS.gdn_tree_backward(sel(q), sel(k), sel(v), sel(g), sel(beta), chain, sel(do))
    _check_grads(f"agentic_l chunk {chunk} path", [sel(x) for x in grads], ref)
    off = ~on.cuda()
    for name, x in zip(GRAD_NAMES, grads):
        assert float(x[off].abs().max()) == 0.0, name
