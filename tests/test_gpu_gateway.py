"""GPU parity of tree_attn_gw_fwd / tree_attn_gw_bwd (attention of a child
partition over cached ancestor rows, "Tree Training" §3.3, App. B.2-B.5)
against the float64 gateway oracle, which is itself pinned to the unsplit
tree in test_oracle_gateway.py. On the GPU side the cached rows come from
tree_attn_gw_export and the cached-row gradients go back through
tree_attn_gw_relay; the oracle does its own RoPE.

Tolerances as for plain tree attention: O and LSE max-abs <= 2e-2; dQ, dK,
dV, dK_past, dV_past relative L2 <= 5e-2.
"""
import numpy as np
import pytest
import torch

import tree_packed_attention_amd as ta
import workloads
from oracle import attention as OA
from oracle import gateway as GW
from oracle import pack as OP
from test_gpu_attention import GRAD_TOL, LSE_TOL, O_TOL, host, max_abs, rel_l2

pytestmark = pytest.mark.gpu
THETA = 10000.0


def _subtree_ends(par):
    se = np.arange(1, len(par) + 1, dtype=np.int64)
    for i in range(len(par) - 1, -1, -1):
        if par[i] >= 0:
            se[par[i]] = max(se[par[i]], se[i])
    return se


def _pick_child(par, min_sub=64, min_past=129):
    """A cut whose gateway needs padding (past_len not a multiple of 128)
    and whose child partition spans several tiles."""
    par = np.asarray(par)
    se = _subtree_ends(par)
    best = None
    for c in range(len(par)):
        if par[c] < 0 or se[c] - c < min_sub:
            continue
        sp = GW.split_at(par, c)
        if sp["past_len"] >= min_past and sp["past_len"] % 128 != 0 and not sp["visible"].all():
            return c
        best = c if best is None else best
    return best


def _setup(seqs, groups, Hq, Hkv, d, dtype, seed, children):
    po = OP.pack(seqs, groups)
    par, pos = np.asarray(po["par"]), np.asarray(po["pos"])
    q, k, v, do = workloads.dense_inputs(len(par), Hq, Hkv, d, dtype, seed)
    sp = GW.split_at(par, children)
    P, e = sp["parent_rows"], sp["past_len"]
    # the oracle rotates the cached keys itself; the GPU side takes them from
    # the parent's tensors with tree_attn_gw_export (see _gpu)
    kp = torch.from_numpy(OA.rope(k[P[:e]].double().numpy(), pos[P[:e]], THETA))
    vp = v[P[:e]].clone()
    vis = torch.from_numpy(sp["visible"].astype(np.uint8))
    parts = []
    for C, cpar in zip(sp["child_rows"], sp["child_par"]):
        parts.append(dict(q=q[C].contiguous(), k=k[C].contiguous(), v=v[C].contiguous(), do=do[C].contiguous(),
                          par=cpar, pos=GW._depths(cpar).astype(np.int32), se=_subtree_ends(cpar).astype(np.int32)))
    return dict(sp=sp, k_past=kp, v_past=vp, vis=vis, parts=parts, k=k, v=v, pos=pos.astype(np.int32),
                past_rows=np.asarray(P[:e], np.int32))


def _export(s):
    """The cached rows as a parent partition hands them over: the library
    exports them from the whole tree's k and v at the tree's positions."""
    rows = torch.from_numpy(s["past_rows"]).cuda()
    return ta.tree_attn_gw_export(s["k"].cuda(), s["v"].cuda(), torch.from_numpy(s["pos"]).cuda(), rows, 0, THETA)


def _gpu(part, s, accumulate=False, dk_past=None, dv_past=None):
    c = lambda t: t.cuda()
    pos = torch.from_numpy(part["pos"]).cuda()
    se = torch.from_numpy(part["se"]).cuda()
    q, k, v, do = c(part["q"]), c(part["k"]), c(part["v"]), c(part["do"])
    kp, vp = _export(s)
    vis = c(s["vis"])
    off = s["sp"]["pos_offset"]
    o, lse, ws = ta.tree_attn_gw_fwd(q, k, v, pos, se, off, kp, vp, vis, rope_theta=THETA, with_bwd_workspace=True)
    g = ta.tree_attn_gw_bwd(q, k, v, o, lse, do, pos, se, off, kp, vp, vis, rope_theta=THETA, workspace=ws,
                            reuse_prep=True, dk_past=dk_past, dv_past=dv_past, accumulate=accumulate)
    torch.cuda.synchronize()
    return (o, lse) + tuple(g)


def _oracle(part, s):
    f = lambda t: t.double().numpy()
    args = (f(part["q"]), f(part["k"]), f(part["v"]))
    # the oracle's cached keys: rotated in float64 and rounded to the input
    # precision, as the parent's prep stores them
    s = dict(s, k_past=s["k_past"].to(part["q"].dtype))
    O, LSE = GW.forward(*args, part["par"], f(s["k_past"]), f(s["v_past"]), s["sp"]["visible"],
                        s["sp"]["pos_offset"], theta=THETA)
    grads = GW.backward(*args, f(part["do"]), part["par"], f(s["k_past"]), f(s["v_past"]), s["sp"]["visible"],
                        s["sp"]["pos_offset"], theta=THETA)
    return (O, LSE) + tuple(grads)


def _check(gpu, ref, name):
    o, lse = host(gpu[0]), host(gpu[1])
    errs = dict(o=max_abs(o, ref[0]), lse=max_abs(lse, ref[1]))
    for n, a, b in zip(("dq", "dk", "dv", "dk_past", "dv_past"), gpu[2:], ref[2:]):
        errs[n] = rel_l2(host(a), b)
    print(name, {k: f"{x:.2e}" for k, x in errs.items()}, flush=True)
    assert errs["o"] <= O_TOL and errs["lse"] <= LSE_TOL, errs
    for n in ("dq", "dk", "dv", "dk_past", "dv_past"):
        assert errs[n] <= GRAD_TOL, (n, errs)


CASES = {
    "forest_gqa4_d128": (lambda: workloads.random_forest(31, [700]), 8, 2, 128, "bf16", 31),
    "tree_mha_d64": (lambda: workloads.random_forest(32, [520]), 4, 4, 64, "bf16", 32),
    "tree_d16": (lambda: workloads.random_forest(33, [400]), 2, 1, 16, "bf16", 33),
    "tree_f32_d64": (lambda: workloads.random_forest(34, [450]), 2, 2, 64, "f32", 34),
}


@pytest.mark.parametrize("case", list(CASES))
def test_child_partition_matches_oracle(case):
    make, Hq, Hkv, d, dtype, seed = CASES[case]
    seqs, groups = make()
    par = np.asarray(OP.pack(seqs, groups)["par"])
    child = _pick_child(par)
    print(f"\n[case] {case} child={child}", flush=True)
    s = _setup(seqs, groups, Hq, Hkv, d, dtype, seed, child)
    print("past_len", s["sp"]["past_len"], "visible", int(s["sp"]["visible"].sum()), "T", len(s["parts"][0]["par"]),
          flush=True)
    _check(_gpu(s["parts"][0], s), _oracle(s["parts"][0], s), case)


def test_long_prompt_gateway_full_size_heads():
    """The multi-step shape: a 1024-token prompt cached, one 400-token
    trajectory as the child partition, 32 q / 8 kv heads, d = 128."""
    prompt = list(range(1024))
    seqs = [prompt + [20000 + 1000 * b + j for j in range(400)] for b in range(3)]
    par = np.asarray(OP.pack(seqs, None)["par"])
    child = 1024  # first token of the first trajectory
    assert par[child] == 1023
    print("\n[case] long_prompt", flush=True)
    s = _setup(seqs, None, 32, 8, 128, "bf16", 41, child)
    assert s["sp"]["past_len"] == 1024 and s["sp"]["visible"].all() and s["sp"]["pos_offset"] == 1024
    _check(_gpu(s["parts"][0], s), _oracle(s["parts"][0], s), "long_prompt")


def test_gateway_with_cut_key_tiles():
    """A 1024-token prompt cached over a 2000-token chain (4 q / 1 kv head,
    d = 128): each key tile of the cached rows carries 32 query blocks per
    head (128 iterations), over the per-CU share of the dK/dV work (C = 66),
    so dK_past / dV_past of those rows, and dK / dV of the chain's first
    keys, come from the summed partials of cut tiles."""
    prompt = list(range(1024))
    seqs = [prompt + [20000 + j for j in range(2000)], prompt + [30000 + j for j in range(64)]]
    par = np.asarray(OP.pack(seqs, None)["par"])
    child = 1024
    assert par[child] == 1023
    print("\n[case] cut_gateway", flush=True)
    s = _setup(seqs, None, 4, 1, 128, "bf16", 43, child)
    assert s["sp"]["past_len"] == 1024 and len(s["parts"][0]["par"]) == 2000
    _check(_gpu(s["parts"][0], s), _oracle(s["parts"][0], s), "cut_gateway")


def test_two_children_accumulate_into_the_gateway():
    """Eq. 18: the second child's cached-row gradients add to the first's."""
    seqs, groups = workloads.random_forest(35, [600])
    par = np.asarray(OP.pack(seqs, groups)["par"])
    se = _subtree_ends(par)
    kids = {}
    for i, p in enumerate(par):
        if p >= 0 and se[i] - i >= 16:
            kids.setdefault(int(p), []).append(i)
    cut_kids = max((v for v in kids.values() if len(v) >= 2), key=lambda v: GW.split_at(par, v[:2])["past_len"])
    print(f"\n[case] two children {cut_kids[:2]}", flush=True)
    s = _setup(seqs, groups, 4, 2, 128, "bf16", 35, cut_kids[:2])
    g1 = _gpu(s["parts"][0], s)
    g2 = _gpu(s["parts"][1], s, accumulate=True, dk_past=g1[5].clone(), dv_past=g1[6].clone())
    r1, r2 = _oracle(s["parts"][0], s), _oracle(s["parts"][1], s)
    assert rel_l2(host(g2[5]), r1[5] + r2[5]) <= GRAD_TOL
    assert rel_l2(host(g2[6]), r1[6] + r2[6]) <= GRAD_TOL
    # the accumulated rows are exactly the float32 sum of the two calls
    g2_alone = _gpu(s["parts"][1], s)
    assert torch.equal(g2[5], g1[5] + g2_alone[5]) and torch.equal(g2[6], g1[6] + g2_alone[6])
    _check(g2[:5] + g2_alone[5:], r2, "second child")


def test_empty_gateway_is_the_plain_entry_point_bitwise():
    seqs, groups = workloads.random_forest(36, [300, 120])
    p = ta.tree_pack(seqs, groups)
    q, k, v, do = workloads.dense_inputs(p["T"], 4, 2, 128, "bf16", 36, device="cuda")
    pos = torch.from_numpy(p["pos"]).cuda()
    se = torch.from_numpy(p["subtree_end"]).cuda()
    z = torch.zeros(0, 2, 128, dtype=torch.bfloat16, device="cuda")
    zv = torch.zeros(0, dtype=torch.uint8, device="cuda")
    o1, l1, ws1 = ta.tree_attn_fwd(q, k, v, pos, se, with_bwd_workspace=True)
    g1 = ta.tree_attn_bwd(q, k, v, o1, l1, do, pos, se, workspace=ws1, reuse_prep=True)
    o2, l2, ws2 = ta.tree_attn_gw_fwd(q, k, v, pos, se, 0, z, z, zv, with_bwd_workspace=True)
    g2 = ta.tree_attn_gw_bwd(q, k, v, o2, l2, do, pos, se, 0, z, z, zv, workspace=ws2, reuse_prep=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2[:3]):
        assert torch.equal(a, b)


def test_masked_gateway_rows_get_no_gradient_and_no_weight():
    """All cached rows masked: the child is plain tree attention (at any
    pos_offset, RoPE being relative) and the cached rows' gradients are 0."""
    seqs, groups = workloads.random_forest(37, [260])
    p = ta.tree_pack(seqs, groups)
    T = p["T"]
    q, k, v, do = workloads.dense_inputs(T, 4, 2, 64, "bf16", 37, device="cuda")
    pos = torch.from_numpy(p["pos"]).cuda()
    se = torch.from_numpy(p["subtree_end"]).cuda()
    g = torch.Generator().manual_seed(37)
    kp = torch.randn(150, 2, 64, generator=g).to(torch.bfloat16).cuda()
    vp = torch.randn(150, 2, 64, generator=g).to(torch.bfloat16).cuda()
    vis = torch.zeros(150, dtype=torch.uint8, device="cuda")
    o, lse, ws = ta.tree_attn_gw_fwd(q, k, v, pos, se, 77, kp, vp, vis, with_bwd_workspace=True)
    dq, dk, dv, dkp, dvp = ta.tree_attn_gw_bwd(q, k, v, o, lse, do, pos, se, 77, kp, vp, vis, workspace=ws,
                                               reuse_prep=True)
    torch.cuda.synchronize()
    f = lambda t: host(t).astype(np.float64)
    O, LSE = OA.forward_branches(f(q), f(k), f(v), p["parent"], p["pos"])
    rq, rk, rv = OA.backward_branches(f(q), f(k), f(v), f(do), p["parent"], p["pos"])
    assert max_abs(host(o), O) <= O_TOL and max_abs(host(lse), LSE) <= LSE_TOL
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        assert rel_l2(host(a), b) <= GRAD_TOL
    assert not dkp.any() and not dvp.any()


# ----------------------------------------------------------------- planned partitions end to end


def _run_partitioned(seqs, groups, Hq, Hkv, d, dtype, seed, capacity):
    """Plans the packed tree with tree_partition and runs every partition on
    the GPU with its own device tensors, in plan order (parents first):
    tree-root partitions through the plain entry points, the others through
    the gateway of their cut token's ancestors (the cut token included, all
    visible) at pos_offset = its depth + 1. The gateway rows are built with
    tree_attn_gw_export from each ancestor partition that holds part of the
    chain, and after every backward their float32 gradients go back with
    tree_attn_gw_relay into those partitions' dK, dV (Tree Training App. B.2,
    B.5, Eq. 18). Only library calls touch the data on the GPU side. Returns
    the assembled outputs and the plan."""
    p = ta.tree_pack(seqs, groups)
    T = p["T"]
    par, pos = p["parent"], p["pos"]
    q, k, v, do = workloads.dense_inputs(T, Hq, Hkv, d, dtype, seed)
    plan = ta.tree_partition(p["node_start"], p["node_end"], p["node_parent"], capacity)
    node_of = np.repeat(np.arange(p["n_nodes"]), p["node_end"] - p["node_start"])
    tok_part = plan["node_part"][node_of]
    loc = -np.ones(T, np.int64)  # token -> index inside its own partition
    parts = []
    for b in range(len(plan["part_tokens"])):
        R = np.nonzero(tok_part == b)[0]
        loc[R] = np.arange(len(R))
        inside = (par[R] >= 0) & (tok_part[np.maximum(par[R], 0)] == b)  # parent in this partition
        lpar = np.where(inside, loc[np.maximum(par[R], 0)], -1)
        cutn = int(plan["part_cut"][b])
        off = 0 if cutn < 0 else int(pos[p["node_end"][cutn] - 1]) + 1
        lpos = (pos[R] - off).astype(np.int32)
        assert np.all(lpos[lpar < 0] == 0)
        c = lambda t: t[torch.as_tensor(R)].contiguous().cuda()
        parts.append(dict(R=R, off=off, cut=cutn, q=c(q), k=c(k), v=c(v), do=c(do),
                          pos=torch.from_numpy(lpos).cuda(), se=torch.from_numpy(_subtree_ends(lpar).astype(np.int32)).cuda()))
    relays = []
    for b, P in enumerate(parts):
        if P["cut"] < 0:
            o, lse, ws = ta.tree_attn_fwd(P["q"], P["k"], P["v"], P["pos"], P["se"], rope_theta=THETA,
                                          with_bwd_workspace=True)
            g = ta.tree_attn_bwd(P["q"], P["k"], P["v"], o, lse, P["do"], P["pos"], P["se"], rope_theta=THETA,
                                 workspace=ws, reuse_prep=True)
        else:
            A = [int(p["node_end"][P["cut"]] - 1)]
            while par[A[-1]] >= 0:
                A.append(int(par[A[-1]]))
            A = np.array(A[::-1])
            assert len(A) == P["off"]
            kp = torch.empty(len(A), Hkv, d, dtype=q.dtype, device="cuda")
            vp = torch.empty_like(kp)
            pieces = []  # (ancestor partition, first cached row, local rows)
            for a in sorted(set(int(x) for x in tok_part[A])):
                sel = np.nonzero(tok_part[A] == a)[0]
                assert np.array_equal(sel, np.arange(sel[0], sel[-1] + 1))  # a contiguous run of the chain
                rows = torch.as_tensor(loc[A[sel]].astype(np.int32)).cuda()
                Pa = parts[a]
                ta.tree_attn_gw_export(Pa["k"], Pa["v"], Pa["pos"], rows, Pa["off"], THETA,
                                       k_past=kp[sel[0]:sel[-1] + 1], v_past=vp[sel[0]:sel[-1] + 1])
                pieces.append((a, int(sel[0]), int(sel[-1]) + 1, rows))
            vis = torch.ones(len(A), dtype=torch.uint8).cuda()
            o, lse, ws = ta.tree_attn_gw_fwd(P["q"], P["k"], P["v"], P["pos"], P["se"], P["off"], kp, vp, vis,
                                             rope_theta=THETA, with_bwd_workspace=True)
            g = ta.tree_attn_gw_bwd(P["q"], P["k"], P["v"], o, lse, P["do"], P["pos"], P["se"], P["off"], kp, vp, vis,
                                    rope_theta=THETA, workspace=ws, reuse_prep=True)
            relays.append((g[3], g[4], pieces))
        P.update(o=o, lse=lse, dq=g[0], dk=g[1], dv=g[2])
    # every partition's own backward has run: relay the cached rows' gradients
    for dkp, dvp, pieces in relays:
        for a, r0, r1, rows in pieces:
            Pa = parts[a]
            ta.tree_attn_gw_relay(dkp[r0:r1].contiguous(), dvp[r0:r1].contiguous(), rows, Pa["pos"], Pa["dk"],
                                  Pa["dv"], Pa["off"], THETA)
    torch.cuda.synchronize()
    O = np.zeros((T, Hq, d))
    LSE = np.zeros((Hq, T))
    dq = np.zeros((T, Hq, d))
    dk = np.zeros((T, Hkv, d))
    dv = np.zeros((T, Hkv, d))
    for P in parts:
        R = P["R"]
        O[R], LSE[:, R], dq[R], dk[R], dv[R] = host(P["o"]), host(P["lse"]), host(P["dq"]), host(P["dk"]), host(P["dv"])
    return dict(p=p, plan=plan, q=q, k=k, v=v, do=do, O=O, LSE=LSE, dq=dq, dk=dk, dv=dv)


def test_export_is_the_prep_rotation_and_relay_adds_the_rotated_gradient():
    """tree_attn_gw_export rotates rows at pos_offset + pos as the oracle's
    RoPE does, and copies the values; the relay adds the transposed rotation
    of the float32 gradient (checked against its definition on the oracle's
    rotation). A child partition of one token under a gateway exported from
    its ancestor chain reproduces that token appended to the unsplit tree."""
    rng = np.random.default_rng(3)
    T, Hkv, d, off = 300, 2, 64, 37
    seqs, groups = workloads.random_forest(12, [T])
    pk = ta.tree_pack(seqs, groups)
    T = pk["T"]
    _, k, v, _ = workloads.dense_inputs(T, 2, Hkv, d, "bf16", 9, device="cuda")
    pos = torch.from_numpy(pk["pos"]).cuda()
    rows_np = rng.permutation(T)[:120].astype(np.int32)
    rows = torch.as_tensor(rows_np).cuda()
    kp, vp = ta.tree_attn_gw_export(k, v, pos, rows, off, THETA)
    torch.cuda.synchronize()
    ref = OA.rope(host(k)[rows_np].astype(np.float64), pk["pos"][rows_np] + off, THETA)
    assert max_abs(host(kp), ref) <= 2e-2 and torch.equal(vp, v[rows.long()])
    # relay: dk += R^T g, dv += h, in float32 then rounded once
    g = torch.randn(120, Hkv, d, device="cuda")
    h = torch.randn(120, Hkv, d, device="cuda")
    dk0 = torch.randn(T, Hkv, d, device="cuda").to(torch.bfloat16)
    dv0 = torch.randn(T, Hkv, d, device="cuda").to(torch.bfloat16)
    dk, dv = dk0.clone(), dv0.clone()
    ta.tree_attn_gw_relay(g, h, rows, pos, dk, dv, off, THETA)
    torch.cuda.synchronize()
    exp_k = host(dk0).astype(np.float64)
    exp_v = host(dv0).astype(np.float64)
    exp_k[rows_np] += OA.rope_transpose(host(g).astype(np.float64), pk["pos"][rows_np] + off, THETA)
    exp_v[rows_np] += host(h)
    assert max_abs(host(dk), exp_k) <= 3e-2 and max_abs(host(dv), exp_v) <= 3e-2
    untouched = np.setdiff1d(np.arange(T), rows_np)
    assert np.array_equal(host(dk)[untouched], host(dk0)[untouched])
    # the exported keys are the ones the attention prep rotates: a child of
    # one token under a gateway of the partition's whole ancestor chain at
    # this offset sees exactly the rotated keys of the unsplit layout
    chain = np.array(sorted(set(OP.ancestors_or_self(pk["parent"], T - 1))), np.int32)
    kc, vc = ta.tree_attn_gw_export(k, v, pos, torch.as_tensor(chain).cuda(), 0, THETA)
    qx = torch.randn(1, 2, d, device="cuda").to(torch.bfloat16)
    kx = torch.randn(1, Hkv, d, device="cuda").to(torch.bfloat16)
    vx = torch.randn(1, Hkv, d, device="cuda").to(torch.bfloat16)
    one = torch.zeros(1, dtype=torch.int32, device="cuda")
    ox, lx, _ = ta.tree_attn_gw_fwd(qx, kx, vx, one, one + 1, len(chain), kc, vc,
                                    torch.ones(len(chain), dtype=torch.uint8, device="cuda"), rope_theta=THETA)
    # the same token appended under T - 1 in the unsplit tree
    qf = torch.zeros(T + 1, 2, d, dtype=torch.bfloat16, device="cuda")
    qf[T] = qx[0]
    kf = torch.cat([k, kx]).contiguous()
    vf = torch.cat([v, vx]).contiguous()
    posf = torch.cat([pos, pos[T - 1:T] + 1]).contiguous()
    sef = torch.from_numpy(np.append(np.where(np.isin(np.arange(T), chain), T + 1, pk["subtree_end"]),
                                     T + 1).astype(np.int32)).cuda()
    of, lf, _ = ta.tree_attn_fwd(qf, kf, vf, posf, sef, rope_theta=THETA)
    torch.cuda.synchronize()
    # the two runs tile and sum the same visible keys in another order, so
    # the float32 LSE may differ in its last bits; a key rotated differently
    # by even one bf16 unit would move it by far more
    assert torch.equal(ox[0], of[T])
    assert float((lx[:, 0] - lf[:, T]).abs().max()) <= 1e-5


@pytest.mark.parametrize("capacity", [600, 1500])
def test_planned_partitions_reproduce_the_unsplit_tree(capacity):
    """A 3000-token tree (depth <= 6) cut by tree_partition into partitions of
    at most `capacity` tokens, several levels deep; the assembled result
    equals the oracle on the unsplit tree."""
    seqs, groups = workloads.random_tree(41, 6, 3000, 16, 300)
    print(f"\n[case] planned partitions, capacity {capacity}", flush=True)
    r = _run_partitioned(seqs, groups, 8, 2, 128, "bf16", 41, capacity)
    plan = r["plan"]
    depth = 0
    for b in range(len(plan["part_parent"])):
        lvl, x = 0, b
        while plan["part_parent"][x] >= 0:
            x, lvl = plan["part_parent"][x], lvl + 1
        depth = max(depth, lvl)
    print(f"partitions {len(plan['part_tokens'])}, levels {depth + 1}", flush=True)
    assert len(plan["part_tokens"]) >= 3 and depth >= 1
    po = OP.pack(seqs, groups)
    qn, kn, vn, don = host(r["q"]), host(r["k"]), host(r["v"]), host(r["do"])
    O, LSE = OA.forward_branches(qn, kn, vn, po["par"], po["pos"])
    rdq, rdk, rdv = OA.backward_branches(qn, kn, vn, don, po["par"], po["pos"])
    errs = dict(o=max_abs(r["O"], O), lse=max_abs(r["LSE"], LSE), dq=rel_l2(r["dq"], rdq), dk=rel_l2(r["dk"], rdk),
                dv=rel_l2(r["dv"], rdv))
    print({k: f"{x:.2e}" for k, x in errs.items()}, flush=True)
    assert errs["o"] <= O_TOL and errs["lse"] <= LSE_TOL
    assert errs["dq"] <= GRAD_TOL and errs["dk"] <= GRAD_TOL and errs["dv"] <= GRAD_TOL
