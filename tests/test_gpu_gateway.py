"""GPU parity of tree_attn_gw_fwd / tree_attn_gw_bwd (attention of a child
partition over cached ancestor rows, "Tree Training" §3.3, App. B.2-B.5)
against the float64 gateway oracle, which is itself pinned to the unsplit
tree in test_oracle_gateway.py.

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
    kp = torch.from_numpy(OA.rope(k[P[:e]].double().numpy(), pos[P[:e]], THETA)).to(q.dtype)
    vp = v[P[:e]].clone()
    vis = torch.from_numpy(sp["visible"].astype(np.uint8))
    parts = []
    for C, cpar in zip(sp["child_rows"], sp["child_par"]):
        parts.append(dict(q=q[C].contiguous(), k=k[C].contiguous(), v=v[C].contiguous(), do=do[C].contiguous(),
                          par=cpar, pos=GW._depths(cpar).astype(np.int32), se=_subtree_ends(cpar).astype(np.int32)))
    return dict(sp=sp, k_past=kp, v_past=vp, vis=vis, parts=parts)


def _gpu(part, s, accumulate=False, dk_past=None, dv_past=None):
    c = lambda t: t.cuda()
    pos = torch.from_numpy(part["pos"]).cuda()
    se = torch.from_numpy(part["se"]).cuda()
    q, k, v, do = c(part["q"]), c(part["k"]), c(part["v"]), c(part["do"])
    kp, vp, vis = c(s["k_past"]), c(s["v_past"]), c(s["vis"])
    off = s["sp"]["pos_offset"]
    o, lse, ws = ta.tree_attn_gw_fwd(q, k, v, pos, se, off, kp, vp, vis, rope_theta=THETA, with_bwd_workspace=True)
    g = ta.tree_attn_gw_bwd(q, k, v, o, lse, do, pos, se, off, kp, vp, vis, rope_theta=THETA, workspace=ws,
                            reuse_prep=True, dk_past=dk_past, dv_past=dv_past, accumulate=accumulate)
    torch.cuda.synchronize()
    return (o, lse) + tuple(g)


def _oracle(part, s):
    f = lambda t: t.double().numpy()
    args = (f(part["q"]), f(part["k"]), f(part["v"]))
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
