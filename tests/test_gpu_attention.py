"""GPU parity of tree_attn_fwd / tree_attn_bwd against the float64 oracle.

Tolerances (the stated targets): O and LSE max-abs <= 2e-2; dQ, dK, dV relative
L2 <= 5e-2. Small cases compare every element with the per-branch oracle;
full-size workloads compare every row and key of whole kv groups with the
whole-tree ancestor-chain oracle (on the largest tree, with the upstream
gradient on two heads of the group), plus sampled rows on all heads.
"""
import numpy as np
import pytest
import torch

import tree_packed_attention_amd as ta
import workloads
from oracle import attention as OA
from oracle import pack as OP

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_TOL = 2e-2
GRAD_TOL = 5e-2


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def rel_l2(a, b):
    """Relative L2 error; where the exact gradient is identically zero (one
    visible key per query makes dS = 0), relative error is undefined and the
    absolute max error is returned, to be held to the forward tolerance."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    if nb <= 1e-9 * np.sqrt(b.size):
        err = float(np.max(np.abs(a - b))) if a.size else 0.0
        return err * (GRAD_TOL / O_TOL)
    return float(np.linalg.norm(a - b) / nb)


def host(t):
    return t.detach().float().cpu().numpy()


def run_gpu(seqs, groups, Hq, Hkv, d, dtype, seed, theta=10000.0):
    p = ta.tree_pack(seqs, groups)
    T = p["T"]
    q, k, v, do = workloads.dense_inputs(T, Hq, Hkv, d, dtype, seed, device="cuda")
    pos = torch.from_numpy(p["pos"]).cuda()
    se = torch.from_numpy(p["subtree_end"]).cuda()
    o, lse, ws = ta.tree_attn_fwd(q, k, v, pos, se, rope_theta=theta, with_bwd_workspace=True)
    dq, dk, dv = ta.tree_attn_bwd(q, k, v, o, lse, do, pos, se, rope_theta=theta, workspace=ws, reuse_prep=True)
    torch.cuda.synchronize()
    return dict(p=p, q=q, k=k, v=v, do=do, o=o, lse=lse, dq=dq, dk=dk, dv=dv, pos=pos, se=se)


SMALL_CASES = {
    "trie_page_example": (lambda: workloads.sequences("ex_a"), 1, 1, 16, "f32"),
    "prefix_merge_example": (lambda: workloads.sequences("ex_b"), 1, 1, 16, "f32"),
    "forest_ragged_gqa4": (lambda: workloads.random_forest(3, [333, 250, 97]), 8, 2, 128, "bf16"),
    "forest_d64_mha": (lambda: workloads.random_forest(4, [200, 190]), 4, 4, 64, "bf16"),
    "forest_d16": (lambda: workloads.random_forest(5, [150, 77]), 2, 1, 16, "bf16"),
    "forest_f32_d64": (lambda: workloads.random_forest(6, [260, 41]), 2, 2, 64, "f32"),
    "chain_causal": (lambda: ([list(range(200))], [0]), 2, 1, 128, "bf16"),
    "varlen_disjoint": (lambda: ([[1000 + i] + list(range(40 + 23 * i)) for i in range(5)], None), 4, 2, 128, "bf16"),
    "single_token": (lambda: ([[5]], None), 2, 1, 128, "bf16"),
    "deep_tree_gqa8": (lambda: workloads.random_tree(11, 6, 1500, 16, 200), 16, 2, 128, "bf16"),
}


@pytest.mark.parametrize("case", list(SMALL_CASES))
def test_small_cases_full_oracle(case):
    make, Hq, Hkv, d, dtype = SMALL_CASES[case]
    seqs, groups = make()
    print(f"\n[case] {case}", flush=True)
    r = run_gpu(seqs, groups, Hq, Hkv, d, dtype, seed=17)
    po = OP.pack(seqs, groups)
    qn, kn, vn, don = host(r["q"]), host(r["k"]), host(r["v"]), host(r["do"])
    O, LSE = OA.forward_branches(qn, kn, vn, po["par"], po["pos"])
    dq, dk, dv = OA.backward_branches(qn, kn, vn, don, po["par"], po["pos"])
    errs = dict(o=max_abs(host(r["o"]), O), lse=max_abs(host(r["lse"]), LSE), dq=rel_l2(host(r["dq"]), dq),
                dk=rel_l2(host(r["dk"]), dk), dv=rel_l2(host(r["dv"]), dv))
    print(case, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs["o"] <= O_TOL and errs["lse"] <= LSE_TOL
    assert errs["dq"] <= GRAD_TOL and errs["dk"] <= GRAD_TOL and errs["dv"] <= GRAD_TOL


def test_short_prompt_group_full():
    """8 trees of 256-token prompt + 4 x 128-token branches, 32q/8kv, d=128."""
    seqs, groups = workloads.sequences("short")
    c = workloads.WORKLOADS["short"]
    r = run_gpu(seqs, groups, c["Hq"], c["Hkv"], c["d"], c["dtype"], c["seed"])
    po = OP.pack(seqs, groups)
    qn, kn, vn, don = host(r["q"]), host(r["k"]), host(r["v"]), host(r["do"])
    O, LSE = OA.forward_branches(qn, kn, vn, po["par"], po["pos"])
    assert max_abs(host(r["o"]), O) <= O_TOL
    assert max_abs(host(r["lse"]), LSE) <= LSE_TOL
    dq, dk, dv = OA.backward_branches(qn, kn, vn, don, po["par"], po["pos"])
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert rel_l2(host(r[name]), ref) <= GRAD_TOL, name


def _check_group(r, po, c, hk, q_heads=None):
    """Every row and key of kv group hk against the whole-tree ancestor-chain
    oracle: O, LSE and dQ of its q heads (or of those listed), dK and dV."""
    G = c["Hq"] // c["Hkv"]
    hs = slice(hk * G, (hk + 1) * G)
    heads = list(range(hk * G, (hk + 1) * G)) if q_heads is None else list(q_heads)
    qn, kn, vn, don = host(r["q"][:, hs]), host(r["k"][:, hk:hk + 1]), host(r["v"][:, hk:hk + 1]), host(r["do"][:, hs])
    rel = [h - hk * G for h in heads]
    O, LSE = OA.forward_chains(qn, kn, vn, po["par"], q_heads=rel)
    assert max_abs(host(r["o"][:, heads]), O) <= O_TOL
    assert max_abs(host(r["lse"][heads]), LSE) <= LSE_TOL
    dq, dk, dv = OA.backward_chains(qn, kn, vn, don, po["par"], q_heads=rel)
    errs = dict(dq=rel_l2(host(r["dq"][:, heads]), dq), dk=rel_l2(host(r["dk"][:, hk:hk + 1]), dk),
                dv=rel_l2(host(r["dv"][:, hk:hk + 1]), dv))
    print(f"kv group {hk} heads {heads[0]}..{heads[-1]}: {', '.join(f'{k} {v:.2e}' for k, v in errs.items())}",
          flush=True)
    assert max(errs.values()) <= GRAD_TOL, errs
    return dk, dv


def test_multistep_batch_whole_kv_groups():
    """Long prompt, multi-step trajectories (4 trees, 28672 tokens, 32q/8kv):
    every row and key of the whole batch for kv groups 0 and 7."""
    seqs, groups = workloads.sequences("multistep")
    c = workloads.WORKLOADS["multistep"]
    r = run_gpu(seqs, groups, c["Hq"], c["Hkv"], c["d"], c["dtype"], c["seed"])
    po = OP.pack(seqs, groups)
    for hk in (0, c["Hkv"] - 1):
        _check_group(r, po, c, hk)


def _heavy_keys(po):
    """The keys with the most descendants: the root segment and every key
    whose subtree holds more than a tenth of the tree (the fork points of the
    upper levels)."""
    size = po["se"] - np.arange(po["T"])
    return np.nonzero(size > po["T"] // 10)[0]


def test_random_agentic_tree_whole_kv_group():
    """Random agentic tree (32768 tokens, depth <= 6, 64q/8kv, d=128) at full
    size: every row and key of kv group 0 (its 8 q heads) element-wise,
    including the root segment and fork keys that gather gradients from
    thousands of descendants."""
    seqs, groups = workloads.sequences("agentic")
    c = workloads.WORKLOADS["agentic"]
    r = run_gpu(seqs, groups, c["Hq"], c["Hkv"], c["d"], c["dtype"], c["seed"])
    po = OP.pack(seqs, groups)
    dk, dv = _check_group(r, po, c, 0)
    heavy = _heavy_keys(po)
    assert len(heavy) > 1000
    assert rel_l2(host(r["dk"][:, :1])[heavy], dk[heavy]) <= GRAD_TOL
    assert rel_l2(host(r["dv"][:, :1])[heavy], dv[heavy]) <= GRAD_TOL


def test_random_agentic_tree_large_whole_kv_group():
    """Large random tree (131072 tokens, depth <= 10, 64q/8kv, d=128) at full
    size. The upstream gradient is the workload's on q heads 56 and 63 (the
    first and last head of kv group 7) and zero on the others, so the
    oracle needs two heads while the kernels run all 64 over every block:
    dK and dV of every key of group 7 (root segment and all forks included),
    O, LSE and dQ of every row of heads 56 and 63, element-wise; dQ of the
    zero-gradient heads of the group must be exactly zero. Sampled rows check
    O and LSE on all heads."""
    seqs, groups = workloads.sequences("agentic_l")
    c = workloads.WORKLOADS["agentic_l"]
    p = ta.tree_pack(seqs, groups)
    T = p["T"]
    q, k, v, do = workloads.dense_inputs(T, c["Hq"], c["Hkv"], c["d"], c["dtype"], c["seed"], device="cuda")
    keep = torch.zeros(c["Hq"], dtype=torch.bool, device="cuda")
    keep[[56, 63]] = True
    do = do * keep[None, :, None].to(do.dtype)
    pos = torch.from_numpy(p["pos"]).cuda()
    se = torch.from_numpy(p["subtree_end"]).cuda()
    o, lse, ws = ta.tree_attn_fwd(q, k, v, pos, se, with_bwd_workspace=True)
    dq, dk, dv = ta.tree_attn_bwd(q, k, v, o, lse, do, pos, se, workspace=ws, reuse_prep=True)
    torch.cuda.synchronize()
    assert ta.tree_attn_workspace_status(ws) == 0
    r = dict(q=q, k=k, v=v, do=do, o=o, lse=lse, dq=dq, dk=dk, dv=dv)
    po = OP.pack(seqs, groups)
    dkr, dvr = _check_group(r, po, c, 7, q_heads=[56, 63])
    heavy = _heavy_keys(po)
    assert len(heavy) > 1000
    assert rel_l2(host(dk[:, 7:8])[heavy], dkr[heavy]) <= GRAD_TOL
    assert rel_l2(host(dv[:, 7:8])[heavy], dvr[heavy]) <= GRAD_TOL
    assert torch.count_nonzero(dq[:, 57:63]) == 0
    rng = np.random.default_rng(42)
    rows = _sample_rows(po, 12, rng)
    O, LSE = OA.forward_rows(_Rows(q, rows), host(k), host(v), po["par"], rows)
    rt = torch.as_tensor(rows, device="cuda")
    assert max_abs(host(o[rt]), O) <= O_TOL
    assert max_abs(host(lse[:, rt]), LSE) <= LSE_TOL


class _Rows:
    """Array-like view of selected rows of a [T, H, d] tensor (for the
    per-row oracle functions, which read q[i:i+1] and do[i, h] only)."""

    def __init__(self, t, rows):
        self.idx = {int(x): n for n, x in enumerate(rows)}
        self.data = host(t[torch.as_tensor(np.asarray(rows), device=t.device)])
        self.shape = tuple(t.shape)

    def __getitem__(self, key):
        if isinstance(key, slice):
            n = self.idx[key.start]
            return self.data[n:n + 1]
        i, h = key
        return self.data[self.idx[int(i)], h]


def _sample_rows(po, n, rng):
    T = po["T"]
    fixed = [0, 1, 63, 64, 127, 128, T // 2, T - 129, T - 128, T - 2, T - 1]
    fixed += list(po["node_start"][:: max(1, len(po["node_start"]) // 8)])
    rows = sorted(set(int(x) for x in fixed if 0 <= x < T) | set(int(x) for x in rng.integers(0, T, n)))
    return rows


PLAN_CASES = {
    "forest_ragged": (lambda: workloads.random_forest(3, [333, 250, 97]), 8, 2, 128),
    "deep_tree": (lambda: workloads.random_tree(11, 6, 1500, 16, 200), 4, 1, 64),
    "single_token": (lambda: ([[5]], None), 1, 1, 16),
    "short": (lambda: workloads.sequences("short"), 32, 8, 128),
    "multistep": (lambda: workloads.sequences("multistep"), 32, 8, 128),
    "agentic": (lambda: workloads.sequences("agentic"), 64, 8, 128),
}


@pytest.mark.parametrize("case", list(PLAN_CASES))
def test_device_tile_plan_matches_oracle(case):
    """The tile plan the device builds (per 128-row query tile: 64-key tiles
    visited and those among them taken unmasked) equals the oracle's
    classification of every tile, and the status word stays clear."""
    make, Hq, Hkv, d = PLAN_CASES[case]
    seqs, groups = make()
    p = ta.tree_pack(seqs, groups)
    T = p["T"]
    q, k, v, _ = workloads.dense_inputs(T, Hq, Hkv, d, "bf16", 1, device="cuda")
    o, lse, ws = ta.tree_attn_fwd(q, k, v, torch.from_numpy(p["pos"]).cuda(), torch.from_numpy(p["subtree_end"]).cuda())
    ne, fu = ta.tree_attn_plan_counts(ws, T, Hq, Hkv, d)
    assert ta.tree_attn_workspace_status(ws) == 0
    from oracle import tiles as OT

    one, ofu = OT.tile_counts_per_qtile(OP.pack(seqs, groups)["se"], T, 128, 64)
    n = len(one)
    assert np.array_equal(ne[:n], one) and np.array_equal(fu[:n], ofu)
    assert not ne[n:].any() and not fu[n:].any()
    print(case, "non-empty", int(ne.sum()), "full", int(fu.sum()), flush=True)


def test_bitwise_deterministic_and_reuse_prep():
    seqs, groups = workloads.random_forest(8, [700, 300])
    p = ta.tree_pack(seqs, groups)
    T = p["T"]
    q, k, v, do = workloads.dense_inputs(T, 8, 2, 128, "bf16", 3, device="cuda")
    pos = torch.from_numpy(p["pos"]).cuda()
    se = torch.from_numpy(p["subtree_end"]).cuda()
    outs = []
    for reuse in (False, True, True):
        o, lse, ws = ta.tree_attn_fwd(q, k, v, pos, se, with_bwd_workspace=True)
        g = ta.tree_attn_bwd(q, k, v, o, lse, do, pos, se, workspace=ws, reuse_prep=reuse)
        outs.append([o, lse, *g])
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    for a, b in zip(outs[1], outs[2]):
        assert torch.equal(a, b)


def _star(n_branch, prompt, branch):
    """One prompt shared by n_branch disjoint branches: the prompt's keys see
    every row, so their tiles carry far more dK/dV work than the rest."""
    return [list(range(prompt)) + [10_000 + b * branch + i for i in range(branch)] for b in range(n_branch)], None


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 1)])
def test_dkdv_cut_tiles(Hq, Hkv):
    """128-token prompt + 64 branches of 64 (T = 4224): the prompt's key tile
    has 66 query blocks per head, several times the per-CU share of the
    work, so its dK/dV iterations are cut into chunks whose partial sums a
    second kernel adds. Whole-tensor parity with the per-branch oracle, and
    bitwise equal results on a second backward."""
    seqs, groups = _star(64, 128, 64)
    print(f"\n[case] star Hq={Hq} Hkv={Hkv}", flush=True)
    r = run_gpu(seqs, groups, Hq, Hkv, 128, "bf16", seed=23)
    assert r["p"]["T"] == 4224
    po = OP.pack(seqs, groups)
    qn, kn, vn, don = host(r["q"]), host(r["k"]), host(r["v"]), host(r["do"])
    dq, dk, dv = OA.backward_branches(qn, kn, vn, don, po["par"], po["pos"])
    errs = dict(dq=rel_l2(host(r["dq"]), dq), dk=rel_l2(host(r["dk"]), dk), dv=rel_l2(host(r["dv"]), dv),
                dk_prompt=rel_l2(host(r["dk"])[:128], dk[:128]), dv_prompt=rel_l2(host(r["dv"])[:128], dv[:128]))
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert max(errs.values()) <= GRAD_TOL
    ws = ta.attn_workspace(r["p"]["T"], Hq, Hkv, 128, True, "cuda")
    o, lse, ws = ta.tree_attn_fwd(r["q"], r["k"], r["v"], r["pos"], r["se"], workspace=ws)
    again = ta.tree_attn_bwd(r["q"], r["k"], r["v"], o, lse, r["do"], r["pos"], r["se"], workspace=ws,
                             reuse_prep=True)
    torch.cuda.synchronize()
    for a, b in zip((r["dq"], r["dk"], r["dv"]), again):
        assert torch.equal(a, b)


def test_autograd_function_matches_entry_points():
    seqs, groups = workloads.random_forest(9, [300])
    p = ta.tree_pack(seqs, groups)
    T = p["T"]
    q, k, v, do = workloads.dense_inputs(T, 4, 2, 64, "bf16", 4, device="cuda")
    pos = torch.from_numpy(p["pos"]).cuda()
    se = torch.from_numpy(p["subtree_end"]).cuda()
    qq, kk, vv = (x.clone().requires_grad_(True) for x in (q, k, v))
    o = ta.TreeAttention.apply(qq, kk, vv, pos, se)
    o.backward(do)
    o2, lse2, _ = ta.tree_attn_fwd(q, k, v, pos, se)
    dq2, dk2, dv2 = ta.tree_attn_bwd(q, k, v, o2, lse2, do, pos, se)
    assert torch.equal(o, o2)
    assert torch.equal(qq.grad, dq2) and torch.equal(kk.grad, dk2) and torch.equal(vv.grad, dv2)


def test_no_rope_and_custom_scale():
    seqs, groups = workloads.random_forest(10, [260])
    r = run_gpu(seqs, groups, 2, 1, 64, "bf16", 5, theta=0.0)
    po = OP.pack(seqs, groups)
    # theta = 0 disables RoPE: the oracle rotates by position 0 (identity)
    vis = OP.visibility_dense(po["par"])
    qn, kn, vn, don = host(r["q"]), host(r["k"]), host(r["v"]), host(r["do"])
    O, LSE = OA.forward_dense(qn, kn, vn, vis, np.zeros(po["T"]))
    assert max_abs(host(r["o"]), O) <= O_TOL and max_abs(host(r["lse"]), LSE) <= LSE_TOL
    # backward without RoPE: the per-branch oracle at theta = 0
    dq, dk, dv = OA.backward_branches(qn, kn, vn, don, po["par"], po["pos"], theta=0.0)
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert rel_l2(host(r[name]), ref) <= GRAD_TOL, name
    q, k, v = r["q"], r["k"], r["v"]
    o, lse, ws = ta.tree_attn_fwd(q, k, v, r["pos"], r["se"], softmax_scale=0.05, with_bwd_workspace=True)
    O2, L2 = OA.forward_dense(qn, kn, vn, vis, po["pos"], scale=0.05)
    assert max_abs(host(o), O2) <= O_TOL and max_abs(host(lse), L2) <= LSE_TOL
    # backward at a scale other than 1/sqrt(d), with RoPE, and with both
    for theta in (10000.0, 0.0):
        o, lse, ws = ta.tree_attn_fwd(q, k, v, r["pos"], r["se"], softmax_scale=0.05, rope_theta=theta,
                                      with_bwd_workspace=True)
        g = ta.tree_attn_bwd(q, k, v, o, lse, r["do"], r["pos"], r["se"], softmax_scale=0.05, rope_theta=theta,
                             workspace=ws, reuse_prep=True)
        ref = OA.backward_branches(qn, kn, vn, don, po["par"], po["pos"], scale=0.05, theta=theta)
        for name, a, b in zip(("dq", "dk", "dv"), g, ref):
            assert rel_l2(host(a), b) <= GRAD_TOL, (theta, name)
