"""GPU parity of tree_attn_fwd / tree_attn_bwd against the float64 oracle.

Tolerances (the stated targets): O and LSE max-abs <= 2e-2; dQ, dK, dV relative
L2 <= 5e-2. Small cases compare every element with the per-branch oracle;
full-size workloads compare every element of selected trees / kv groups, or
sampled rows and keys plus identities that hold at any size.
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


def _tree_slice(po, t):
    ts, te = int(po["tree_start"][t]), int(po["tree_start"][t + 1])
    par = po["par"][ts:te].copy()
    par[par >= 0] -= ts
    return ts, te, par, po["pos"][ts:te]


def test_multistep_trees_full_per_group():
    """Long prompt, multi-step trajectories (4 trees, 28672 tokens, 32q/8kv).
    Whole trees 0 and 3 for kv groups 0 and 7 against the per-branch oracle."""
    seqs, groups = workloads.sequences("multistep")
    c = workloads.WORKLOADS["multistep"]
    r = run_gpu(seqs, groups, c["Hq"], c["Hkv"], c["d"], c["dtype"], c["seed"])
    po = OP.pack(seqs, groups)
    G = c["Hq"] // c["Hkv"]
    for t in (0, 3):
        ts, te, par, pos = _tree_slice(po, t)
        for hk in (0, c["Hkv"] - 1):
            hs = slice(hk * G, (hk + 1) * G)
            qn = host(r["q"][ts:te, hs])
            kn = host(r["k"][ts:te, hk:hk + 1])
            vn = host(r["v"][ts:te, hk:hk + 1])
            don = host(r["do"][ts:te, hs])
            O, LSE = OA.forward_branches(qn, kn, vn, par, pos)
            assert max_abs(host(r["o"][ts:te, hs]), O) <= O_TOL
            assert max_abs(host(r["lse"][hs, ts:te]), LSE) <= LSE_TOL
            dq, dk, dv = OA.backward_branches(qn, kn, vn, don, par, pos)
            assert rel_l2(host(r["dq"][ts:te, hs]), dq) <= GRAD_TOL
            assert rel_l2(host(r["dk"][ts:te, hk:hk + 1]), dk) <= GRAD_TOL
            assert rel_l2(host(r["dv"][ts:te, hk:hk + 1]), dv) <= GRAD_TOL
            print(f"tree {t} kv {hk} ok", flush=True)


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


def _small_subtree_keys(po, n, rng, max_sub=48):
    size = po["se"] - np.arange(po["T"])
    cand = np.nonzero(size <= max_sub)[0]
    keys = list(rng.choice(cand, size=min(n, len(cand)), replace=False))
    # include keys at a node boundary and the last token
    keys += [int(po["T"] - 1)]
    return sorted(set(int(x) for x in keys))


@pytest.mark.parametrize("name", ["agentic", "agentic_l"])
def test_random_agentic_tree_sampled(name):
    """Random agentic trees (32768 tokens, depth <= 6; 131072 tokens, depth
    <= 10), 64q/8kv, d=128, at full size. Sampled query rows (O, LSE, dQ over
    all heads), sampled keys (dK, dV), and two identities over all keys."""
    seqs, groups = workloads.sequences(name)
    c = workloads.WORKLOADS[name]
    r = run_gpu(seqs, groups, c["Hq"], c["Hkv"], c["d"], c["dtype"], c["seed"])
    po = OP.pack(seqs, groups)
    rng = np.random.default_rng(42)
    n_rows = 24 if name == "agentic" else 12
    rows = _sample_rows(po, n_rows, rng)
    print(f"\n{name}: {len(rows)} rows", flush=True)
    kn = host(r["k"])
    vn = host(r["v"])
    qv = _Rows(r["q"], rows)
    dov = _Rows(r["do"], rows)
    O, LSE = OA.forward_rows(qv, kn, vn, po["par"], rows)
    rt = torch.as_tensor(rows, device="cuda")
    assert max_abs(host(r["o"][rt]), O) <= O_TOL
    assert max_abs(host(r["lse"][:, rt]), LSE) <= LSE_TOL
    dq = OA.backward_rows_dq(qv, kn, vn, dov, po["par"], rows)
    assert rel_l2(host(r["dq"][rt]), dq) <= GRAD_TOL
    print(f"{name}: rows ok", flush=True)

    keys = _small_subtree_keys(po, 4 if name == "agentic" else 3, rng)
    need = sorted(set(int(i) for j in keys for i in OA.subtree_rows(po["par"], j)))
    qk = _Rows(r["q"], need)
    dok = _Rows(r["do"], need)
    kvh = [0, c["Hkv"] - 1]
    dk, dv = OA.backward_keys(qk, kn, vn, dok, po["par"], keys, kv_heads=kvh)
    kt = torch.as_tensor(keys, device="cuda")
    assert rel_l2(host(r["dk"][kt][:, kvh]), dk) <= GRAD_TOL
    assert rel_l2(host(r["dv"][kt][:, kvh]), dv) <= GRAD_TOL
    print(f"{name}: keys ok", flush=True)

    # identities over every key: softmax rows sum to one, so sum_j dV_j equals
    # the summed upstream gradient of each group; and sum_j dS_ij = 0, so the
    # re-rotated dK sums to zero.
    G = c["Hq"] // c["Hkv"]
    sum_dv = r["dv"].double().sum(0)
    sum_do = r["do"].double().view(-1, c["Hkv"], G, c["d"]).sum((0, 2))
    assert rel_l2(sum_dv.cpu().numpy(), sum_do.cpu().numpy()) <= GRAD_TOL
    dkr = OA.rope(host(r["dk"]).astype(np.float64), po["pos"], 10000.0)
    ratio = np.linalg.norm(dkr.sum(0)) / np.linalg.norm(dkr, axis=-1).sum()
    assert ratio < 1e-3, ratio


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
    qn, kn, vn = host(r["q"]), host(r["k"]), host(r["v"])
    O, LSE = OA.forward_dense(qn, kn, vn, vis, np.zeros(po["T"]))
    assert max_abs(host(r["o"]), O) <= O_TOL and max_abs(host(r["lse"]), LSE) <= LSE_TOL
    q, k, v = r["q"], r["k"], r["v"]
    o, lse, _ = ta.tree_attn_fwd(q, k, v, r["pos"], r["se"], softmax_scale=0.05)
    O2, L2 = OA.forward_dense(qn, kn, vn, vis, po["pos"], scale=0.05)
    assert max_abs(host(o), O2) <= O_TOL and max_abs(host(lse), L2) <= LSE_TOL
