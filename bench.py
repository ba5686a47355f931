"""Benchmark of the tree-attention hot path on one MI355X.

A step is one pass of the device hot path over one packed batch: RoPE at
depth positions + tile plan, tree-masked forward, and backward (dQ, dK, dV),
through the C ABI. Inputs (q, k, v, dO and the packer's pos / subtree_end)
are resident in HBM before the timed region. Reported value: visible-pair
TFLOP/s, 14 * d * P * Hq per step (forward 4, backward 10), P = sum(pos + 1).

Also reported on the same line: the host packer's time (not in the step), a
partition-boundary leg (tree 0 unsplit vs split after its prompt, the child
partitions through the gateway entry points),
the tile classification, tree_logprob on 16384 bf16 rows x 151936 vocab with
every row referenced 3 times (its own timed leg, HBM GB/s) and in unique form
with the packer's weights g/K on the random agentic tree (32768 rows x 32000
vocab), per-kernel HIP
event timings, the roofline of the dominant kernel and the CPU oracle timed
on a bounded sample.

Legs on the same line: the other attention workloads (short-prompt groups,
the random agentic trees of 32768 and 131072 tokens), each with forward,
backward and the whole step timed apart as medians of 20 HIP-event timings.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload multistep]
    python bench.py --cpu-report    (host-only oracle measurements, no GPU)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-attn fwd+bwd visible-pair TFLOP/s and % bf16 MFMA peak; packed tokens/s"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 dense bf16 FLOP/clk x 2.4 GHz
PEAK_HBM_GBPS = 8000.0

DESCR = {
    "short": "short-prompt groups: 8 trees x (256-token prompt + 4 branches x 128), T=6144, 32q/8kv, d=128, bf16",
    "multistep": "long prompt, multi-step: 4 trees x (1024-token prompt + 8 trajectories x 2 steps "
                 "[256 resp; +256 tool +256 resp]), T=28672, 32q/8kv, d=128, bf16",
    "agentic": "random agentic tree, depth<=6, branching U{1,2,3}, segments U{64..1024}, T=32768, 64q/8kv, d=128, bf16",
    "agentic_l": "random agentic tree, depth<=10, T=131072, 64q/8kv, d=128, bf16",
}

# algorithmic FLOPs per visible pair and query head, per kernel group, in units of d
KERNEL_FLOPS = {"attn_fwd": 4, "attn_bwd_dkdv": 8, "attn_bwd_dq": 2}


def host_info():
    """The host the CPU baseline runs on: cores, CPU model, BLAS, RAM."""
    info = {"nproc": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as fh:
            for line in fh:
                if line.startswith("MemTotal"):
                    info["ram_gb"] = round(int(line.split()[1]) / 2 ** 20, 1)
                    break
    except OSError:
        pass
    try:
        info["nproc"] = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    try:
        from threadpoolctl import threadpool_info

        blas = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = int(blas[0].get("num_threads", 1))
    except Exception:  # pragma: no cover
        pass
    return info


def _oracle_attn(seqs, groups, cfg, n_trees, n_groups, seed=77):
    """The float64 per-branch oracle, fwd then bwd, on trees 0 .. n_trees-1
    x kv groups 0 .. n_groups-1 of the workload. Returns (fwd s, bwd s,
    visible-pair FLOPs (14 d P Hq), tokens)."""
    import workloads
    from oracle import attention as OA
    from oracle import pack as OP

    po = OP.pack(seqs, groups)
    n_trees = min(n_trees, len(po["tree_start"]) - 1)
    G = cfg["Hq"] // cfg["Hkv"]
    f = lambda t: t.float().numpy()
    tf = tb = flops = 0.0
    toks = 0
    for tr in range(n_trees):
        ts, te = int(po["tree_start"][tr]), int(po["tree_start"][tr + 1])
        par = po["par"][ts:te].copy()
        par[par >= 0] -= ts
        P = int((po["pos"][ts:te] + 1).sum())
        toks += te - ts
        for g in range(n_groups):
            q, k, v, do = workloads.dense_inputs(te - ts, G, 1, cfg["d"], "bf16", seed + 100 * tr + g)
            t0 = time.perf_counter()
            OA.forward_branches(f(q), f(k), f(v), par, po["pos"][ts:te], check_agree=False)
            t1 = time.perf_counter()
            OA.backward_branches(f(q), f(k), f(v), f(do), par, po["pos"][ts:te])
            t2 = time.perf_counter()
            tf += t1 - t0
            tb += t2 - t1
            flops += 14.0 * cfg["d"] * P * G
    return tf, tb, flops, toks, n_trees


def cpu_baseline(seqs, groups, cfg, n_trees=3, n_groups=2):
    """The float64 oracle as it stands, on the host cores: per-branch fwd +
    bwd on the first n_trees trees x the first n_groups kv groups of the
    workload (a bounded sample), plus the oracle packer on the whole batch
    and the oracle log-prob on 256 rows of the 151936-token vocabulary."""
    import workloads
    from oracle import logprob as OL
    from oracle import pack as OP

    info = host_info()
    t0 = time.perf_counter()
    OP.pack(seqs, groups)
    pack_s = time.perf_counter() - t0
    tf, tb, flops, toks, nt = _oracle_attn(seqs, groups, cfg, n_trees, n_groups)
    R, V = 256, 151936
    src, tgt, w = workloads.repeated_rows_entries(R, V, 3, 5)
    z = workloads.logits_input(R, V, "bf16", 5).double().numpy()
    t0 = time.perf_counter()
    OL.logprob(z, src, tgt, w.astype(np.float32) if hasattr(w, "astype") else w)
    lp_s = time.perf_counter() - t0
    G = cfg["Hq"] // cfg["Hkv"]
    cores = info.get("blas_threads", info.get("nproc", 1))
    return {"value": flops / (tf + tb) / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"trees 0..{nt - 1} ({toks} tokens) x kv groups 0..{n_groups - 1} ({G} q heads each), "
                      f"fwd+bwd per branch, float64 NumPy, {tf + tb:.1f} s for {flops / 1e9:.1f} visible-pair GFLOP",
            "host": info, "stage_s": {"pack_whole_batch": round(pack_s, 3), "attn_fwd_sample": round(tf, 3),
                                      "attn_bwd_sample": round(tb, 3),
                                      "logprob_256_rows_fused": round(lp_s, 3)},
            "logprob_gbps": round(2.0 * R * V * 2 / lp_s / 1e9, 3)}


def cpu_report():
    """Longer host-only oracle measurements (no GPU work): every host core
    and one thread on the short-prompt batch, per stage; the multistep
    sample of the default line; the large random tree's attention on kv
    groups 0 and 7 with the whole-tree ancestor-chain oracle, scaled to all
    8 groups (labelled extrapolated)."""
    import workloads
    from oracle import attention as OA
    from oracle import pack as OP

    out = {"host": host_info()}
    for name, nt, ng in (("short", 8, 8), ("multistep", 3, 2)):
        seqs, groups = workloads.sequences(name)
        cfg = workloads.WORKLOADS[name]
        tf, tb, flops, toks, n = _oracle_attn(seqs, groups, cfg, nt, ng)
        out[name] = {"trees": n, "kv_groups": ng, "tokens": toks, "fwd_s": round(tf, 3), "bwd_s": round(tb, 3),
                     "tflops": round(flops / (tf + tb) / 1e12, 5)}
        print(f"[cpu] {name}: fwd {tf:.2f} s, bwd {tb:.2f} s", flush=True)
    try:
        from threadpoolctl import threadpool_limits

        seqs, groups = workloads.sequences("short")
        cfg = workloads.WORKLOADS["short"]
        with threadpool_limits(limits=1):
            tf, tb, flops, toks, n = _oracle_attn(seqs, groups, cfg, 8, 8)
        out["short_one_thread"] = {"fwd_s": round(tf, 3), "bwd_s": round(tb, 3),
                                   "tflops": round(flops / (tf + tb) / 1e12, 5)}
        print(f"[cpu] short, one thread: fwd {tf:.2f} s, bwd {tb:.2f} s", flush=True)
    except ImportError:  # pragma: no cover
        pass
    seqs, groups = workloads.sequences("agentic_l")
    cfg = workloads.WORKLOADS["agentic_l"]
    po = OP.pack(seqs, groups)
    T, G = po["T"], cfg["Hq"] // cfg["Hkv"]
    P = int((po["pos"].astype(np.int64) + 1).sum())
    q, k, v, do = workloads.dense_inputs(T, cfg["Hq"], cfg["Hkv"], cfg["d"], "bf16", cfg["seed"])
    tf = tb = 0.0
    for hk in (0, cfg["Hkv"] - 1):
        f = lambda t: t.float().numpy()
        qq, kk, vv, dd = f(q[:, hk * G:(hk + 1) * G]), f(k[:, hk:hk + 1]), f(v[:, hk:hk + 1]), f(do[:, hk * G:(hk + 1) * G])
        t0 = time.perf_counter()
        OA.forward_chains(qq, kk, vv, po["par"])
        t1 = time.perf_counter()
        OA.backward_chains(qq, kk, vv, dd, po["par"])
        t2 = time.perf_counter()
        tf += t1 - t0
        tb += t2 - t1
        print(f"[cpu] agentic_l kv group {hk}: fwd {t1 - t0:.1f} s, bwd {t2 - t1:.1f} s", flush=True)
    scale = cfg["Hkv"] / 2.0
    out["agentic_l"] = {"kv_groups_run": [0, cfg["Hkv"] - 1], "oracle": "whole-tree ancestor chains",
                        "fwd_s_extrapolated": round(tf * scale, 1), "bwd_s_extrapolated": round(tb * scale, 1),
                        "tflops_extrapolated": round(14.0 * cfg["d"] * P * cfg["Hq"] / ((tf + tb) * scale) / 1e12, 5),
                        "label": "extrapolated: 2 of 8 kv groups run, times scaled by 4"}
    print(json.dumps(out), flush=True)


def tile_report(p):
    """Tile classification of a packed batch: at 128x64 (the kernels'
    forward and dQ tiles) and 128x128, over the whole batch and within each
    tree (cross-tree tiles, all empty, left out)."""
    import tree_packed_attention_amd as ta

    T, se = p["T"], p["subtree_end"]
    out = {}
    for BQ, BK in ((128, 64), (128, 128)):
        full, partial, empty, causal = ta.tree_tile_stats(se, T, BQ, BK)
        wf = wp = we = wc = 0
        ts = p["tree_start"]
        for t in range(len(ts) - 1):
            a, b = int(ts[t]), int(ts[t + 1])
            f_, p_, e_, c_ = ta.tree_tile_stats((se[a:b] - a).astype(np.int32), b - a, BQ, BK)
            wf, wp, we, wc = wf + f_, wp + p_, we + e_, wc + c_
        out[f"{BQ}x{BK}"] = {"full": full, "partial": partial, "empty": empty, "causal": causal,
                             "skip": round(empty / causal, 4),
                             "within_tree": {"full": wf, "partial": wp, "empty": we, "causal": wc,
                                             "skip": round(we / max(wc, 1), 4)}}
    return out


def attn_leg(name, dev, reps=20, warmup=3):
    """One workload: forward, backward and the whole step timed separately
    with HIP events on the launch stream (median of `reps` after `warmup`),
    visible-pair TFLOP/s with the backward counted both ways (10 d P Hq,
    FlashAttention's convention with the recomputed scores, and the strict
    8 d P Hq), tile classification, per-kernel times."""
    import torch

    import tree_packed_attention_amd as ta
    import workloads

    cfg = workloads.WORKLOADS[name]
    seqs, groups = workloads.sequences(name)
    p = ta.tree_pack(seqs, groups)
    T, Hq, Hkv, d = p["T"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    P = int((p["pos"].astype(np.int64) + 1).sum())
    q, k, v, do = workloads.dense_inputs(T, Hq, Hkv, d, "bf16", cfg["seed"], device=dev)
    pos = torch.from_numpy(p["pos"]).to(dev)
    se = torch.from_numpy(p["subtree_end"]).to(dev)
    ws = ta.attn_workspace(T, Hq, Hkv, d, True, dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    fwd_ms, bwd_ms, step_ms = [], [], []
    for i in range(warmup + reps):
        e0, e1, e2 = ev(), ev(), ev()
        e0.record()
        o, lse, _ = ta.tree_attn_fwd(q, k, v, pos, se, workspace=ws)
        e1.record()
        ta.tree_attn_bwd(q, k, v, o, lse, do, pos, se, workspace=ws, reuse_prep=True)
        e2.record()
        e2.synchronize()
        if i >= warmup:
            fwd_ms.append(e0.elapsed_time(e1))
            bwd_ms.append(e1.elapsed_time(e2))
            step_ms.append(e0.elapsed_time(e2))
    ta.tree_attn_profile_enable(True)
    for _ in range(3):
        o, lse, _ = ta.tree_attn_fwd(q, k, v, pos, se, workspace=ws)
        ta.tree_attn_bwd(q, k, v, o, lse, do, pos, se, workspace=ws, reuse_prep=True)
    torch.cuda.synchronize()
    kern = {n: round(tot / max(c, 1), 4) for n, (tot, c) in ta.tree_attn_profile_read().items()}
    ta.tree_attn_profile_enable(False)
    status = ta.tree_attn_workspace_status(ws)
    del ws, q, k, v, do, o, lse
    torch.cuda.empty_cache()
    med = lambda x: float(np.median(x))
    fm, bm, sm = med(fwd_ms), med(bwd_ms), med(step_ms)
    u = d * P * Hq
    return {"workload": DESCR[name], "T": T, "visible_pairs": P, "Hq": Hq, "Hkv": Hkv, "d": d,
            "trees": p["n_trees"], "reps": reps, "warmup": warmup,
            "fwd_ms_median": round(fm, 4), "bwd_ms_median": round(bm, 4), "step_ms_median": round(sm, 4),
            "fwd_tflops": round(4 * u / fm / 1e9, 2), "bwd_tflops": round(10 * u / bm / 1e9, 2),
            "bwd_tflops_strict_8dPH": round(8 * u / bm / 1e9, 2), "step_tflops": round(14 * u / sm / 1e9, 2),
            "pct_bf16_peak": round(100.0 * 14 * u / sm / 1e9 / PEAK_BF16_TFLOPS, 2),
            "packed_tokens_per_s": round(T / (sm * 1e-3), 1), "tiles": tile_report(p), "kernel_ms": kern,
            "status_word": status}


def gateway_leg(seqs, groups, cfg, dev, steps):
    """Partition boundary ("Tree Training" §3.3, App. B): tree 0 of the batch
    unsplit vs split after its shared prefix (parent partition = the prefix
    chain; the subtrees under it = child partitions of that cut, in one
    gateway call over the cached, rotated prefix K/V). Both are timed
    fwd+bwd."""
    import torch

    import tree_packed_attention_amd as ta
    import workloads

    g0 = [s_ for s_, g in zip(seqs, groups) if g == groups[0]]
    L = 0
    while all(len(s_) > L and s_[L] == g0[0][L] for s_ in g0):
        L += 1
    full = ta.tree_pack(g0, None)
    T, Hq, Hkv, d = full["T"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    q, k, v, do = workloads.dense_inputs(T, Hq, Hkv, d, "bf16", cfg["seed"] + 7, device=dev)
    pos = torch.from_numpy(full["pos"]).to(dev)
    se = torch.from_numpy(full["subtree_end"]).to(dev)
    assert int(full["pos"][L - 1]) == L - 1 and int(full["subtree_end"][L - 1]) == T  # the prompt is a chain

    # the parent partition's own tensors (its prompt chain) and the child
    # partitions' tensors, sliced before the timed region
    pq, pk, pv, pdo = (t[:L].contiguous() for t in (q, k, v, do))
    vis = torch.ones(L, dtype=torch.uint8, device=dev)
    ppos, pse = pos[:L].contiguous(), torch.full((L,), L, dtype=torch.int32, device=dev)
    rows = torch.arange(L, dtype=torch.int32, device=dev)  # every prompt token is a cached row
    k_past = torch.empty(L, Hkv, d, dtype=q.dtype, device=dev)
    v_past = torch.empty_like(k_past)
    cq, ck, cv, cdo = (t[L:].contiguous() for t in (q, k, v, do))
    cpos, cse = (pos[L:] - L).contiguous(), (se[L:] - L).contiguous()
    ws_full = ta.attn_workspace(T, Hq, Hkv, d, True, dev)
    ws_par = ta.attn_workspace(L, Hq, Hkv, d, True, dev)
    ws_ch = ta.gw_workspace(T - L, L, Hq, Hkv, d, True, dev)

    def unsplit():
        o, lse, _ = ta.tree_attn_fwd(q, k, v, pos, se, workspace=ws_full)
        return o, ta.tree_attn_bwd(q, k, v, o, lse, do, pos, se, workspace=ws_full, reuse_prep=True)

    def split():
        # parent forward, hand-over of its rotated K and V rows, child
        # forward and backward through the gateway, parent backward, relay of
        # the cached rows' float32 gradients into the parent's dK, dV
        o1, l1, _ = ta.tree_attn_fwd(pq, pk, pv, ppos, pse, workspace=ws_par)
        ta.tree_attn_gw_export(pk, pv, ppos, rows, 0, 10000.0, k_past=k_past, v_past=v_past)
        o2, l2, _ = ta.tree_attn_gw_fwd(cq, ck, cv, cpos, cse, L, k_past, v_past, vis, workspace=ws_ch)
        g = ta.tree_attn_gw_bwd(cq, ck, cv, o2, l2, cdo, cpos, cse, L, k_past, v_past, vis, workspace=ws_ch,
                                reuse_prep=True)
        gp = ta.tree_attn_bwd(pq, pk, pv, o1, l1, pdo, ppos, pse, workspace=ws_par, reuse_prep=True)
        ta.tree_attn_gw_relay(g[3], g[4], rows, ppos, gp[1], gp[2], 0, 10000.0)
        return o2, (gp, g)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            out = fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3, out

    ms_full, (o_full, g_full) = timed(unsplit)
    ms_split, (o_child, (gp, gc)) = timed(split)
    P_child = int((cpos.long() + 1).sum().item()) + L * (T - L)
    rel = lambda a, b: float((a.float() - b.float()).norm() / b.float().norm())
    return {"workload": f"tree 0 (T={T}) split after its {L}-token shared prefix: parent partition = the prefix, "
                        f"child partitions = the subtrees under it ({T - L} tokens) in one gateway call; the split "
                        f"includes the export of the cached rows and the relay of their gradients",
            "unsplit_ms": round(ms_full, 4), "split_ms": round(ms_split, 4),
            "split_overhead": round(ms_split / ms_full - 1.0, 4),
            "child_visible_pairs": P_child,
            "max_abs_child_o_vs_unsplit": round(float((o_child.float() - o_full[L:].float()).abs().max()), 5),
            "rel_l2_parent_dk_vs_unsplit": round(rel(gp[1], g_full[1][:L]), 5),
            "rel_l2_parent_dv_vs_unsplit": round(rel(gp[2], g_full[2][:L]), 5)}


def ssm_leg(seqs, groups, dev, steps):
    """Tree SSM kernels on the same packed batch, at the shape of a hybrid
    model's linear-attention layer: 16 q/k heads and 32 v heads of 128, conv
    width 2*16*128 + 32*128 = 8192 channels, K = 4, bf16. Times the tree conv
    forward and backward and the tree-routed gated delta rule forward and
    backward, each against its algorithmic HBM bytes (inputs read once,
    outputs written once)."""
    import numpy as np
    import torch

    import tree_packed_attention_amd as ta
    import workloads

    p = ta.tree_pack(seqs, groups)
    T = p["T"]
    H, Hv, d, C, K = 16, 32, 128, 8192, 4
    t0 = time.perf_counter()
    plan = ta.tree_gdn_plan(p["node_start"], p["node_end"], p["node_parent"], 64)
    plan_ms = (time.perf_counter() - t0) * 1e3
    plan_dev = torch.from_numpy(plan).to(dev)
    q, k, v, g, beta = workloads.gdn_inputs(T, H, Hv, d, d, "bf16", 3, device=dev)
    gws = ta.gdn_workspace(q, v, plan, backward=True)
    gdo = workloads.gdn_dout(T, Hv, d, "bf16", 3, device=dev)
    x, dy, w, b = workloads.conv_inputs(T, C, K, "bf16", 3, device=dev)
    par = torch.from_numpy(p["parent"]).to(dev)
    pos = torch.from_numpy(p["pos"]).to(dev)
    se = torch.from_numpy(p["subtree_end"]).to(dev)
    cws = torch.empty(ta.library().tree_conv_workspace_bytes(T, C, K), dtype=torch.uint8, device=dev)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ta.tree_attn_profile_enable(True)
        t1 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t1) / steps
        ks = ta.tree_attn_profile_read()
        ta.tree_attn_profile_enable(False)
        return dt, {n: round(tot / max(c, 1), 4) for n, (tot, c) in ks.items()}

    gdn_s, gdn_k = timed(lambda: ta.tree_gdn_fwd(q, k, v, g, beta, plan, plan_dev=plan_dev, workspace=gws))
    # the backward reads the forward's chunk states from the workspace (left by the last forward above)
    gdnb_s, gdnb_k = timed(lambda: ta.tree_gdn_bwd(q, k, v, g, beta, gdo, plan, gws, plan_dev=plan_dev))
    cf_s, _ = timed(lambda: ta.tree_conv_fwd(x, w, b, par, 1))
    cb_s, _ = timed(lambda: ta.tree_conv_bwd(x, dy, w, b, par, pos, se, 1, workspace=cws))
    gdn_bytes = T * (2 * H * d * 2 + 2 * Hv * d * 2 + 8 * Hv)
    gdnb_bytes = T * (4 * H * d * 2 + 3 * Hv * d * 2 + 16 * Hv)
    cf_bytes, cb_bytes = 2.0 * T * C * 2, 3.0 * T * C * 2
    nc = int(plan[0])
    gdn_flop = nc * Hv * (6.0 * 64 * d * d + 64 * 64 * 4.0 * d)
    return {"workload": f"multistep batch T={T}, gated delta rule 16 q/k x 32 v heads, dk=dv=128; conv C=8192 K=4; bf16",
            "chunks": nc, "chains": int(plan[1]), "levels": int(plan[2]), "plan_ms_host": round(plan_ms, 3),
            "gdn_fwd_ms": round(gdn_s * 1e3, 4), "gdn_fwd_gbps": round(gdn_bytes / gdn_s / 1e9, 1),
            "gdn_fwd_tflops_chunked": round(gdn_flop / gdn_s / 1e12, 2), "gdn_kernel_ms": gdn_k,
            "gdn_bwd_ms": round(gdnb_s * 1e3, 4), "gdn_bwd_gbps": round(gdnb_bytes / gdnb_s / 1e9, 1),
            "gdn_bwd_kernel_ms": gdnb_k,
            "conv_fwd_ms": round(cf_s * 1e3, 4), "conv_fwd_gbps": round(cf_bytes / cf_s / 1e9, 1),
            "conv_bwd_ms": round(cb_s * 1e3, 4), "conv_bwd_gbps": round(cb_bytes / cb_s / 1e9, 1),
            "hbm_peak_gbps": PEAK_HBM_GBPS}


def partition_leg():
    """The host partition planner on the large random agentic tree (131072
    tokens, depth <= 10) at a 32768-token capacity: partitions, levels, host
    time, and the tokens one pass processes when every sequence is
    flattened, when partitions re-read their ancestors (no differentiable
    boundaries), and with boundaries (every token once; "Tree Training"
    Fig. 5 compares the same three)."""
    import numpy as np

    import tree_packed_attention_amd as ta
    import workloads

    seqs, groups = workloads.sequences("agentic_l")
    p = ta.tree_pack(seqs, groups)
    cap = 32768
    t0 = time.perf_counter()
    plan = ta.tree_partition(p["node_start"], p["node_end"], p["node_parent"], cap)
    ms = (time.perf_counter() - t0) * 1e3
    lens = (p["node_end"] - p["node_start"]).astype(np.int64)
    npar = p["node_parent"]
    part = plan["node_part"]
    recompute = int(lens.sum())
    for b in range(len(plan["part_tokens"])):
        anc = set()
        for v in np.nonzero((part == b) & ((npar < 0) | (part[np.maximum(npar, 0)] != b)))[0]:
            u = npar[v]
            while u >= 0:
                anc.add(int(u))
                u = npar[u]
        recompute += int(sum(lens[u] for u in anc))
    levels = []
    for b in range(len(plan["part_parent"])):
        lv, x = 0, b
        while plan["part_parent"][x] >= 0:
            x, lv = plan["part_parent"][x], lv + 1
        levels.append(lv)
    return {"workload": "random agentic tree, depth<=10, T=131072", "capacity": cap,
            "partitions": int(len(plan["part_tokens"])), "levels": int(max(levels) + 1),
            "max_partition_tokens": int(plan["part_tokens"].max()), "plan_ms_host": round(ms, 3),
            "tokens_flattened": int(sum(len(s_) for s_ in seqs)), "tokens_standard_partitioning": recompute,
            "tokens_with_boundaries": int(p["T"])}


# The files the attention kernels' device code is compiled from: the counter
# summaries are valid while these are unchanged.
ATTN_DEVICE_SOURCES = ("attention.hip", "ta_device.h", "ta_lds.h")


def measured_traffic(kernel, workload):
    """Calibrated HBM bytes per dispatch of `kernel` on `workload` from the
    committed rocprofv3 counter summaries, if they were taken on the current
    sources of the attention kernels (else None)."""
    import glob
    import hashlib

    h = hashlib.sha256()
    for name in ATTN_DEVICE_SOURCES:
        with open(os.path.join(ROOT, "tree_packed_attention_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    sha = h.hexdigest()[:16]
    for fn in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(fn) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    if (rec.get("source_sha") == sha and rec.get("workload", "multistep") == workload
                            and kernel in rec.get("bytes_per_dispatch", {})):
                        return int(rec["bytes_per_dispatch"][kernel])
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="multistep", choices=sorted(DESCR))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-logprob", action="store_true")
    ap.add_argument("--no-gateway", action="store_true")
    ap.add_argument("--no-ssm", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="skip the other attention workloads' legs")
    ap.add_argument("--cpu-report", action="store_true",
                    help="only the longer host-side oracle measurements (no GPU work), as one JSON line")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="first run a plain device copy of this many bytes (calibrates HBM counters)")
    args = ap.parse_args()
    if args.cpu_report:
        import numpy as np  # noqa: F401

        cpu_report()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU sharding is a design "
              "note, not a built path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tree_packed_attention_amd as ta
    import workloads

    dev = torch.device("cuda:0")
    if args.copy_bytes > 0:
        a = torch.empty(args.copy_bytes, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {args.copy_bytes} bytes x 3", flush=True)
        del a, b
    cfg = workloads.WORKLOADS[args.workload]
    seqs, groups = workloads.sequences(args.workload)
    t0 = time.perf_counter()
    p = ta.tree_pack(seqs, groups)
    pack_ms = (time.perf_counter() - t0) * 1e3
    T, Hq, Hkv, d = p["T"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    P = int((p["pos"].astype(np.int64) + 1).sum())
    flops = 14.0 * d * P * Hq
    full, partial, empty, causal = ta.tree_tile_stats(p["subtree_end"], T, 128, 64)
    print(f"[bench] {args.workload}: T={T} P={P} tiles full/partial/empty={full}/{partial}/{empty}", flush=True)

    q, k, v, do = workloads.dense_inputs(T, Hq, Hkv, d, "bf16", cfg["seed"], device=dev)
    pos = torch.from_numpy(p["pos"]).to(dev)
    se = torch.from_numpy(p["subtree_end"]).to(dev)
    ws = ta.attn_workspace(T, Hq, Hkv, d, True, dev)

    def step():
        o, lse, _ = ta.tree_attn_fwd(q, k, v, pos, se, workspace=ws)
        return ta.tree_attn_bwd(q, k, v, o, lse, do, pos, se, workspace=ws, reuse_prep=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ta.tree_attn_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kern = ta.tree_attn_profile_read()
    ta.tree_attn_profile_enable(False)
    ms_step = dt / args.steps * 1e3
    value = flops * args.steps / dt / 1e12
    print(f"[bench] attention step {ms_step:.3f} ms, {value:.1f} TFLOP/s", flush=True)

    kernel_ms = {n: tot / max(cnt, 1) for n, (tot, cnt) in kern.items()}
    del ws
    torch.cuda.empty_cache()
    # the same workload again, forward and backward timed apart (medians)
    head = attn_leg(args.workload, dev)
    print(f"[bench] {args.workload}: fwd {head['fwd_ms_median']:.3f} ms, bwd {head['bwd_ms_median']:.3f} ms "
          f"(medians)", flush=True)
    legs = {}
    if not args.no_legs:
        for name in ("short", "multistep", "agentic", "agentic_l"):
            if name == args.workload:
                continue
            legs[name] = attn_leg(name, dev)
            print(f"[bench] leg {name}: step {legs[name]['step_ms_median']:.3f} ms, "
                  f"{legs[name]['step_tflops']:.1f} TFLOP/s ({legs[name]['pct_bf16_peak']:.1f} %)", flush=True)
    dom = max((n for n in kernel_ms if n in KERNEL_FLOPS), key=lambda n: kernel_ms[n])
    achieved = KERNEL_FLOPS[dom] * d * P * Hq / (kernel_ms[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom + "_kernel", args.workload), "traffic_unit": "bytes per launch (HBM, calibrated)",
                "flops_per_launch": KERNEL_FLOPS[dom] * d * P * Hq}

    lp = None
    if not args.no_logprob:
        R, V = 16384, 151936
        src, tgt, w = workloads.repeated_rows_entries(R, V, 3, 5)
        z = workloads.logits_input(R, V, "bf16", 5, device=dev)
        s_t = torch.as_tensor(src, device=dev)
        t_t = torch.as_tensor(tgt, device=dev)
        w_t = torch.as_tensor(w, device=dev)
        lws = torch.empty(ta.library().tree_logprob_workspace_bytes(R, len(src)), dtype=torch.uint8, device=dev)
        for _ in range(2):
            ta.tree_logprob(z, s_t, t_t, w_t, workspace=lws)
        torch.cuda.synchronize()
        ta.tree_attn_profile_enable(True)
        n_lp = max(3, args.steps // 2)
        t0 = time.perf_counter()
        for _ in range(n_lp):
            ta.tree_logprob(z, s_t, t_t, w_t, workspace=lws)
        torch.cuda.synchronize()
        lp_dt = (time.perf_counter() - t0) / n_lp
        lk = ta.tree_attn_profile_read()
        ta.tree_attn_profile_enable(False)
        M = len(src)
        alg = 2.0 * R * V * 2 + 12.0 * M + 4.0 * R
        rows_ms = lk["lp_rows"][0] / lk["lp_rows"][1]
        lp = {"workload": "16384 bf16 rows x 151936 vocab, M=49152 (each row 3x), fused fwd+bwd",
              "ms": round(lp_dt * 1e3, 4), "gbps": round(alg / lp_dt / 1e9, 1),
              "row_kernel_ms": round(rows_ms, 4), "row_kernel_gbps": round(2.0 * R * V * 2 / (rows_ms * 1e-3) / 1e9, 1),
              "hbm_peak_gbps": PEAK_HBM_GBPS,
              "kernel_ms": {n: round(tot / max(c, 1), 4) for n, (tot, c) in lk.items()}}
        # the clipped policy loss on the same rows: per-entry advantage, old
        # log-probability (ratios in every clip region) and mask
        adv, ratio, mask = workloads.policy_inputs(M, 5)
        a_t = torch.as_tensor(adv, device=dev)
        o_t = ta.tree_logprob(z, s_t, t_t, w_t, with_grad=False, workspace=lws)[0] - torch.as_tensor(
            np.log(ratio).astype(np.float32), device=dev)
        m_t = torch.as_tensor(mask, device=dev)
        for _ in range(2):
            ta.tree_logprob_ppo(z, s_t, t_t, w_t, a_t, o_t, m_t, workspace=lws)
        torch.cuda.synchronize()
        ta.tree_attn_profile_enable(True)
        t0 = time.perf_counter()
        for _ in range(n_lp):
            ta.tree_logprob_ppo(z, s_t, t_t, w_t, a_t, o_t, m_t, workspace=lws)
        torch.cuda.synchronize()
        pp_dt = (time.perf_counter() - t0) / n_lp
        pk = ta.tree_attn_profile_read()
        ta.tree_attn_profile_enable(False)
        alg_pp = 2.0 * R * V * 2 + 25.0 * M + 4.0 * R
        lp["policy_loss"] = {"ms": round(pp_dt * 1e3, 4), "gbps": round(alg_pp / pp_dt / 1e9, 1),
                             "eps": [0.2, 0.2], "masked_frac": round(1.0 - float(mask.mean()), 4),
                             "kernel_ms": {n: round(tot / max(c, 1), 4) for n, (tot, c) in pk.items()}}
        print(f"[bench] tree_logprob {lp['ms']:.3f} ms, {lp['gbps']:.0f} GB/s; clipped policy loss "
              f"{lp['policy_loss']['ms']:.3f} ms", flush=True)
        del z
        # the per-token weights g/K of the random agentic tree in unique form:
        # one entry per token with a parent (M = T - 1 per tree), row = the
        # parent, target = the token, weight = the packer's g/K
        aseqs, agroups = workloads.sequences("agentic")
        ap = ta.tree_pack(aseqs, agroups)
        at = np.nonzero(ap["parent"] >= 0)[0]
        Ra, Va = ap["T"], 32000
        za = workloads.logits_input(Ra, Va, "bf16", 4, device=dev)
        sa_t = torch.as_tensor(ap["parent"][at], device=dev)
        ta_t = torch.as_tensor(ap["ids"][at], device=dev)
        wa_t = torch.as_tensor(ap["weight"][at], device=dev)
        aws = torch.empty(ta.library().tree_logprob_workspace_bytes(Ra, len(at)), dtype=torch.uint8, device=dev)
        for _ in range(2):
            ta.tree_logprob(za, sa_t, ta_t, wa_t, workspace=aws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n_lp):
            ta.tree_logprob(za, sa_t, ta_t, wa_t, workspace=aws)
        torch.cuda.synchronize()
        ua_dt = (time.perf_counter() - t0) / n_lp
        alg_u = 2.0 * Ra * Va * 2 + 12.0 * len(at) + 4.0 * Ra
        lp["unique_agentic"] = {"workload": f"random agentic tree (T={Ra}), unique form M={len(at)}, weights g/K, "
                                            f"{Ra} bf16 rows x {Va} vocab, fused fwd+bwd",
                                "ms": round(ua_dt * 1e3, 4), "gbps": round(alg_u / ua_dt / 1e9, 1)}
        print(f"[bench] tree_logprob unique form (agentic tree) {lp['unique_agentic']['ms']:.3f} ms, "
              f"{lp['unique_agentic']['gbps']:.0f} GB/s", flush=True)
        del za

    gw = None
    if not args.no_gateway:
        print("[bench] gateway leg ...", flush=True)
        gw = gateway_leg(seqs, groups, cfg, dev, max(3, args.steps // 2))
        print(f"[bench] gateway: unsplit {gw['unsplit_ms']:.3f} ms, split {gw['split_ms']:.3f} ms", flush=True)

    ssm = None
    if not args.no_ssm:
        print("[bench] tree SSM leg ...", flush=True)
        ssm = ssm_leg(seqs, groups, dev, max(3, args.steps // 2))
        print(f"[bench] gdn fwd {ssm['gdn_fwd_ms']:.3f} ms, gdn bwd {ssm['gdn_bwd_ms']:.3f} ms {ssm['gdn_bwd_kernel_ms']}, "
              f"conv fwd {ssm['conv_fwd_ms']:.3f} ms "
              f"({ssm['conv_fwd_gbps']:.0f} GB/s), conv bwd {ssm['conv_bwd_ms']:.3f} ms", flush=True)

    part = partition_leg()
    print(f"[bench] partition plan: {part['partitions']} partitions, {part['levels']} levels, "
          f"{part['plan_ms_host']:.2f} ms host", flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu oracle baseline ...", flush=True)
        cpu = cpu_baseline(seqs, groups, cfg)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": DESCR[args.workload], "T": T, "visible_pairs": P, "Hq": Hq, "Hkv": Hkv, "d": d,
                   "trees": p["n_trees"], "fwd_bwd_flop": flops},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "packed_tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "tiles_128x64": {"full": full, "partial": partial, "empty": empty, "causal": causal,
                         "skip": round(empty / causal, 4)},
        "kernel_ms": {n: round(x, 4) for n, x in kernel_ms.items()},
        "medians": {k_: head[k_] for k_ in ("fwd_ms_median", "bwd_ms_median", "step_ms_median", "fwd_tflops",
                                            "bwd_tflops", "bwd_tflops_strict_8dPH", "step_tflops", "pct_bf16_peak",
                                            "reps", "warmup")},
        "tiles": head["tiles"], "legs": legs,
        "pack_ms_host": round(pack_ms, 2),
        "roofline": roofline, "tree_logprob": lp, "gateway": gw, "tree_ssm": ssm, "partition": part,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
