"""Pins of the attention oracle: closed forms, a library routine, two
independent formulations, finite differences. CPU only, float64."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attention as OA
from oracle import pack as OP


def _tiny_case(rng, Hq=2, Hkv=1, d=16, n_seqs_max=5, len_max=6, vocab=3):
    seqs, groups = workloads.random_small_forest(rng, n_seqs_max, len_max, vocab)
    p = OP.pack(seqs, groups)
    T = p["T"]
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    do = rng.standard_normal((T, Hq, d))
    return p, q, k, v, do


def test_rope_matches_complex_rotation():
    # rotate-half RoPE == multiply (x_k + i x_{k+d/2}) by exp(i * pos * theta^(-2k/d))
    rng = np.random.default_rng(0)
    L, H, d, theta = 9, 3, 16, 10000.0
    x = rng.standard_normal((L, H, d))
    pos = rng.integers(0, 5000, size=L)
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    freq = np.array([theta ** (-2.0 * kk / d) for kk in range(d // 2)])
    rot = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    want = np.concatenate([rot.real, rot.imag], axis=-1)
    assert np.allclose(OA.rope(x, pos, theta), want, atol=1e-12, rtol=0)
    # position 0 is the identity; the inverse undoes the rotation
    assert np.array_equal(OA.rope(x, np.zeros(L), theta), x)
    assert np.allclose(OA.rope_transpose(OA.rope(x, pos, theta), pos, theta), x, atol=1e-12)


def test_rope_is_relative():
    rng = np.random.default_rng(1)
    d = 16
    a = rng.standard_normal((1, 1, d))
    b = rng.standard_normal((1, 1, d))
    s0 = (OA.rope(a, [7], 1e4) * OA.rope(b, [3], 1e4)).sum()
    s1 = (OA.rope(a, [107], 1e4) * OA.rope(b, [103], 1e4)).sum()
    assert abs(s0 - s1) < 1e-12


def test_zero_queries_closed_form():
    # q = 0: all visible scores are equal, so LSE_i = ln(pos_i + 1) and O_i is
    # the mean of v over i's ancestors and itself
    rng = np.random.default_rng(2)
    for _ in range(20):
        p, q, k, v, _ = _tiny_case(rng, Hq=2, Hkv=2)
        q[:] = 0.0
        O, LSE = OA.forward_branches(q, k, v, p["par"], p["pos"])
        for i in range(p["T"]):
            chain = OP.ancestors_or_self(p["par"], i)
            assert np.allclose(LSE[:, i], np.log(len(chain)), atol=1e-13)
            assert np.allclose(O[i], v[chain].mean(axis=0), atol=1e-13)
        assert np.allclose(np.exp(LSE).sum(axis=1), (p["pos"] + 1).sum())


def test_chain_equals_library_causal_attention():
    rng = np.random.default_rng(3)
    T, Hq, Hkv, d = 11, 4, 2, 16
    p = OP.pack([list(range(T))])
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    O, _ = OA.forward_branches(q, k, v, p["par"], p["pos"])
    pos = np.arange(T)
    # rotate with an independent complex formulation, then torch's SDPA
    freq = np.array([1e4 ** (-2.0 * kk / d) for kk in range(d // 2)])

    def rot(x):
        z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos[:, None, None] * freq)
        return np.concatenate([z.real, z.imag], axis=-1)

    G = Hq // Hkv
    qt = torch.from_numpy(rot(q)).permute(1, 0, 2)
    kt = torch.from_numpy(np.repeat(rot(k), G, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, G, axis=1)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    assert np.allclose(O, ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_branches_equal_dense_mask_and_rows():
    rng = np.random.default_rng(4)
    for _ in range(30):
        p, q, k, v, _ = _tiny_case(rng, Hq=4, Hkv=2)
        O1, L1 = OA.forward_branches(q, k, v, p["par"], p["pos"])
        vis = OP.visibility_dense(p["par"])
        O2, L2 = OA.forward_dense(q, k, v, vis, p["pos"])
        assert np.allclose(O1, O2, atol=1e-12) and np.allclose(L1, L2, atol=1e-12)
        rows = np.arange(p["T"])
        O3, L3 = OA.forward_rows(q, k, v, p["par"], rows)
        assert np.allclose(O1, O3, atol=1e-12) and np.allclose(L1, L3, atol=1e-12)


def _objective(q, k, v, do, p):
    O, _ = OA.forward_dense(q, k, v, OP.visibility_dense(p["par"]), p["pos"])
    return float(np.sum(O * do))


def test_backward_finite_differences():
    rng = np.random.default_rng(5)
    for _ in range(4):
        p, q, k, v, do = _tiny_case(rng, Hq=2, Hkv=1, d=16, n_seqs_max=3, len_max=4)
        dq, dk, dv = OA.backward_branches(q, k, v, do, p["par"], p["pos"])
        eps = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            idx = [tuple(rng.integers(0, s) for s in x.shape) for _ in range(12)]
            for ix in idx:
                xp = x.copy(); xp[ix] += eps
                xm = x.copy(); xm[ix] -= eps
                args_p = dict(q=q, k=k, v=v); args_p[name] = xp
                args_m = dict(q=q, k=k, v=v); args_m[name] = xm
                fd = (_objective(args_p["q"], args_p["k"], args_p["v"], do, p)
                      - _objective(args_m["q"], args_m["k"], args_m["v"], do, p)) / (2 * eps)
                assert abs(fd - g[ix]) < 1e-6 * max(1.0, abs(fd)), (name, ix, fd, g[ix])


def test_sampled_gradient_formulations_agree():
    rng = np.random.default_rng(6)
    for _ in range(10):
        p, q, k, v, do = _tiny_case(rng, Hq=4, Hkv=2)
        dq, dk, dv = OA.backward_branches(q, k, v, do, p["par"], p["pos"])
        rows = np.arange(p["T"])
        assert np.allclose(OA.backward_rows_dq(q, k, v, do, p["par"], rows), dq, atol=1e-11)
        dk2, dv2 = OA.backward_keys(q, k, v, do, p["par"], rows)
        assert np.allclose(dk2, dk, atol=1e-11) and np.allclose(dv2, dv, atol=1e-11)


def test_no_eos_leaves_do_not_feed_shared_values():
    # worked example: with no loss on D, E, G their rows carry no upstream
    # gradient, so V_B collects only what queries B, C and F send it
    rng = np.random.default_rng(7)
    p = OP.pack([[0, 1, 2, 3], [0, 1, 2, 4], [0, 1, 5, 6]])
    T, d = p["T"], 16
    q = rng.standard_normal((T, 1, d))
    k = rng.standard_normal((T, 1, d))
    v = rng.standard_normal((T, 1, d))
    do = rng.standard_normal((T, 1, d))
    do[[3, 4, 6]] = 0.0
    _, _, dv = OA.backward_branches(q, k, v, do, p["par"], p["pos"])
    vis = OP.visibility_dense(p["par"])
    qr, kr = OA.rope(q, p["pos"], 1e4), OA.rope(k, p["pos"], 1e4)
    want = np.zeros(d)
    for i in (1, 2, 5):  # B, C, F
        s = np.where(vis[i], kr[:, 0] @ qr[i, 0] / 4.0, -np.inf)
        pr = np.exp(s - s.max()); pr /= pr.sum()
        want += pr[1] * do[i, 0]
    assert np.allclose(dv[1, 0], want, atol=1e-12)


def test_gqa_group_sum():
    # with all query heads of a group identical, dK/dV equal G times the
    # single-head result
    rng = np.random.default_rng(8)
    p, q, k, v, do = _tiny_case(rng, Hq=1, Hkv=1)
    dq1, dk1, dv1 = OA.backward_branches(q, k, v, do, p["par"], p["pos"])
    G = 3
    dqg, dkg, dvg = OA.backward_branches(np.repeat(q, G, 1), k, v, np.repeat(do, G, 1), p["par"], p["pos"])
    assert np.allclose(dkg, G * dk1, atol=1e-12) and np.allclose(dvg, G * dv1, atol=1e-12)
    assert np.allclose(dqg, np.repeat(dq1, G, 1), atol=1e-12)


def test_chain_formulation_equals_branches():
    """The whole-tree ancestor-chain formulation (each packed row as a query
    once, over its own chain) equals the per-branch oracle on random trees,
    forward and backward, including a GQA group sum and a scale and theta
    other than the defaults."""
    rng = np.random.default_rng(123)
    for trial in range(25):
        seqs, groups = workloads.random_small_forest(rng, n_seqs_max=6, len_max=9, vocab=3, n_groups_max=3)
        p = OP.pack(seqs, groups)
        T = p["T"]
        Hq, Hkv, d = (4, 2, 16) if trial % 2 else (2, 1, 8)
        q, k, v, do = (rng.standard_normal(s) for s in ((T, Hq, d), (T, Hkv, d), (T, Hkv, d), (T, Hq, d)))
        scale, theta = (None, 10000.0) if trial % 3 else (0.3, 500.0)
        O, L = OA.forward_branches(q, k, v, p["par"], p["pos"], scale=scale, theta=theta)
        dq, dk, dv = OA.backward_branches(q, k, v, do, p["par"], p["pos"], scale=scale, theta=theta)
        blk = (2, 3, 256)[trial % 3]  # blocks shorter than the segments, too
        O2, L2 = OA.forward_chains(q, k, v, p["par"], scale=scale, theta=theta, block=blk)
        dq2, dk2, dv2 = OA.backward_chains(q, k, v, do, p["par"], scale=scale, theta=theta, block=blk)
        for a, b in ((O, O2), (L, L2), (dq, dq2), (dk, dk2), (dv, dv2)):
            assert np.max(np.abs(a - b)) < 1e-9
        # one kv group alone: its q heads, its keys
        hk = Hkv - 1
        O3, L3 = OA.forward_chains(q, k, v, p["par"], kv_heads=[hk], scale=scale, theta=theta)
        _, dk3, dv3 = OA.backward_chains(q, k, v, do, p["par"], kv_heads=[hk], scale=scale, theta=theta)
        G = Hq // Hkv
        assert np.max(np.abs(O3 - O[:, hk * G:(hk + 1) * G])) < 1e-9
        assert np.max(np.abs(dk3[:, 0] - dk[:, hk])) < 1e-9 and np.max(np.abs(dv3[:, 0] - dv[:, hk])) < 1e-9
        # an upstream gradient on one q head of the group only: the listed
        # head alone gives the group's dK, dV (the per-branch oracle sees the
        # zero gradients of the other heads)
        h1 = hk * G + G - 1
        do1 = np.zeros_like(do)
        do1[:, h1] = do[:, h1]
        _, dk4, dv4 = OA.backward_branches(q, k, v, do1, p["par"], p["pos"], scale=scale, theta=theta)
        dq5, dk5, dv5 = OA.backward_chains(q, k, v, do1, p["par"], kv_heads=[hk], q_heads=[h1], scale=scale,
                                           theta=theta)
        O5, _ = OA.forward_chains(q, k, v, p["par"], kv_heads=[hk], q_heads=[h1], scale=scale, theta=theta)
        assert np.max(np.abs(dk5[:, 0] - dk4[:, hk])) < 1e-9 and np.max(np.abs(dv5[:, 0] - dv4[:, hk])) < 1e-9
        assert np.max(np.abs(dq5[:, 0] - dq[:, h1])) < 1e-9 and np.max(np.abs(O5[:, 0] - O[:, h1])) < 1e-9


def test_chain_segments_and_depths():
    p = OP.pack(*workloads.sequences("ex_a"))
    # A B C D | E | F G  (E's parent is C, F's parent is B)
    assert OA.chain_segments(p["par"]) == [(0, 4), (4, 5), (5, 7)]
    assert np.array_equal(OA.depths(p["par"]), p["pos"])


def test_theta_zero_is_no_rotation():
    """rope_theta = 0 switches RoPE off: the same as rotating every token by
    position 0 (the identity) at any base, forward and backward."""
    rng = np.random.default_rng(8)
    p = OP.pack(*workloads.random_small_forest(rng, n_seqs_max=5, len_max=8, vocab=3))
    T = p["T"]
    q, k, v, do = (rng.standard_normal(s) for s in ((T, 2, 8), (T, 1, 8), (T, 1, 8), (T, 2, 8)))
    O, L = OA.forward_branches(q, k, v, p["par"], p["pos"], theta=0.0)
    O2, L2 = OA.forward_dense(q, k, v, OP.visibility_dense(p["par"]), np.zeros(T), theta=10000.0)
    assert np.max(np.abs(O - O2)) < 1e-12 and np.max(np.abs(L - L2)) < 1e-12
    x = rng.standard_normal((T, 2, 8))
    assert np.array_equal(OA.rope(x, p["pos"], 0.0), x) and np.array_equal(OA.rope_transpose(x, p["pos"], 0.0), x)
    dq, dk, dv = OA.backward_branches(q, k, v, do, p["par"], p["pos"], theta=0.0)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk))
