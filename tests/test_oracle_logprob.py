"""Pins of the log-prob oracle: the worked example's mapping, the gradient
rule at a shared row, the branch-averaged loss identity, closed forms, a
library routine and finite differences. CPU only, float64."""
import json
import os

import numpy as np
import scipy.special

import workloads
from oracle import logprob as OL
from oracle import pack as OP


def test_lse_matches_library():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((5, 37)) * 4
    assert np.allclose(OL.row_lse(z), scipy.special.logsumexp(z, axis=1), atol=1e-13)


def test_worked_example_entries_and_shared_row_gradient(golden_dir):
    with open(os.path.join(golden_dir, "trie_packing_example.json")) as f:
        gd = json.load(f)
    tok = gd["tokens"]
    seqs = [[tok[c] for c in s] for s in gd["sequences"]]
    p = OP.pack(seqs)
    src, tgt, w = OL.occurrence_entries(p, seqs)
    assert src.tolist() == gd["source_rows"]
    assert tgt.tolist() == [tok[c] for c in gd["targets"]]
    rng = np.random.default_rng(1)
    z = rng.standard_normal((p["T"], 32))
    _, _, _, dz = OL.logprob(z, src, tgt, np.ones(len(src)))
    # row C (packed 2): (p_C - e_D) + (p_C - e_E)
    pc = np.exp(z[2] - scipy.special.logsumexp(z[2]))
    want = 2 * pc
    want[tok["D"]] -= 1
    want[tok["E"]] -= 1
    assert np.allclose(dz[2], want, atol=1e-14)
    # rows D, E, G (leaves) predict nothing
    assert np.all(dz[[3, 4, 6]] == 0)


def test_branch_average_identity():
    # Eq. 1 (per-sequence sums averaged over K) == Eq. 4 (sum_t g_t/K l_t)
    rng = np.random.default_rng(2)
    for _ in range(200):
        seqs, groups = workloads.random_small_forest(rng, vocab=5)
        p = OP.pack(seqs, groups)
        V = 5
        z = rng.standard_normal((p["T"], V)) * 3
        sep = OL.sep_avg_loss(z, p, seqs)
        src, tgt, w = OL.unique_entries(p)
        _, _, tree, _ = OL.logprob(z, src, tgt, w, with_grad=False)
        assert abs(sep - tree) <= 1e-12 * max(1.0, abs(sep))


def test_occurrence_and_unique_forms_agree():
    rng = np.random.default_rng(3)
    for _ in range(50):
        seqs, groups = workloads.random_small_forest(rng, vocab=4)
        p = OP.pack(seqs, groups)
        z = rng.standard_normal((p["T"], 4))
        a = OL.logprob(z, *OL.occurrence_entries(p, seqs))
        b = OL.logprob(z, *OL.unique_entries(p))
        assert abs(a[2] - b[2]) < 1e-12
        assert np.allclose(a[3], b[3], atol=1e-13)


def test_zero_logits_closed_form():
    R, V = 4, 32
    z = np.zeros((R, V))
    src = np.array([0, 1, 1, 3])
    tgt = np.array([5, 0, 31, 5])
    w = np.array([0.5, 1.0, 0.25, 2.0])
    s = 0.7
    logp, lse, loss, dz = OL.logprob(z, src, tgt, w, grad_scale=s)
    assert np.allclose(logp, -np.log(V), atol=1e-15)
    assert abs(-np.log(V) - (-3.4657359027997265)) < 1e-15
    assert abs(loss - w.sum() * np.log(V)) < 1e-13
    want = np.zeros((R, V))
    for m in range(4):
        want[src[m]] += s * w[m] / V
        want[src[m], tgt[m]] -= s * w[m]
    assert np.allclose(dz, want, atol=1e-15)
    assert np.all(dz[2] == 0)


def test_finite_differences():
    rng = np.random.default_rng(4)
    R, V, M = 3, 6, 7
    z = rng.standard_normal((R, V))
    src = rng.integers(0, R, M)
    tgt = rng.integers(0, V, M)
    w = rng.random(M)
    _, _, _, dz = OL.logprob(z, src, tgt, w, grad_scale=1.0)
    eps = 1e-6
    for r in range(R):
        for c in range(V):
            zp = z.copy(); zp[r, c] += eps
            zm = z.copy(); zm[r, c] -= eps
            fd = (OL.logprob(zp, src, tgt, w, with_grad=False)[2]
                  - OL.logprob(zm, src, tgt, w, with_grad=False)[2]) / (2 * eps)
            assert abs(fd - dz[r, c]) < 1e-7


# ---------------------------------------------------------------- clipped policy loss


def _policy_case(seed, R=6, V=11, M=14, margin=0.05, eps=0.2):
    """Random rows and entries whose ratios lie in every region of the clip
    (below 1 - eps, inside, above 1 + eps) but at least `margin` from the
    clip edges, so a finite-difference step never crosses one."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((R, V)) * 2
    src = rng.integers(0, R - 1, M)  # the last row is never referenced
    tgt = rng.integers(0, V, M)
    src[:3] = src[3:6]
    tgt[:3] = tgt[3:6]  # repeated (row, target) pairs with their own advantages
    w = rng.random(M) + 0.1
    adv = rng.standard_normal(M)
    lp, _, _, _ = OL.logprob(z, src, tgt, np.zeros(M), with_grad=False)
    choices = np.array([0.5, 0.7, 0.9, 1.0, 1.1, 1.3, 1.6])
    assert np.min(np.abs(choices[:, None] - np.array([1 - eps, 1 + eps])[None])) >= margin
    r = choices[rng.integers(0, len(choices), M)]
    old = lp - np.log(r)
    return z, src, tgt, w, adv, old


def test_policy_loss_truth_table():
    """The four sign/side cases of the clipped surrogate, values worked by
    hand: (r, A) -> (l, coef = -dl/dlogp) with eps = 0.2, w = 1."""
    z = np.zeros((1, 4))  # logp = -ln 4 for every target
    lp = -np.log(4.0)
    cases = [  # r, A, l, coef
        (1.5, 1.0, -1.2, 0.0),    # A > 0 above the range: clipped, no gradient
        (0.5, 1.0, -0.5, 0.5),    # A > 0 below the range: min is r A, gradient A r
        (0.5, -1.0, 0.8, 0.0),    # A < 0 below the range: clipped
        (1.5, -1.0, 1.5, -1.5),   # A < 0 above the range: min is r A
        (1.1, 2.0, -2.2, 2.2),    # inside the range: unclipped
    ]
    for r, A, l_want, c_want in cases:
        _, _, loss, dz, coef = OL.clipped_policy_loss(z, [0], [1], [1.0], [A], [lp - np.log(r)])
        assert abs(loss - l_want) < 1e-12, (r, A)
        assert abs(coef[0] - c_want) < 1e-12, (r, A)
        # dlogits = coef * (softmax - e_tgt); softmax of zeros is 1/4
        want = np.full(4, 0.25 * c_want)
        want[1] -= c_want
        assert np.allclose(dz[0], want, atol=1e-14)


def test_policy_loss_finite_differences():
    for seed in range(3):
        z, src, tgt, w, adv, old = _policy_case(seed)
        gs = 0.75
        _, _, loss, dz, coef = OL.clipped_policy_loss(z, src, tgt, w, adv, old, grad_scale=gs)
        assert np.any(coef == 0) and np.any(coef != 0)  # both branches are exercised
        h = 1e-6
        fd = np.zeros_like(z)
        for i in range(z.shape[0]):
            for j in range(z.shape[1]):
                zp, zm = z.copy(), z.copy()
                zp[i, j] += h
                zm[i, j] -= h
                fd[i, j] = (OL.clipped_policy_loss(zp, src, tgt, w, adv, old, with_grad=False)[2]
                            - OL.clipped_policy_loss(zm, src, tgt, w, adv, old, with_grad=False)[2]) / (2 * h)
        assert np.max(np.abs(gs * fd - dz)) < 1e-7
        assert np.all(dz[-1] == 0)


def test_policy_loss_on_policy_is_the_policy_gradient_objective():
    """At old_logp = logp (ratio 1) with no clipping, the loss is
    -sum w A (Tree Training §3.1: the RL per-token objective -A log p, whose
    value at the sampling policy contributes -A per unit ratio) and the
    gradient is that of -sum w A log p."""
    z, src, tgt, w, adv, _ = _policy_case(7)
    lp, _, _, _ = OL.logprob(z, src, tgt, np.zeros(len(src)), with_grad=False)
    _, _, loss, dz, _ = OL.clipped_policy_loss(z, src, tgt, w, adv, lp, eps_low=np.inf, eps_high=np.inf)
    assert abs(loss + np.sum(w * adv)) < 1e-12
    # independent gradient of -sum w A logp: w A (softmax - e_tgt) per entry
    soft = np.exp(z - scipy.special.logsumexp(z, axis=1, keepdims=True))
    want = np.zeros_like(z)
    for m in range(len(src)):
        want[src[m]] += w[m] * adv[m] * soft[src[m]]
        want[src[m], tgt[m]] -= w[m] * adv[m]
    assert np.allclose(dz, want, atol=1e-13)


def test_policy_loss_keeps_each_occurrence_advantage():
    """Two occurrences of one prediction with advantages +1 and -1 and ratio
    1.5: per occurrence the loss is -1.2 + 1.5 = 0.3, while averaging the
    advantages first would give 0 (the pages warn against that)."""
    z = np.zeros((1, 4))
    lp = -np.log(4.0)
    _, _, loss, _, coef = OL.clipped_policy_loss(z, [0, 0], [2, 2], [1.0, 1.0], [1.0, -1.0],
                                                 [lp - np.log(1.5)] * 2)
    assert abs(loss - 0.3) < 1e-12
    assert coef.tolist() == [0.0, -1.5]


def test_policy_loss_mask_drops_the_entry():
    z, src, tgt, w, adv, old = _policy_case(11)
    mask = np.ones(len(src))
    mask[[2, 5, 9]] = 0
    _, _, loss, dz, _ = OL.clipped_policy_loss(z, src, tgt, w, adv, old, mask=mask)
    keep = mask > 0
    _, _, loss2, dz2, _ = OL.clipped_policy_loss(z, src[keep], tgt[keep], w[keep], adv[keep], old[keep])
    assert abs(loss - loss2) < 1e-12 and np.allclose(dz, dz2, atol=1e-14)
