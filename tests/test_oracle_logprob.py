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
