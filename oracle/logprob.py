"""Oracle: per-occurrence log-probabilities on shared logit rows, weighted
loss, and the gradient scatter-added into the shared rows.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows
---------------
* "Trie packing" page, "Share logits, preserve every prediction": the row of
  node u predicts the token after u; nine prediction occurrences of the worked
  example use four distinct rows, gathered as log_softmax(z)[source_rows,
  targets].
* Same page, "Combine gradients at the shared logits": for target y,
  l = -z_y + log sum_j exp z_j, so dl/dz = p - e_y, and the contributions of
  several targets on one row add.
* "Tree Training" §3.1 Eq. 1-4 and §3.2 "Loss Weights": the branch-averaged
  loss equals sum_t (g_t / K) l_t, a per-token weight applied elementwise.

Definitions (float64):
  lse_r   = log sum_v exp z[r, v]
  logp_m  = z[src_m, tgt_m] - lse[src_m]
  loss    = -sum_m w_m logp_m
  dlogits = grad_scale * d loss / d z
          = grad_scale * sum_{m: src_m = r} w_m (softmax(z_r) - e_{tgt_m})
Rows that no entry references get a zero gradient.
"""
from __future__ import annotations

import numpy as np


def row_lse(z):
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]


def logprob(z, src, tgt, w, grad_scale=1.0, with_grad=True):
    """Returns (logp [M], lse [R], loss scalar, dlogits [R, V] or None)."""
    z = np.asarray(z, dtype=np.float64)
    src = np.asarray(src, dtype=np.int64)
    tgt = np.asarray(tgt, dtype=np.int64)
    w = np.asarray(w, dtype=np.float64)
    lse = row_lse(z)
    logp = z[src, tgt] - lse[src]
    loss = -np.sum(w * logp)
    if not with_grad:
        return logp, lse, loss, None
    R, V = z.shape
    soft = np.exp(z - lse[:, None])
    dz = np.zeros((R, V))
    for m in range(len(src)):
        r = src[m]
        dz[r] += w[m] * soft[r]
        dz[r, tgt[m]] -= w[m]
    return logp, lse, loss, grad_scale * dz


def occurrence_entries(packed, seqs):
    """One entry per original prediction occurrence ("Trie packing" page, the
    source_rows / targets arrays): for sequence k and offset s < len_k - 1,
    row = packed index of token s, target = token s+1, weight = 1 / K_k."""
    src, tgt, w = [], [], []
    kot = packed["K_of_token"]
    for k, s in enumerate(seqs):
        occ = packed["occ"][k]
        K = kot[occ[0]]
        for a in range(len(s) - 1):
            src.append(occ[a])
            tgt.append(int(s[a + 1]))
            w.append(1.0 / K)
    return np.array(src, np.int64), np.array(tgt, np.int64), np.array(w, np.float64)


def unique_entries(packed):
    """One entry per packed token that has a parent: row = its parent, target =
    the token, weight = g_t / K (Eq. 4). A tree root predicts nothing."""
    par, ids = packed["par"], packed["ids"]
    g, kot = packed["g"], packed["K_of_token"]
    t = np.nonzero(par >= 0)[0]
    return par[t].astype(np.int64), ids[t].astype(np.int64), g[t] / kot[t].astype(np.float64)


def sep_avg_loss(z, packed, seqs, groups=None):
    """Eq. 1 computed literally: every sequence on its own, per-sequence sums
    of -log p(next token), averaged over the K sequences of its tree, trees
    added. Row logits of an unpacked occurrence are the packed row's logits
    (forward equivalence, Eq. 6)."""
    z = np.asarray(z, dtype=np.float64)
    lse = row_lse(z)
    kot = packed["K_of_token"]
    total = 0.0
    for k, s in enumerate(seqs):
        occ = packed["occ"][k]
        K = kot[occ[0]]
        seq_sum = 0.0
        for a in range(len(s) - 1):
            r = occ[a]
            seq_sum += -(z[r, int(s[a + 1])] - lse[r])
        total += seq_sum / K
    return total


def clipped_policy_loss(z, src, tgt, w, adv, old_logp, mask=None, eps_low=0.2, eps_high=0.2, grad_scale=1.0,
                        with_grad=True):
    """Per-occurrence clipped policy loss on shared logit rows.

    Follows the "Trie packing" page (the PPO/GRPO paragraph after "Why
    indexing matters": every occurrence keeps its own advantage, old
    log-probability, clipping, mask and weight; advantages are not averaged
    before the nonlinear loss) and "Tree Training" §3.1 (an RL per-token
    objective -A_t log p, weighted like any per-token loss). The clipping
    rule is not spelled out on the pages; it is read as the PPO clipped
    surrogate (Schulman et al., 2017, the clipped objective):

      r_m    = exp(logp_m - old_logp_m)
      l_m    = -min(r_m A_m, clip(r_m, 1 - eps_low, 1 + eps_high) A_m)
      loss   = sum_m w_m mask_m l_m
      dloss/dlogp_m = -w_m mask_m A_m r_m   if r_m A_m <= clip(r_m) A_m
                      0                     otherwise (the clipped branch is
                                            the minimum, a constant in logp)
      dlogits_r = grad_scale * sum_{m: src_m = r} dloss/dlogp_m (e_{tgt_m} - softmax(z_r))

    At a tie inside the clip range both branches have the same derivative, so
    ties count as unclipped. Returns (logp [M], lse [R], loss, dlogits [R, V]
    or None, coef [M] = -dloss/dlogp)."""
    logp, lse, _, _ = logprob(z, src, tgt, np.zeros(len(np.asarray(src))), with_grad=False)
    w = np.asarray(w, dtype=np.float64)
    adv = np.asarray(adv, dtype=np.float64)
    old = np.asarray(old_logp, dtype=np.float64)
    mk = np.ones_like(w) if mask is None else np.asarray(mask, dtype=np.float64)
    r = np.exp(logp - old)
    a = r * adv
    b = np.clip(r, 1.0 - eps_low, 1.0 + eps_high) * adv
    loss = float(np.sum(w * mk * -np.minimum(a, b)))
    coef = np.where(a <= b, w * mk * adv * r, 0.0)
    if not with_grad:
        return logp, lse, loss, None, coef
    # the gradient through logp is the weighted log-prob gradient with the
    # per-entry coefficients in place of the weights
    _, _, _, dz = logprob(z, src, tgt, coef, grad_scale=grad_scale)
    return logp, lse, loss, dz, coef
