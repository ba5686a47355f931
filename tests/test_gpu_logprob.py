"""GPU parity of tree_logprob against the float64 oracle.

Tolerances (mirroring the attention ones):
logp, row lse and loss max-abs <= 2e-2 (loss relative for large M); dlogits
relative L2 <= 5e-2. Tighter internal checks: logp max-abs <= 1e-3 for
float32 logits.
"""
import numpy as np
import pytest
import torch

import tree_packed_attention_amd as ta
import workloads
from oracle import logprob as OL
from oracle import pack as OP

pytestmark = pytest.mark.gpu


def host(t):
    return t.detach().double().cpu().numpy()


def _run(z, src, tgt, w, gs=1.0, with_grad=True):
    zt = z.cuda()
    s = torch.as_tensor(np.asarray(src), dtype=torch.int32).cuda()
    t = torch.as_tensor(np.asarray(tgt), dtype=torch.int32).cuda()
    ww = torch.as_tensor(np.asarray(w), dtype=torch.float32).cuda()
    out = ta.tree_logprob(zt, s, t, ww, grad_scale=gs, with_grad=with_grad)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["ex_a", "ex_b"])
@pytest.mark.parametrize("form", ["occurrence", "unique"])
def test_worked_examples(name, form):
    seqs, groups = workloads.sequences(name)
    po = OP.pack(seqs, groups)
    if form == "occurrence":
        src, tgt, w = OL.occurrence_entries(po, seqs)
    else:
        src, tgt, w = OL.unique_entries(po)
    z = workloads.logits_input(po["T"], 32, "f32", 1)
    logp, lse, loss, dz = _run(z, src, tgt, w.astype(np.float32), gs=0.5)
    r_logp, r_lse, r_loss, r_dz = OL.logprob(z.double().numpy(), src, tgt, w.astype(np.float32), grad_scale=0.5)
    assert np.max(np.abs(host(logp) - r_logp)) <= 1e-5
    assert np.max(np.abs(host(lse) - r_lse)) <= 1e-5
    assert abs(float(loss) - r_loss) <= 1e-5
    assert np.max(np.abs(host(dz) - r_dz)) <= 1e-6


@pytest.mark.parametrize("V,dtype", [(1000, "bf16"), (1003, "bf16"), (32000, "bf16"), (5000, "f32"), (7, "f32")])
def test_random_rows(V, dtype):
    R, M = 50, 400
    rng = np.random.default_rng(V)
    src = rng.integers(0, R - 3, M)      # the last 3 rows are never referenced
    tgt = rng.integers(0, V, M)
    tgt[:40] = tgt[40:80]                # repeated (row, target) pairs are common
    src[:40] = src[40:80]
    w = rng.random(M).astype(np.float32)
    z = workloads.logits_input(R, V, dtype, V) * 3
    logp, lse, loss, dz = _run(z, src, tgt, w, gs=1.5)
    r_logp, r_lse, r_loss, r_dz = OL.logprob(z.double().numpy(), src, tgt, w, grad_scale=1.5)
    assert np.max(np.abs(host(logp) - r_logp)) <= (1e-3 if dtype == "f32" else 2e-2)
    assert np.max(np.abs(host(lse) - r_lse)) <= 2e-2
    assert abs(float(loss) - r_loss) <= 2e-2 * max(1.0, abs(r_loss)) * 1e-2
    d = host(dz)
    assert np.linalg.norm(d - r_dz) / np.linalg.norm(r_dz) <= 5e-2
    assert np.all(d[R - 3:] == 0)


def test_agentic_unique_form_weights():
    """Per-token weights g/K on the 32768-token agentic tree, unique form
    (M = T - 1) over bf16 logits [32768, 32000]; sampled rows."""
    seqs, groups = workloads.sequences("agentic")
    p = ta.tree_pack(seqs, groups)
    po = OP.pack(seqs, groups)
    assert np.array_equal(p["weight"].view(np.uint32), po["weight"].view(np.uint32))
    t = np.nonzero(p["parent"] >= 0)[0]
    src, tgt, w = p["parent"][t], p["ids"][t], p["weight"][t]
    z = workloads.logits_input(p["T"], 32000, "bf16", 4, device="cuda")
    logp, lse, loss, dz = _run(z, src, tgt, w)
    rows = np.unique(np.concatenate([src[:: 997], [0, p["T"] - 2]]))
    zr = host(z[torch.as_tensor(rows, device="cuda")])
    sel = np.isin(src, rows)
    remap = {int(r): n for n, r in enumerate(rows)}
    s2 = np.array([remap[int(x)] for x in src[sel]])
    r_logp, r_lse, _, r_dz = OL.logprob(zr, s2, tgt[sel], w[sel])
    assert np.max(np.abs(host(logp)[sel] - r_logp)) <= 2e-2
    assert np.max(np.abs(host(lse)[rows] - r_lse)) <= 2e-2
    d = host(dz[torch.as_tensor(rows, device="cuda")])
    assert np.linalg.norm(d - r_dz) / np.linalg.norm(r_dz) <= 5e-2
    # the loss over all entries from the GPU's own logp is the GPU loss
    lp = host(logp)
    assert abs(float(loss) + float(np.sum(w.astype(np.float64) * lp))) <= 1e-3 * abs(float(loss))


def test_large_vocab_repeated_rows_full_size():
    """16384 bf16 rows x 151936 vocab, every row referenced 3 times (M = 49152,
    w = 1/3). Loss over all rows (row lse from the oracle, in chunks); logp
    and lse of every row; dlogits of every row at the columns no entry
    targets, and in full (target corrections included) on sampled rows."""
    R, V = 16384, 151936
    src, tgt, w = workloads.repeated_rows_entries(R, V, 3, 5)
    z = workloads.logits_input(R, V, "bf16", 5, device="cuda")
    logp, lse, loss, dz = _run(z, src, tgt, w)
    # loss via oracle lse of every row, chunked
    r_lse = np.empty(R)
    for a in range(0, R, 512):
        r_lse[a:a + 512] = OL.row_lse(host(z[a:a + 512]))
    zt = host(z[torch.as_tensor(src.astype(np.int64), device="cuda"), torch.as_tensor(tgt.astype(np.int64), device="cuda")])
    r_logp_all = zt - r_lse[src]
    r_loss = -np.sum(w.astype(np.float64) * r_logp_all)
    assert np.max(np.abs(host(lse) - r_lse)) <= 2e-2
    assert np.max(np.abs(host(logp) - r_logp_all)) <= 2e-2
    assert abs(float(loss) - r_loss) <= 2e-2 * 1e-3 * abs(r_loss) + 2e-2
    rows = np.array([0, 1, 777, 8191, 16383])
    sel = np.isin(src, rows)
    remap = {int(r): n for n, r in enumerate(rows)}
    _, _, _, r_dz = OL.logprob(host(z[torch.as_tensor(rows, device="cuda")]),
                               np.array([remap[int(x)] for x in src[sel]]), tgt[sel], w[sel])
    d = host(dz[torch.as_tensor(rows, device="cuda")])
    assert np.linalg.norm(d - r_dz) / np.linalg.norm(r_dz) <= 5e-2
    # every row, every column that no entry targets: dlogits = W_r p = W_r exp(z - lse_r)
    # with the oracle's lse (W_r = sum of the row's weights), to bf16 rounding
    W = np.bincount(src, weights=w.astype(np.float64), minlength=R)
    src_t = torch.as_tensor(src.astype(np.int64), device="cuda")
    tgt_t = torch.as_tensor(tgt.astype(np.int64), device="cuda")
    for a in range(0, R, 512):
        b = min(a + 512, R)
        lse_c = torch.as_tensor(r_lse[a:b], device="cuda", dtype=torch.float64)
        W_c = torch.as_tensor(W[a:b], device="cuda", dtype=torch.float64)
        exp = (W_c[:, None] * torch.exp(z[a:b].double() - lse_c[:, None])).float()
        diff = (dz[a:b].float() - exp).abs()
        m = (src_t >= a) & (src_t < b)
        diff[src_t[m] - a, tgt_t[m]] = 0.0  # target columns: checked on the sampled rows above
        assert bool((diff <= 1e-2 * exp + 1e-7).all()), a


def test_invalid_entries_and_forward_only():
    R, V = 8, 64
    z = workloads.logits_input(R, V, "f32", 2)
    src = np.array([0, 9, 3, -1, 2, 2])
    tgt = np.array([1, 1, 64, 5, 3, 3])
    w = np.ones(6, np.float32)
    logp, lse, loss, dz = _run(z, src, tgt, w)
    lp = host(logp)
    assert np.isnan(lp[[1, 2, 3]]).all() and np.isfinite(lp[[0, 4, 5]]).all()
    assert np.isnan(float(loss))
    valid = [0, 4, 5]
    _, _, _, r_dz = OL.logprob(z.double().numpy(), src[valid], tgt[valid], w[valid])
    assert np.max(np.abs(host(dz) - r_dz)) <= 1e-6
    logp2, _, _, dz2 = _run(z, src[valid], tgt[valid], w[valid], with_grad=False)
    assert dz2 is None and np.max(np.abs(host(logp2) - lp[valid])) == 0


# Row sizes on both sides of the 256 entries the row kernel keeps in LDS:
# rows up to 256 entries take the LDS entry tables, larger rows (1500 is also
# more than one entry per thread) the general path; targets repeat in a row.
WIDE_COUNTS = [0, 1, 255, 256, 257, 1500, 3, 0]


def _wide_rows(seed):
    rng = np.random.default_rng(seed)
    src = np.concatenate([np.full(c, r) for r, c in enumerate(WIDE_COUNTS)])
    tgt = rng.integers(0, 300, src.size)
    perm = rng.permutation(src.size)
    return src[perm], tgt[perm], rng


# 4096 / 2052: 256 threads per row; 32768: the largest row at 256 threads (16
# vectors each); 40000: 1024 threads per row
@pytest.mark.parametrize("V,dtype", [(4096, "bf16"), (2052, "f32"), (32768, "bf16"), (40000, "bf16")])
def test_wide_rows_both_paths(V, dtype):
    R = len(WIDE_COUNTS)
    src, tgt, rng = _wide_rows(V)
    w = rng.random(src.size).astype(np.float32)
    z = workloads.logits_input(R, V, dtype, 7) * 3
    logp, lse, loss, dz = _run(z, src, tgt, w, gs=0.75)
    r_logp, r_lse, r_loss, r_dz = OL.logprob(z.double().numpy(), src, tgt, w, grad_scale=0.75)
    assert np.max(np.abs(host(logp) - r_logp)) <= (1e-3 if dtype == "f32" else 2e-2)
    assert np.max(np.abs(host(lse) - r_lse)) <= 2e-2
    assert abs(float(loss) - r_loss) <= 1e-4 * max(1.0, abs(r_loss))
    d = host(dz)
    for r in range(R):  # every row, both paths, element by element, relative to the row's scale
        # (W_r p reaches tens here: float32 rounding of lse and of the sums)
        tol = (2e-5 if dtype == "f32" else 2e-2) * max(1.0, np.max(np.abs(r_dz[r])))
        assert np.max(np.abs(d[r] - r_dz[r])) <= tol, r
    assert np.all(d[[0, R - 1]] == 0)
    again = _run(z, src, tgt, w, gs=0.75)
    for x, y in zip((logp, lse, loss, dz), again):
        assert torch.equal(x, y)


def test_wide_rows_policy_loss():
    V, R = 4096, len(WIDE_COUNTS)
    src, tgt, rng = _wide_rows(5)
    M = src.size
    w = (rng.random(M) + 0.1).astype(np.float32)
    adv, ratio, mask = workloads.policy_inputs(M, 11)
    z = workloads.logits_input(R, V, "f32", 8) * 3
    zd = z.double().numpy()
    old = _old_logp(zd, src, tgt, ratio)
    logp, lse, loss, dz = _run_ppo(z, src, tgt, w, adv, old, mask, gs=1.25)
    r_logp, r_lse, r_loss, r_dz, coef = OL.clipped_policy_loss(zd, src, tgt, w, adv, old, mask, EPS, EPS, 1.25)
    assert np.any(coef == 0) and np.any(coef != 0)
    assert np.max(np.abs(host(logp) - r_logp)) <= 1e-3
    assert abs(float(loss) - r_loss) <= 1e-4 * max(1.0, abs(r_loss))
    d = host(dz)
    for r in range(R):
        assert np.max(np.abs(d[r] - r_dz[r])) <= 1e-4 * max(1.0, np.max(np.abs(r_dz[r]))), r


def test_bitwise_deterministic():
    R, V, M = 300, 4096, 3000
    rng = np.random.default_rng(1)
    src = rng.integers(0, R, M)
    tgt = rng.integers(0, 16, M)  # many duplicate targets per row
    w = rng.random(M).astype(np.float32)
    z = workloads.logits_input(R, V, "bf16", 3)
    a = _run(z, src, tgt, w)
    b = _run(z, src, tgt, w)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ---------------------------------------------------------------- clipped policy loss

EPS = 0.2


def _run_ppo(z, src, tgt, w, adv, old, mask, gs=1.0, with_grad=True, eps=(EPS, EPS)):
    cu = lambda a, dt: torch.as_tensor(np.asarray(a), dtype=dt).cuda()
    out = ta.tree_logprob_ppo(z.cuda(), cu(src, torch.int32), cu(tgt, torch.int32), cu(w, torch.float32),
                              cu(adv, torch.float32), cu(old, torch.float32),
                              None if mask is None else cu(mask, torch.uint8), eps_low=eps[0], eps_high=eps[1],
                              grad_scale=gs, with_grad=with_grad)
    torch.cuda.synchronize()
    return out


def _old_logp(zd, src, tgt, ratio):
    """old_logp from the oracle's logp and the drawn ratios (rounded to fp32,
    as the kernel reads it)."""
    lp = zd[src, tgt] - OL.row_lse(zd)[src]
    return (lp - np.log(ratio)).astype(np.float32)


@pytest.mark.parametrize("V,dtype", [(1000, "bf16"), (1003, "bf16"), (32000, "bf16"), (5000, "f32"), (7, "f32")])
def test_policy_loss_random_rows(V, dtype):
    R, M = 50, 400
    rng = np.random.default_rng(V + 7)
    src = rng.integers(0, R - 3, M)      # the last 3 rows are never referenced
    tgt = rng.integers(0, V, M)
    tgt[:40] = tgt[40:80]                # repeated predictions, each with its own advantage
    src[:40] = src[40:80]
    w = (rng.random(M) + 0.1).astype(np.float32)
    adv, ratio, mask = workloads.policy_inputs(M, V)
    z = workloads.logits_input(R, V, dtype, V) * 3
    zd = z.double().numpy()
    old = _old_logp(zd, src, tgt, ratio)
    logp, lse, loss, dz = _run_ppo(z, src, tgt, w, adv, old, mask, gs=1.5)
    r_logp, r_lse, r_loss, r_dz, coef = OL.clipped_policy_loss(zd, src, tgt, w, adv, old, mask, EPS, EPS, 1.5)
    assert np.any(coef == 0) and np.any(coef != 0)
    assert np.max(np.abs(host(logp) - r_logp)) <= (1e-3 if dtype == "f32" else 2e-2)
    assert np.max(np.abs(host(lse) - r_lse)) <= 2e-2
    assert abs(float(loss) - r_loss) <= 1e-3 * max(1.0, abs(r_loss))
    d = host(dz)
    assert np.linalg.norm(d - r_dz) / np.linalg.norm(r_dz) <= 5e-2
    assert np.all(d[R - 3:] == 0)


def test_policy_loss_small_exact_f32():
    """The worked example's occurrence entries (fp32 logits, vocab 32) with
    per-occurrence advantages: tight agreement."""
    seqs, groups = workloads.sequences("ex_a")
    po = OP.pack(seqs, groups)
    src, tgt, w = OL.occurrence_entries(po, seqs)
    M = len(src)
    adv, ratio, mask = workloads.policy_inputs(M, 1, mask_frac=0.2)
    z = workloads.logits_input(po["T"], 32, "f32", 1)
    zd = z.double().numpy()
    old = _old_logp(zd, src, tgt, ratio)
    logp, lse, loss, dz = _run_ppo(z, src, tgt, w.astype(np.float32), adv, old, mask, gs=0.5)
    r_logp, _, r_loss, r_dz, _ = OL.clipped_policy_loss(zd, src, tgt, w.astype(np.float32), adv, old, mask, EPS, EPS,
                                                        0.5)
    assert np.max(np.abs(host(logp) - r_logp)) <= 1e-5
    assert abs(float(loss) - r_loss) <= 1e-5
    assert np.max(np.abs(host(dz) - r_dz)) <= 1e-6


def test_policy_loss_unclipped_on_policy_equals_weighted_logprob():
    """No clipping (eps = inf): the gradient coefficient is w A r, so with
    ratio ~1 the result matches tree_logprob with weights w A (up to r - 1,
    i.e. fp32 rounding of old_logp)."""
    R, V, M = 40, 2000, 300
    rng = np.random.default_rng(3)
    src = rng.integers(0, R, M)
    tgt = rng.integers(0, V, M)
    w = (rng.random(M) + 0.1).astype(np.float32)
    adv, _, _ = workloads.policy_inputs(M, 3)
    z = workloads.logits_input(R, V, "f32", 9)
    zd = z.double().numpy()
    old = _old_logp(zd, src, tgt, np.ones(M))
    _, _, loss, dz = _run_ppo(z, src, tgt, w, adv, old, None, eps=(float("inf"), float("inf")))
    _, _, _, dz2 = _run(z, src, tgt, (w * adv).astype(np.float32))
    assert abs(float(loss) + float(np.sum(w.astype(np.float64) * adv))) <= 1e-4 * np.sum(np.abs(w * adv))
    assert np.max(np.abs(host(dz) - host(dz2))) <= 1e-5


def test_policy_loss_large_vocab_full_size():
    """16384 bf16 rows x 151936 vocab, every row referenced 3 times (M =
    49152), per-entry advantages, ratios in every clip region, 10 % masked.
    Loss and logp over all entries (row lse from the oracle, in chunks);
    dlogits on sampled rows."""
    R, V = 16384, 151936
    src, tgt, w = workloads.repeated_rows_entries(R, V, 3, 5)
    M = len(src)
    adv, ratio, mask = workloads.policy_inputs(M, 5)
    z = workloads.logits_input(R, V, "bf16", 5, device="cuda")
    r_lse = np.empty(R)
    for a in range(0, R, 512):
        r_lse[a:a + 512] = OL.row_lse(host(z[a:a + 512]))
    zt = host(z[torch.as_tensor(src.astype(np.int64), device="cuda"), torch.as_tensor(tgt.astype(np.int64), device="cuda")])
    r_logp = zt - r_lse[src]
    old = (r_logp - np.log(ratio)).astype(np.float32)
    logp, lse, loss, dz = _run_ppo(z, src, tgt, w, adv, old, mask)
    r = np.exp(r_logp - old.astype(np.float64))
    a_, b_ = r * adv, np.clip(r, 1 - EPS, 1 + EPS) * adv
    r_loss = float(np.sum(w * mask * -np.minimum(a_, b_)))
    assert np.max(np.abs(host(lse) - r_lse)) <= 2e-2
    assert np.max(np.abs(host(logp) - r_logp)) <= 2e-2
    assert abs(float(loss) - r_loss) <= 1e-3 * np.sum(np.abs(w * adv)) + 2e-2
    rows = np.array([0, 1, 777, 8191, 16383])
    sel = np.isin(src, rows)
    remap = {int(x): n for n, x in enumerate(rows)}
    _, _, _, r_dz, _ = OL.clipped_policy_loss(host(z[torch.as_tensor(rows, device="cuda")]),
                                              np.array([remap[int(x)] for x in src[sel]]), tgt[sel], w[sel], adv[sel],
                                              old[sel], mask[sel], EPS, EPS)
    d = host(dz[torch.as_tensor(rows, device="cuda")])
    assert np.linalg.norm(d - r_dz) / np.linalg.norm(r_dz) <= 5e-2


def test_policy_loss_invalid_and_masked_entries_and_determinism():
    R, V = 8, 64
    z = workloads.logits_input(R, V, "f32", 2)
    src = np.array([0, 9, 3, 2, 2, 5])
    tgt = np.array([1, 1, 3, 3, 3, 70])
    w = np.ones(6, np.float32)
    adv = np.array([1, 1, -1, 2, -2, 1], np.float32)
    old = np.full(6, -3.0, np.float32)
    mask = np.array([1, 1, 1, 1, 1, 0], np.uint8)   # the second invalid entry is masked
    logp, _, loss, dz = _run_ppo(z, src, tgt, w, adv, old, mask)
    lp = host(logp)
    assert np.isnan(lp[[1, 5]]).all() and np.isfinite(lp[[0, 2, 3, 4]]).all()
    assert np.isnan(float(loss))                    # entry 1 is invalid and on
    valid = [0, 2, 3, 4]
    _, _, _, r_dz, _ = OL.clipped_policy_loss(z.double().numpy(), src[valid], tgt[valid], w[valid], adv[valid],
                                              old[valid], mask[valid], EPS, EPS)
    assert np.max(np.abs(host(dz) - r_dz)) <= 1e-5
    mask[1] = 0
    _, _, loss2, _ = _run_ppo(z, src, tgt, w, adv, old, mask)
    assert np.isfinite(float(loss2))
    a = _run_ppo(z, src, tgt, w, adv, old, mask)
    b = _run_ppo(z, src, tgt, w, adv, old, mask)
    bits = lambda t: t.reshape(-1).view(torch.uint8)  # NaN logp of invalid entries compared bitwise
    for x, y in zip(a, b):
        assert torch.equal(bits(x), bits(y))
