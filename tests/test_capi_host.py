"""Host-side tests of the C ABI: the library loads and exports every declared
symbol; tree_pack is bit-exact against the oracle; tile statistics match the
oracle; argument validation returns the documented codes before any HIP call.
No GPU needed."""
import ctypes
import os
import re

import numpy as np
import pytest

import tree_packed_attention_amd as ta
import workloads
from oracle import pack as OP
from oracle import tiles as OT

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_match_header():
    with open(os.path.join(ROOT, "include", "tree_attn.h")) as f:
        hdr = f.read()
    declared = set(re.findall(r"^\s*(?:const char\*|int|size_t)\s+(tree_\w+)\s*\(", hdr, re.M))
    assert declared == set(ta.EXPORTS)
    lib = ta.library()
    for name in declared:
        assert hasattr(lib, name), name


def _compare(p, o):
    pairs = [("ids", "ids"), ("pos", "pos"), ("subtree_end", "se"), ("parent", "par"), ("path_count", "g"),
             ("node_start", "node_start"), ("node_end", "node_end"), ("node_parent", "node_parent"),
             ("node_subtree_end", "node_se"), ("tree_start", "tree_start")]
    for a, b in pairs:
        assert np.array_equal(p[a], o[b]), a
    assert p["weight"].dtype == np.float32 and np.array_equal(p["weight"].view(np.uint32), o["weight"].view(np.uint32))
    assert np.array_equal(p["occ_map"], np.concatenate(o["occ"]))
    assert (p["T"], p["n_nodes"], p["n_trees"]) == (o["T"], o["n_nodes"], o["n_trees"])


@pytest.mark.parametrize("name", ["ex_a", "ex_b", "short", "multistep", "agentic", "agentic_l"])
def test_pack_bit_exact_workloads(name):
    seqs, groups = workloads.sequences(name)
    _compare(ta.tree_pack(seqs, groups), OP.pack(seqs, groups))


def test_pack_bit_exact_random_forests():
    rng = np.random.default_rng(99)
    for _ in range(1500):
        seqs, groups = workloads.random_small_forest(rng, n_seqs_max=8, len_max=10, vocab=4, n_groups_max=4)
        _compare(ta.tree_pack(seqs, groups), OP.pack(seqs, groups))


def test_pack_negative_and_large_token_ids():
    seqs = [[-5, 2 ** 31 - 1, 7], [-5, 2 ** 31 - 1, -2 ** 31], [0]]
    _compare(ta.tree_pack(seqs), OP.pack(seqs))


def _raw_pack(flat, offsets, n, groups=None, cap_T=None, cap_nodes=None):
    lib = ta.library()
    total = int(offsets[-1]) if len(offsets) else 0
    cap = max(total, 1)
    bufs = [np.zeros(cap, np.int32) for _ in range(12)]
    sizes = ta.PackSizes()
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = lib.tree_pack(ptr(flat), ptr(offsets), n, ptr(groups), cap if cap_T is None else cap_T,
                       cap if cap_nodes is None else cap_nodes, *[ptr(b) for b in bufs], ctypes.byref(sizes))
    return rc, sizes


def test_pack_errors():
    flat = np.array([1, 2, 3, 4], np.int32)
    rc, _ = _raw_pack(flat, np.array([0, 2, 2, 4], np.int64), 3)
    assert rc == ta.TA_EINVAL and "empty" in ta.last_error()
    rc, _ = _raw_pack(flat, np.array([1, 4], np.int64), 1)
    assert rc == ta.TA_EINVAL
    rc, _ = _raw_pack(flat, np.array([0, 4], np.int64), 0)
    assert rc == ta.TA_EINVAL
    rc, _ = _raw_pack(None, np.array([0, 4], np.int64), 1)
    assert rc == ta.TA_EINVAL
    rc, sizes = _raw_pack(np.array([1, 2, 1, 3], np.int32), np.array([0, 2, 4], np.int64), 2, cap_T=0, cap_nodes=0)
    assert rc == ta.TA_ECAPACITY
    assert (sizes.T, sizes.n_nodes, sizes.n_trees) == (3, 3, 1)
    rc, sizes = _raw_pack(np.array([1, 2, 1, 3], np.int32), np.array([0, 2, 4], np.int64), 2, cap_T=3, cap_nodes=3)
    assert rc == ta.TA_OK and ta.last_error() == ""


@pytest.mark.parametrize("BQ,BK", [(128, 64), (64, 128), (128, 128), (7, 5)])
def test_tile_stats_match_oracle(BQ, BK):
    for name in ("ex_a", "ex_b", "short"):
        p = OP.pack(*workloads.sequences(name))
        assert ta.tree_tile_stats(p["se"], p["T"], BQ, BK) == OT.tile_stats(p["se"], p["T"], BQ, BK)
    rng = np.random.default_rng(5)
    for _ in range(100):
        p = OP.pack(*workloads.random_small_forest(rng, 8, 12, 3))
        assert ta.tree_tile_stats(p["se"], p["T"], BQ, BK) == OT.tile_stats(p["se"], p["T"], BQ, BK)


def test_tile_stats_errors():
    se = np.array([1], np.int32)
    with pytest.raises(ta.TreeAttnError) as e:
        ta.tree_tile_stats(se, 0, 128, 64)
    assert e.value.code == ta.TA_EINVAL


def _gpu_visible():
    import torch

    return torch.cuda.device_count() > 0  # counts devices without initialising one


@pytest.mark.skipif(_gpu_visible(), reason="passes dangling device pointers: run only where no GPU is visible")
def test_device_entry_points_validate_before_hip():
    """Bad arguments are rejected on the host: these calls pass dangling
    pointers on purpose, which would fault if any HIP work were issued, so
    the test runs only on a host without a GPU."""
    lib = ta.library()
    bogus = ctypes.c_void_p(0x1000)
    ws_need = lib.tree_attn_workspace_bytes(100, 4, 2, 64, 0)
    assert ws_need > 0 and ws_need % 256 == 0
    assert lib.tree_attn_workspace_bytes(100, 4, 2, 64, 1) > ws_need
    args = lambda T=100, Hq=4, Hkv=2, d=64, ws=ws_need, wsp=bogus, dt=ta.TA_BF16: (
        bogus, bogus, bogus, dt, T, Hq, Hkv, d, bogus, bogus, 0.0, 10000.0, bogus, bogus, wsp, ws, None)
    assert lib.tree_attn_fwd(*args(T=0)) == ta.TA_EINVAL
    assert lib.tree_attn_fwd(*args(Hq=6, Hkv=4)) == ta.TA_EINVAL
    assert lib.tree_attn_fwd(*args(d=32)) == ta.TA_EUNSUPPORTED
    assert "head dim" in ta.last_error()
    assert lib.tree_attn_fwd(*args(ws=ws_need - 1)) == ta.TA_EINVAL
    assert "workspace too small" in ta.last_error()
    assert lib.tree_attn_fwd(*args(wsp=ctypes.c_void_p(0x1008))) == ta.TA_EINVAL
    assert lib.tree_attn_fwd(*args(dt=7)) == ta.TA_EINVAL
    a = list(args())
    a[8] = None  # pos
    assert lib.tree_attn_fwd(*a) == ta.TA_EINVAL
    a = list(args())
    a[1] = ctypes.c_void_p(0x1008)  # k not 16-byte aligned
    assert lib.tree_attn_fwd(*a) == ta.TA_EINVAL and "16-byte aligned" in ta.last_error()
    bw = lib.tree_attn_workspace_bytes(100, 4, 2, 64, 1)
    bargs = [bogus] * 6 + [ta.TA_BF16, 100, 4, 2, 64, bogus, bogus, 0.0, 1e4, 0, bogus, bogus, bogus, bogus, bw, None]
    bad_flags = list(bargs)
    bad_flags[15] = 8
    assert lib.tree_attn_bwd(*bad_flags) == ta.TA_EINVAL
    small = list(bargs)
    small[20] = ws_need  # forward-sized workspace is too small for the backward
    assert lib.tree_attn_bwd(*small) == ta.TA_EINVAL
    mis = list(bargs)
    mis[5] = ctypes.c_void_p(0x1004)  # dout not 16-byte aligned
    assert lib.tree_attn_bwd(*mis) == ta.TA_EINVAL and "16-byte aligned" in ta.last_error()
    acc_plain = list(bargs)
    acc_plain[15] = ta.TA_ACCUMULATE_PAST  # only meaningful with cached rows
    assert lib.tree_attn_bwd(*acc_plain) == ta.TA_EINVAL
    # partition-boundary entry points
    gw_need = lib.tree_attn_gw_workspace_bytes(100, 300, 4, 2, 64, 0)
    assert gw_need > ws_need
    assert lib.tree_attn_gw_workspace_bytes(100, -1, 4, 2, 64, 0) == 0
    gargs = lambda Lp=300, off=5, kp=bogus, vis=bogus, ws=gw_need: (
        bogus, bogus, bogus, ta.TA_BF16, 100, 4, 2, 64, bogus, bogus, off, kp, bogus, vis, Lp, 0.0, 1e4, bogus,
        bogus, bogus, ws, None)
    assert lib.tree_attn_gw_fwd(*gargs(Lp=-3)) == ta.TA_EINVAL
    assert lib.tree_attn_gw_fwd(*gargs(off=-1)) == ta.TA_EINVAL
    assert lib.tree_attn_gw_fwd(*gargs(kp=None)) == ta.TA_EINVAL and "past" in ta.last_error()
    assert lib.tree_attn_gw_fwd(*gargs(vis=None)) == ta.TA_EINVAL
    assert lib.tree_attn_gw_fwd(*gargs(kp=ctypes.c_void_p(0x1008))) == ta.TA_EINVAL
    assert lib.tree_attn_gw_fwd(*gargs(ws=gw_need - 1)) == ta.TA_EINVAL
    gbw = lib.tree_attn_gw_workspace_bytes(100, 300, 4, 2, 64, 1)
    gb = [bogus] * 6 + [ta.TA_BF16, 100, 4, 2, 64, bogus, bogus, 5, bogus, bogus, bogus, 300, 0.0, 1e4, 0,
                        bogus, bogus, bogus, bogus, bogus, bogus, gbw, None]
    nodk = list(gb)
    nodk[24] = None  # dk_past
    assert lib.tree_attn_gw_bwd(*nodk) == ta.TA_EINVAL
    badf = list(gb)
    badf[20] = 4
    assert lib.tree_attn_gw_bwd(*badf) == ta.TA_EINVAL
    lw = lib.tree_logprob_workspace_bytes(16, 48)
    assert lw > 0
    largs = lambda R=16, V=100, M=48, ws=lw: (bogus, ta.TA_BF16, R, V, bogus, bogus, bogus, M, bogus, None, None,
                                              None, 1.0, bogus, ws, None)
    assert lib.tree_logprob(*largs(R=0)) == ta.TA_EINVAL
    assert lib.tree_logprob(*largs(V=0)) == ta.TA_EINVAL
    assert lib.tree_logprob(*largs(M=-1)) == ta.TA_EINVAL
    assert lib.tree_logprob(*largs(ws=lw - 1)) == ta.TA_EINVAL
    pargs = lambda eps_low=0.2, eps_high=0.2, adv=bogus, old=bogus, ws=lw: (
        bogus, ta.TA_BF16, 16, 100, bogus, bogus, bogus, adv, old, None, 48, eps_low, eps_high, bogus, None, None,
        None, 1.0, bogus, ws, None)
    assert lib.tree_logprob_ppo(*pargs(eps_low=-0.1)) == ta.TA_EINVAL and "eps" in ta.last_error()
    assert lib.tree_logprob_ppo(*pargs(eps_high=float("nan"))) == ta.TA_EINVAL
    assert lib.tree_logprob_ppo(*pargs(adv=None)) == ta.TA_EINVAL and "advantage" in ta.last_error()
    assert lib.tree_logprob_ppo(*pargs(old=None)) == ta.TA_EINVAL
    assert lib.tree_logprob_ppo(*pargs(ws=lw - 1)) == ta.TA_EINVAL
    # read-back of the device tile plan: shape checks before any copy
    pc = lambda n=2, T=100, ws=ws_need, ne=bogus: lib.tree_attn_plan_counts(bogus, ws, T, 0, 4, 2, 64, n, ne, bogus,
                                                                           None)
    assert pc(n=3) == ta.TA_EINVAL and "n_qtiles" in ta.last_error()
    assert pc(T=0) == ta.TA_EINVAL
    assert pc(ws=ws_need - 1) == ta.TA_EINVAL
    assert pc(ne=None) == ta.TA_EINVAL
    st = ctypes.c_int32(0)
    assert lib.tree_attn_workspace_status(None, ctypes.byref(st), None) == ta.TA_EINVAL
    assert lib.tree_attn_workspace_status(bogus, None, None) == ta.TA_EINVAL
