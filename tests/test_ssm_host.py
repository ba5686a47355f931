"""Host-side tests of the tree SSM entry points: the chunk plan of
tree_gdn_plan checked against its definition on random forests, and argument
validation of tree_conv_* / tree_gdn_* before any HIP call. No GPU needed."""
import ctypes

import numpy as np
import pytest

import tree_packed_attention_amd as ta
import workloads
from oracle import pack as OP


def _decode(plan):
    nc, nch, nl, chunk, T = plan[:5]
    o = 8
    cs = plan[o:o + nc]; o += nc
    cl = plan[o:o + nc]; o += nc
    cp = plan[o:o + nc]; o += nc
    cb = plan[o:o + nch + 1]; o += nch + 1
    lc = plan[o:o + nch]; o += nch
    lo = plan[o:o + nl + 1]; o += nl + 1
    co = plan[o:o + nc + 1]; o += nc + 1
    cc = plan[o:o + nch]; o += nch
    assert o == len(plan)
    return dict(nc=nc, nch=nch, nl=nl, chunk=chunk, T=T, cs=cs, cl=cl, cp=cp, cb=cb, lc=lc, lo=lo, co=co, cc=cc)


@pytest.mark.parametrize("seed,chunk", [(1, 64), (2, 16), (3, 5), (4, 1), (5, 64)])
def test_plan_matches_its_definition(seed, chunk):
    seqs, groups = workloads.random_forest(seed, [300, 170, 61], max_depth=5, seg_lo=1, seg_hi=90)
    po = OP.pack(seqs, groups)
    p = _decode(ta.tree_gdn_plan(po["node_start"], po["node_end"], po["node_parent"], chunk))
    T, par = po["T"], po["par"]
    assert p["T"] == T and p["chunk"] == chunk
    # chunks tile [0, T) in order, never cross a node, at most `chunk` long
    assert p["cs"][0] == 0 and np.all(p["cs"][1:] == p["cs"][:-1] + p["cl"][:-1]) and p["cs"][-1] + p["cl"][-1] == T
    assert np.all((p["cl"] >= 1) & (p["cl"] <= chunk))
    node_of = np.repeat(np.arange(po["n_nodes"]), po["node_end"] - po["node_start"])
    assert np.all(node_of[p["cs"]] == node_of[p["cs"] + p["cl"] - 1])
    # a chunk's parent chunk holds the token-level parent of its first token
    chunk_of = np.repeat(np.arange(p["nc"]), p["cl"])
    for c in range(p["nc"]):
        t = p["cs"][c]
        assert p["cp"][c] == (chunk_of[par[t]] if par[t] >= 0 else -1)
        # inside a chunk every token's parent is the token before it
        assert np.all(par[t + 1:t + p["cl"][c]] == np.arange(t, t + p["cl"][c] - 1))
    # chains: maximal runs with parent = previous chunk
    starts = [c for c in range(p["nc"]) if c == 0 or p["cp"][c] != c - 1]
    assert list(p["cb"][:-1]) == starts and p["cb"][-1] == p["nc"]
    chain_of = np.repeat(np.arange(p["nch"]), np.diff(p["cb"]))
    level = np.zeros(p["nch"], int)
    for ch in range(p["nch"]):
        pc = p["cp"][p["cb"][ch]]
        level[ch] = 0 if pc < 0 else level[chain_of[pc]] + 1
    assert p["nl"] == level.max() + 1
    for l in range(p["nl"]):
        got = p["lc"][p["lo"][l]:p["lo"][l + 1]]
        assert list(got) == [ch for ch in range(p["nch"]) if level[ch] == l]
    # child chains of every chunk, in increasing order
    for c in range(p["nc"]):
        got = p["cc"][p["co"][c]:p["co"][c + 1]]
        assert list(got) == [ch for ch in range(p["nch"]) if p["cp"][p["cb"][ch]] == c]
    assert p["co"][-1] == sum(1 for ch in range(p["nch"]) if p["cp"][p["cb"][ch]] >= 0)


def test_plan_errors():
    ns, ne, npar = np.array([0, 5], np.int32), np.array([5, 9], np.int32), np.array([-1, 0], np.int32)
    with pytest.raises(ta.TreeAttnError):
        ta.tree_gdn_plan(ns, ne, npar, chunk=65)
    with pytest.raises(ta.TreeAttnError):
        ta.tree_gdn_plan(ns, np.array([5, 5], np.int32), npar)       # empty node
    with pytest.raises(ta.TreeAttnError):
        ta.tree_gdn_plan(np.array([0, 6], np.int32), ne, npar)       # gap in the layout
    with pytest.raises(ta.TreeAttnError):
        ta.tree_gdn_plan(ns, ne, np.array([-1, 1], np.int32))        # parent not before the node


def test_ssm_argument_validation():
    lib = ta.library()
    bogus = ctypes.c_void_p(0x1000)
    cargs = lambda T=10, C=16, K=4, x=bogus, act=1: (x, ta.TA_BF16, T, C, K, bogus, None, bogus, act, bogus, None)
    assert lib.tree_conv_fwd(*cargs(C=12)) == ta.TA_EINVAL
    assert lib.tree_conv_fwd(*cargs(K=9)) == ta.TA_EINVAL
    assert lib.tree_conv_fwd(*cargs(T=0)) == ta.TA_EINVAL
    assert lib.tree_conv_fwd(*cargs(act=2)) == ta.TA_EINVAL
    assert lib.tree_conv_fwd(*cargs(x=ctypes.c_void_p(0x1008))) == ta.TA_EINVAL
    assert lib.tree_conv_fwd(*cargs(x=None)) == ta.TA_EINVAL
    cw = lib.tree_conv_workspace_bytes(10, 16, 4)
    assert cw > 0
    bargs = lambda ws=cw, C=16: (bogus, bogus, ta.TA_BF16, 10, C, 4, bogus, None, bogus, bogus, bogus, 1, bogus, bogus,
                                 None, bogus, ws, None)
    assert lib.tree_conv_bwd(*bargs(ws=cw - 1)) == ta.TA_EINVAL
    assert lib.tree_conv_bwd(*bargs(C=7)) == ta.TA_EINVAL
    plan = ta.tree_gdn_plan(np.array([0], np.int32), np.array([10], np.int32), np.array([-1], np.int32))
    pp = plan.ctypes.data_as(ctypes.c_void_p)
    gw = lib.tree_gdn_workspace_bytes(2, 4, 64, 64, int(plan[0]))
    gargs = lambda T=10, H=2, Hv=4, dk=64, dv=64, ph=pp, ws=gw: (bogus, bogus, bogus, ta.TA_BF16, bogus, bogus, T, H, Hv,
                                                                 dk, dv, bogus, ph, bogus, bogus, ws, None)
    assert lib.tree_gdn_fwd(*gargs(dk=96)) == ta.TA_EUNSUPPORTED
    assert lib.tree_gdn_fwd(*gargs(Hv=3)) == ta.TA_EINVAL
    assert lib.tree_gdn_fwd(*gargs(T=11)) == ta.TA_EINVAL and "plan" in ta.last_error()
    assert lib.tree_gdn_fwd(*gargs(ws=gw - 1)) == ta.TA_EINVAL
    assert lib.tree_gdn_fwd(*gargs(ph=None)) == ta.TA_EINVAL
    bad = plan.copy()
    bad[3] = 99
    assert lib.tree_gdn_fwd(*gargs(ph=bad.ctypes.data_as(ctypes.c_void_p))) == ta.TA_EINVAL
    # backward: its workspace holds the forward's plus its own
    gb = lib.tree_gdn_bwd_workspace_bytes(2, 4, 64, 64, int(plan[0]), int(plan[1]))
    assert gb > gw
    assert lib.tree_gdn_bwd_workspace_bytes(2, 4, 64, 64, int(plan[0]), int(plan[0]) + 1) == 0
    bw = lambda T=10, H=2, Hv=4, dk=64, dv=64, ph=pp, ws=gb, dq=bogus: (
        bogus, bogus, bogus, ta.TA_BF16, bogus, bogus, bogus, T, H, Hv, dk, dv, bogus, ph, dq, bogus, bogus, bogus,
        bogus, bogus, ws, None)
    assert lib.tree_gdn_bwd(*bw(dk=96)) == ta.TA_EUNSUPPORTED
    assert lib.tree_gdn_bwd(*bw(Hv=3)) == ta.TA_EINVAL
    assert lib.tree_gdn_bwd(*bw(T=11)) == ta.TA_EINVAL and "plan" in ta.last_error()
    assert lib.tree_gdn_bwd(*bw(ws=gw)) == ta.TA_EINVAL and "workspace" in ta.last_error()
    assert lib.tree_gdn_bwd(*bw(dq=None)) == ta.TA_EINVAL
    assert lib.tree_gdn_bwd(*bw(dq=ctypes.c_void_p(0x1008))) == ta.TA_EINVAL
    assert lib.tree_gdn_bwd(*bw(ph=bad.ctypes.data_as(ctypes.c_void_p))) == ta.TA_EINVAL


# ----------------------------------------------------------------- partition planner

from oracle import partition as OPT  # noqa: E402


@pytest.mark.parametrize("seed", range(12))
def test_partition_bit_exact_against_oracle(seed):
    seqs, groups = workloads.random_forest(seed, [400, 150, 33], max_depth=6, seg_lo=1, seg_hi=70)
    po = OP.pack(seqs, groups)
    lens = (po["node_end"] - po["node_start"]).tolist()
    for C in sorted(c for c in {max(lens), max(lens) + 7, 120, 300, 10 ** 7} if c >= max(lens)):
        got = ta.tree_partition(po["node_start"], po["node_end"], po["node_parent"], C)
        want = OPT.plan(lens, po["node_parent"].tolist(), C)
        for key in ("node_part", "part_tokens", "part_parent", "part_cut"):
            assert np.array_equal(got[key], want[key]), (C, key)


def test_partition_random_agentic_tree():
    """The 131072-token depth-10 tree at a 32768-token capacity: invariants
    and agreement with the oracle."""
    seqs, groups = workloads.sequences("agentic_l")
    p = ta.tree_pack(seqs, groups)
    got = ta.tree_partition(p["node_start"], p["node_end"], p["node_parent"], 32768)
    lens = (p["node_end"] - p["node_start"]).tolist()
    want = OPT.plan(lens, p["node_parent"].tolist(), 32768)
    assert np.array_equal(got["node_part"], want["node_part"])
    assert got["part_tokens"].max() <= 32768 and got["part_tokens"].sum() == p["T"]
    assert len(got["part_tokens"]) >= -(-p["T"] // 32768)


def test_partition_errors():
    ns, ne, npar = np.array([0, 5], np.int32), np.array([5, 9], np.int32), np.array([-1, 0], np.int32)
    with pytest.raises(ta.TreeAttnError):
        ta.tree_partition(ns, ne, npar, 4)                            # node 0 is longer than the capacity
    with pytest.raises(ta.TreeAttnError):
        ta.tree_partition(ns, ne, np.array([-1, 1], np.int32), 10)    # parent not before its node
