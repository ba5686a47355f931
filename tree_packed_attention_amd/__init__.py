"""Python binding of libtreeattn.so, the MI355X (gfx950) tree-packed attention library.

Argument marshalling only: every step runs in the library (the host packer
and the HIP kernels). PyTorch supplies device memory and the current stream.
The names follow the C ABI in include/tree_attn.h:

  tree_pack(seqs, groups=None)                     host packer -> dict of numpy arrays
  tree_tile_stats(subtree_end, T, BQ, BK)          host tile classification counts
  tree_attn_fwd(q, k, v, pos, subtree_end, ...)    -> (o, lse)
  tree_attn_bwd(q, k, v, o, lse, dout, pos, subtree_end, ...) -> (dq, dk, dv)
  tree_logprob(logits, src_row, target, weight, ...) -> (logp, row_lse, loss, dlogits)
  tree_logprob_ppo(logits, src_row, target, weight, advantage, old_logp, ...) -> (logp, row_lse, loss, dlogits)
  tree_conv_fwd / tree_conv_bwd(x, ..., parent, ...)  tree-correct causal conv1d and its gradients
  tree_partition(node_start, node_end, node_parent, capacity)  host partition plan -> dict
  tree_gdn_plan(node_start, node_end, node_parent)  host chunk schedule -> int32 numpy plan
  tree_gdn_fwd(q, k, v, g, beta, plan, ...)        tree-routed gated delta rule -> o
  tree_gdn_bwd(q, k, v, g, beta, do, plan, ws)     its gradients -> (dq, dk, dv, dg, dbeta)
  gdn_workspace(q, v, plan, backward=False)        workspace for tree_gdn_fwd (and tree_gdn_bwd)
  TreeAttention                                    torch.autograd.Function over fwd/bwd

The library must be built first (python tree_packed_attention_amd/build.py);
importing this package without it raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtreeattn.so")

TA_OK, TA_EINVAL, TA_ECAPACITY, TA_EUNSUPPORTED, TA_EHIP = 0, -1, -2, -3, -4
TA_BF16, TA_F32 = 0, 1
TA_REUSE_PREP, TA_ACCUMULATE_PAST = 1, 2
TA_STATUS_SUBTREE_END = 1

EXPORTS = (
    "tree_attn_last_error",
    "tree_pack",
    "tree_attn_workspace_bytes",
    "tree_attn_fwd",
    "tree_attn_bwd",
    "tree_attn_gw_workspace_bytes",
    "tree_attn_gw_fwd",
    "tree_attn_gw_bwd",
    "tree_logprob_workspace_bytes",
    "tree_logprob",
    "tree_logprob_ppo",
    "tree_tile_stats",
    "tree_partition",
    "tree_conv_fwd",
    "tree_conv_workspace_bytes",
    "tree_conv_bwd",
    "tree_gdn_plan",
    "tree_gdn_workspace_bytes",
    "tree_gdn_fwd",
    "tree_gdn_bwd_workspace_bytes",
    "tree_gdn_bwd",
    "tree_attn_profile_enable",
    "tree_attn_profile_read",
    "tree_attn_workspace_status",
    "tree_attn_plan_counts",
    "tree_attn_gw_export",
    "tree_attn_gw_relay",
    "tree_logprob_noalloc",
)


class TreeAttnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python tree_packed_attention_amd/build.py` "
        "(there is no fallback implementation)"
    )

# torch ships its own HIP runtime under the same soname; loading torch first
# makes the library bind to that one runtime instead of a second copy.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)
_p, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class PackSizes(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("n_nodes", ctypes.c_int32), ("n_trees", ctypes.c_int32)]


class GdnPlanSizes(ctypes.Structure):
    _fields_ = [("n_chunks", ctypes.c_int32), ("n_chains", ctypes.c_int32), ("n_levels", ctypes.c_int32),
                ("plan_ints", ctypes.c_int32)]


_lib.tree_attn_last_error.restype = ctypes.c_char_p
_lib.tree_attn_last_error.argtypes = []
_lib.tree_pack.restype = ctypes.c_int
_lib.tree_pack.argtypes = [_p, _p, _i32, _p, _i32, _i32] + [_p] * 12 + [ctypes.POINTER(PackSizes)]
_lib.tree_attn_workspace_bytes.restype = _sz
_lib.tree_attn_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32]
_lib.tree_attn_fwd.restype = ctypes.c_int
_lib.tree_attn_fwd.argtypes = [_p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _p, _p, _f32, _f32,
                               _p, _p, _p, _sz, _p]
_lib.tree_attn_bwd.restype = ctypes.c_int
_lib.tree_attn_bwd.argtypes = [_p, _p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _p, _p, _f32, _f32,
                               _i32, _p, _p, _p, _p, _sz, _p]
_lib.tree_attn_gw_workspace_bytes.restype = _sz
_lib.tree_attn_gw_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
_lib.tree_attn_gw_fwd.restype = ctypes.c_int
_lib.tree_attn_gw_fwd.argtypes = [_p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _p, _p, _i32, _p, _p, _p, _i32,
                                  _f32, _f32, _p, _p, _p, _sz, _p]
_lib.tree_attn_gw_bwd.restype = ctypes.c_int
_lib.tree_attn_gw_bwd.argtypes = [_p, _p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _p, _p, _i32, _p, _p,
                                  _p, _i32, _f32, _f32, _i32, _p, _p, _p, _p, _p, _p, _sz, _p]
_lib.tree_logprob_workspace_bytes.restype = _sz
_lib.tree_logprob_workspace_bytes.argtypes = [_i64, _i64]
_lib.tree_logprob.restype = ctypes.c_int
_lib.tree_logprob.argtypes = [_p, ctypes.c_int, _i64, _i64, _p, _p, _p, _i64, _p, _p, _p, _p, _f32, _p, _sz, _p]
_lib.tree_logprob_noalloc.restype = ctypes.c_int
_lib.tree_logprob_noalloc.argtypes = [_p, ctypes.c_int, _i64, _i64, _p, _p, _p, _i64, _p, _p, _p, _p, _f32, _p]
_lib.tree_logprob_ppo.restype = ctypes.c_int
_lib.tree_logprob_ppo.argtypes = [_p, ctypes.c_int, _i64, _i64, _p, _p, _p, _p, _p, _p, _i64, _f32, _f32, _p, _p, _p,
                                  _p, _f32, _p, _sz, _p]
_lib.tree_partition.restype = ctypes.c_int
_lib.tree_partition.argtypes = [_p, _p, _p, _i32, _i64, _p, _p, _p, _p, ctypes.POINTER(ctypes.c_int32)]
_lib.tree_conv_fwd.restype = ctypes.c_int
_lib.tree_conv_fwd.argtypes = [_p, ctypes.c_int, _i32, _i32, _i32, _p, _p, _p, _i32, _p, _p]
_lib.tree_conv_workspace_bytes.restype = _sz
_lib.tree_conv_workspace_bytes.argtypes = [_i32, _i32, _i32]
_lib.tree_conv_bwd.restype = ctypes.c_int
_lib.tree_conv_bwd.argtypes = [_p, _p, ctypes.c_int, _i32, _i32, _i32, _p, _p, _p, _p, _p, _i32, _p, _p, _p, _p, _sz,
                               _p]
_lib.tree_gdn_plan.restype = ctypes.c_int
_lib.tree_gdn_plan.argtypes = [_p, _p, _p, _i32, _i32, _p, _i32, ctypes.POINTER(GdnPlanSizes)]
_lib.tree_gdn_workspace_bytes.restype = _sz
_lib.tree_gdn_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32]
_lib.tree_gdn_fwd.restype = ctypes.c_int
_lib.tree_gdn_fwd.argtypes = [_p, _p, _p, ctypes.c_int, _p, _p, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _sz, _p]
_lib.tree_gdn_bwd_workspace_bytes.restype = _sz
_lib.tree_gdn_bwd_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
_lib.tree_gdn_bwd.restype = ctypes.c_int
_lib.tree_gdn_bwd.argtypes = [_p, _p, _p, ctypes.c_int, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p,
                              _p, _p, _p, _sz, _p]
_lib.tree_tile_stats.restype = ctypes.c_int
_lib.tree_tile_stats.argtypes = [_p, _i32, _i32, _i32] + [ctypes.POINTER(ctypes.c_int64)] * 4
_lib.tree_attn_workspace_status.restype = ctypes.c_int
_lib.tree_attn_workspace_status.argtypes = [_p, ctypes.POINTER(ctypes.c_int32), _p]
_lib.tree_attn_plan_counts.restype = ctypes.c_int
_lib.tree_attn_plan_counts.argtypes = [_p, _sz, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p]
_lib.tree_attn_gw_export.restype = ctypes.c_int
_lib.tree_attn_gw_export.argtypes = [_p, _p, ctypes.c_int, _i32, _i32, _i32, _p, _i32, _f32, _p, _i32, _p, _p, _p]
_lib.tree_attn_gw_relay.restype = ctypes.c_int
_lib.tree_attn_gw_relay.argtypes = [_p, _p, _p, _i32, ctypes.c_int, _i32, _i32, _i32, _p, _i32, _f32, _p, _p, _p]
_lib.tree_attn_profile_enable.restype = ctypes.c_int
_lib.tree_attn_profile_enable.argtypes = [_i32]
_lib.tree_attn_profile_read.restype = ctypes.c_int
_lib.tree_attn_profile_read.argtypes = [_i32, ctypes.c_char_p, _i32, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64)]


def library():
    """The loaded ctypes handle (for tests of the raw ABI)."""
    return _lib


def last_error() -> str:
    return _lib.tree_attn_last_error().decode()


def _check(rc):
    if rc != TA_OK:
        raise TreeAttnError(rc, last_error())


def _np_ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------------------- host


def tree_pack(seqs, groups=None):
    """Packs sequences (iterables of ints) into DFS-serialized prefix trees.

    Returns a dict of int32 / float32 numpy arrays: ids, pos, subtree_end,
    parent, path_count, weight, occ_map (flat) and seq_offsets, node_start,
    node_end, node_parent, node_subtree_end, tree_start; plus T, n_nodes,
    n_trees.
    """
    lens = [len(s) for s in seqs]
    offsets = np.zeros(len(seqs) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lens)
    flat = np.zeros(max(int(offsets[-1]), 1), dtype=np.int32)
    if offsets[-1] > 0:
        flat[: offsets[-1]] = np.concatenate([np.asarray(s, dtype=np.int64) for s in seqs]).astype(np.int32)
    grp = None if groups is None else np.ascontiguousarray(groups, dtype=np.int32)
    total = int(offsets[-1])
    cap = max(total, 1)
    out = {k: np.zeros(cap, dtype=np.int32) for k in
           ("ids", "pos", "subtree_end", "parent", "path_count", "node_start", "node_end", "node_parent",
            "node_subtree_end")}
    out["weight"] = np.zeros(cap, dtype=np.float32)
    out["occ_map"] = np.zeros(cap, dtype=np.int32)
    out["tree_start"] = np.zeros(len(seqs) + 1, dtype=np.int32)
    sizes = PackSizes()
    rc = _lib.tree_pack(_np_ptr(flat), _np_ptr(offsets), len(seqs), _np_ptr(grp), cap, cap,
                        _np_ptr(out["ids"]), _np_ptr(out["pos"]), _np_ptr(out["subtree_end"]),
                        _np_ptr(out["parent"]), _np_ptr(out["path_count"]), _np_ptr(out["weight"]),
                        _np_ptr(out["occ_map"]), _np_ptr(out["node_start"]), _np_ptr(out["node_end"]),
                        _np_ptr(out["node_parent"]), _np_ptr(out["node_subtree_end"]), _np_ptr(out["tree_start"]),
                        ctypes.byref(sizes))
    _check(rc)
    T, N, R = sizes.T, sizes.n_nodes, sizes.n_trees
    for key in ("ids", "pos", "subtree_end", "parent", "path_count", "weight"):
        out[key] = out[key][:T].copy()
    for key in ("node_start", "node_end", "node_parent", "node_subtree_end"):
        out[key] = out[key][:N].copy()
    out["occ_map"] = out["occ_map"][:total].copy()
    out["tree_start"] = out["tree_start"][: R + 1].copy()
    out["seq_offsets"] = offsets
    out.update(T=T, n_nodes=N, n_trees=R)
    return out


def tree_tile_stats(subtree_end, T, BQ, BK):
    se = np.ascontiguousarray(subtree_end, dtype=np.int32)
    vals = [ctypes.c_int64() for _ in range(4)]
    _check(_lib.tree_tile_stats(_np_ptr(se), int(T), int(BQ), int(BK), *[ctypes.byref(v) for v in vals]))
    return tuple(v.value for v in vals)  # full, partial, empty, causal


def tree_attn_profile_enable(on=True):
    _check(_lib.tree_attn_profile_enable(1 if on else 0))


def tree_attn_profile_read():
    """{kernel group: (total_ms, launches)} recorded since profiling was enabled."""
    out = {}
    idx = 0
    buf = ctypes.create_string_buffer(64)
    while True:
        ms, cnt = ctypes.c_double(), ctypes.c_int64()
        if _lib.tree_attn_profile_read(idx, buf, 64, ctypes.byref(ms), ctypes.byref(cnt)) != TA_OK:
            return out
        out[buf.value.decode()] = (ms.value, cnt.value)
        idx += 1


# ---------------------------------------------------------------------------- device


def _torch():
    import torch

    return torch


def _dt(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return TA_BF16
    if t.dtype == torch.float32:
        return TA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev_ptr(t, name, dtype=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, name, shape):
    """Raises ValueError unless tensor t has exactly `shape` (None = any size)."""
    got = tuple(t.shape)
    if len(got) != len(shape) or any(w is not None and g != w for g, w in zip(got, shape)):
        raise ValueError(f"{name} has shape {got}, expected {tuple('*' if w is None else w for w in shape)}")
    return t


def _check_attn(q, k, v, pos, subtree_end, o=None, lse=None, dout=None, past_len=None):
    """Shapes of the attention tensors against (T, Hq, Hkv, d) from q and k."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError(f"q and k must be [T, H, d] (got {tuple(q.shape)} and {tuple(k.shape)})")
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    _shape(k, "k", (T, Hkv, d))
    _shape(v, "v", (T, Hkv, d))
    _shape(pos, "pos", (T,))
    _shape(subtree_end, "subtree_end", (T,))
    if o is not None:
        _shape(o, "o", (T, Hq, d))
    if lse is not None:
        _shape(lse, "lse", (Hq, T))
    if dout is not None:
        _shape(dout, "dout", (T, Hq, d))
    return T, Hq, Hkv, d


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def attn_workspace(T, Hq, Hkv, d, with_bwd, device):
    nbytes = _lib.tree_attn_workspace_bytes(T, Hq, Hkv, d, 1 if with_bwd else 0)
    return _torch().empty(max(nbytes, 256), dtype=_torch().uint8, device=device)


def tree_attn_fwd(q, k, v, pos, subtree_end, softmax_scale=0.0, rope_theta=10000.0, workspace=None,
                  with_bwd_workspace=False):
    """q [T,Hq,d], k/v [T,Hkv,d] (bf16 or f32, same dtype) -> (o [T,Hq,d], lse [Hq,T] f32).

    Returns (o, lse, workspace); pass the workspace to tree_attn_bwd with
    reuse_prep=True to skip the RoPE and tile-plan pass there.
    """
    torch = _torch()
    T, Hq, Hkv, d = _check_attn(q, k, v, pos, subtree_end)
    dev = q.device
    if workspace is None:
        workspace = attn_workspace(T, Hq, Hkv, d, with_bwd_workspace, dev)
    o = torch.empty_like(q)
    lse = torch.empty(Hq, T, dtype=torch.float32, device=dev)
    rc = _lib.tree_attn_fwd(_dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype, dev), _dev_ptr(v, "v", q.dtype, dev), _dt(q),
                            T, Hq, Hkv, d, _dev_ptr(pos, "pos", torch.int32, dev),
                            _dev_ptr(subtree_end, "subtree_end", torch.int32, dev), float(softmax_scale),
                            float(rope_theta), _dev_ptr(o, "o"), _dev_ptr(lse, "lse"),
                            _dev_ptr(workspace, "workspace"), workspace.numel(), _stream(dev))
    _check(rc)
    return o, lse, workspace


def tree_attn_bwd(q, k, v, o, lse, dout, pos, subtree_end, softmax_scale=0.0, rope_theta=10000.0,
                  workspace=None, reuse_prep=False):
    """Gradients (dq, dk, dv) of sum(o * dout); dk/dv summed over each kv group."""
    torch = _torch()
    T, Hq, Hkv, d = _check_attn(q, k, v, pos, subtree_end, o=o, lse=lse, dout=dout)
    dev = q.device
    if workspace is None:
        if reuse_prep:
            raise ValueError("reuse_prep needs the forward's workspace")
        workspace = attn_workspace(T, Hq, Hkv, d, True, dev)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    rc = _lib.tree_attn_bwd(_dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype, dev), _dev_ptr(v, "v", q.dtype, dev),
                            _dev_ptr(o, "o", q.dtype, dev), _dev_ptr(lse, "lse", torch.float32, dev),
                            _dev_ptr(dout, "dout", q.dtype, dev), _dt(q), T, Hq, Hkv, d,
                            _dev_ptr(pos, "pos", torch.int32, dev),
                            _dev_ptr(subtree_end, "subtree_end", torch.int32, dev), float(softmax_scale),
                            float(rope_theta), TA_REUSE_PREP if reuse_prep else 0, _dev_ptr(dq, "dq"),
                            _dev_ptr(dk, "dk"), _dev_ptr(dv, "dv"), _dev_ptr(workspace, "workspace"),
                            workspace.numel(), _stream(dev))
    _check(rc)
    return dq, dk, dv


def tree_attn_workspace_status(workspace):
    """Status word of an attention workspace after its last prep pass (0 = no
    data error; TA_STATUS_SUBTREE_END = a subtree end was clamped). Waits for
    the current stream."""
    st = ctypes.c_int32(0)
    _check(_lib.tree_attn_workspace_status(_dev_ptr(workspace, "workspace"), ctypes.byref(st),
                                           _stream(workspace.device)))
    return st.value


def tree_attn_plan_counts(workspace, T, Hq, Hkv, d, past_len=0):
    """Per 128-row query tile: (non-empty, full) 64-key tile counts of the
    device tile plan in `workspace`, as int32 numpy arrays. Waits for the
    current stream."""
    Lq = -(-int(past_len) // 128) * 128
    nq = -(-(Lq + int(T)) // 256) * 2
    ne = np.zeros(nq, np.int32)
    fu = np.zeros(nq, np.int32)
    _check(_lib.tree_attn_plan_counts(_dev_ptr(workspace, "workspace"), workspace.numel(), int(T), int(past_len),
                                      int(Hq), int(Hkv), int(d), nq, _np_ptr(ne), _np_ptr(fu),
                                      _stream(workspace.device)))
    return ne, fu


def gw_workspace(T, past_len, Hq, Hkv, d, with_bwd, device):
    nbytes = _lib.tree_attn_gw_workspace_bytes(T, past_len, Hq, Hkv, d, 1 if with_bwd else 0)
    if nbytes == 0:
        raise TreeAttnError(TA_EINVAL, f"bad gateway shape T={T} past_len={past_len} Hq={Hq} Hkv={Hkv} d={d}")
    return _torch().empty(nbytes, dtype=_torch().uint8, device=device)


def _past_args(q, k_past, v_past, past_visible):
    torch = _torch()
    dev = q.device
    Lp = k_past.shape[0]
    d = q.shape[2]
    _shape(k_past, "k_past", (Lp, None, d))
    _shape(v_past, "v_past", tuple(k_past.shape))
    _shape(past_visible, "past_visible", (Lp,))
    if Lp == 0:
        return (None, None, None, 0)
    return (_dev_ptr(k_past, "k_past", q.dtype, dev), _dev_ptr(v_past, "v_past", q.dtype, dev),
            _dev_ptr(past_visible, "past_visible", torch.uint8, dev), Lp)


def tree_attn_gw_fwd(q, k, v, pos, subtree_end, pos_offset, k_past, v_past, past_visible, softmax_scale=0.0,
                     rope_theta=10000.0, workspace=None, with_bwd_workspace=False):
    """Tree attention of a child partition over cached ancestor rows.

    q [T,Hq,d], k/v [T,Hkv,d]: the partition's own tokens (pos, subtree_end
    from its packing); k_past (rotated), v_past [past_len,Hkv,d] in q's dtype;
    past_visible uint8 [past_len] (1 = bias 0, 0 = -inf); own positions are
    pos_offset + pos. Returns (o, lse, workspace).
    """
    torch = _torch()
    T, Hq, Hkv, d = _check_attn(q, k, v, pos, subtree_end)
    _shape(k_past, "k_past", (None, Hkv, d))
    dev = q.device
    kp, vp, vis, Lp = _past_args(q, k_past, v_past, past_visible)
    if workspace is None:
        workspace = gw_workspace(T, Lp, Hq, Hkv, d, with_bwd_workspace, dev)
    o = torch.empty_like(q)
    lse = torch.empty(Hq, T, dtype=torch.float32, device=dev)
    rc = _lib.tree_attn_gw_fwd(_dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype, dev), _dev_ptr(v, "v", q.dtype, dev),
                               _dt(q), T, Hq, Hkv, d, _dev_ptr(pos, "pos", torch.int32, dev),
                               _dev_ptr(subtree_end, "subtree_end", torch.int32, dev), int(pos_offset), kp, vp, vis,
                               Lp, float(softmax_scale), float(rope_theta), _dev_ptr(o, "o"), _dev_ptr(lse, "lse"),
                               _dev_ptr(workspace, "workspace"), workspace.numel(), _stream(dev))
    _check(rc)
    return o, lse, workspace


def tree_attn_gw_bwd(q, k, v, o, lse, dout, pos, subtree_end, pos_offset, k_past, v_past, past_visible,
                     softmax_scale=0.0, rope_theta=10000.0, workspace=None, reuse_prep=False, dk_past=None,
                     dv_past=None, accumulate=False):
    """Gradients (dq, dk, dv, dk_past, dv_past); dk_past / dv_past float32,
    with respect to the rotated k_past and v_past. With accumulate=True the
    cached rows' gradients are added to the given dk_past / dv_past."""
    torch = _torch()
    T, Hq, Hkv, d = _check_attn(q, k, v, pos, subtree_end, o=o, lse=lse, dout=dout)
    _shape(k_past, "k_past", (None, Hkv, d))
    for name, t in (("dk_past", dk_past), ("dv_past", dv_past)):
        if t is not None:
            _shape(t, name, tuple(k_past.shape))
    dev = q.device
    kp, vp, vis, Lp = _past_args(q, k_past, v_past, past_visible)
    if workspace is None:
        if reuse_prep:
            raise ValueError("reuse_prep needs the forward's workspace")
        workspace = gw_workspace(T, Lp, Hq, Hkv, d, True, dev)
    if dk_past is None or dv_past is None:
        if accumulate:
            raise ValueError("accumulate needs dk_past and dv_past")
        dk_past = torch.empty(Lp, Hkv, d, dtype=torch.float32, device=dev)
        dv_past = torch.empty(Lp, Hkv, d, dtype=torch.float32, device=dev)
    _shape(dk_past, "dk_past", (Lp, Hkv, d))
    _shape(dv_past, "dv_past", (Lp, Hkv, d))
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    flags = (TA_REUSE_PREP if reuse_prep else 0) | (TA_ACCUMULATE_PAST if accumulate else 0)
    rc = _lib.tree_attn_gw_bwd(_dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype, dev), _dev_ptr(v, "v", q.dtype, dev),
                               _dev_ptr(o, "o", q.dtype, dev), _dev_ptr(lse, "lse", torch.float32, dev),
                               _dev_ptr(dout, "dout", q.dtype, dev), _dt(q), T, Hq, Hkv, d,
                               _dev_ptr(pos, "pos", torch.int32, dev),
                               _dev_ptr(subtree_end, "subtree_end", torch.int32, dev), int(pos_offset), kp, vp, vis,
                               Lp, float(softmax_scale), float(rope_theta), flags, _dev_ptr(dq, "dq"),
                               _dev_ptr(dk, "dk"), _dev_ptr(dv, "dv"),
                               _dev_ptr(dk_past, "dk_past", torch.float32, dev) if Lp else None,
                               _dev_ptr(dv_past, "dv_past", torch.float32, dev) if Lp else None,
                               _dev_ptr(workspace, "workspace"), workspace.numel(), _stream(dev))
    _check(rc)
    return dq, dk, dv, dk_past, dv_past


def _check_logprob(logits, src_row, target, weight, *per_entry):
    if logits.dim() != 2:
        raise ValueError(f"logits must be [R, V] (got {tuple(logits.shape)})")
    M = src_row.numel()
    _shape(src_row, "src_row", (M,))
    _shape(target, "target", (M,))
    _shape(weight, "weight", (M,))
    for name, t in per_entry:
        if t is not None:
            _shape(t, name, (M,))
    return logits.shape


def tree_attn_gw_export(k, v, pos, rows, pos_offset=0, rope_theta=10000.0, k_past=None, v_past=None):
    """Cached gateway rows from one partition's own tokens: k_past[r] = k of
    rows[r] rotated at pos_offset + pos[rows[r]], v_past[r] = its v. k, v
    [T, Hkv, d]; pos [T] int32; rows [n] int32 (device). Writes into the given
    k_past / v_past (e.g. a slice of a larger gateway) or new tensors.
    Returns (k_past, v_past)."""
    torch = _torch()
    if k.dim() != 3:
        raise ValueError(f"k must be [T, Hkv, d] (got {tuple(k.shape)})")
    T, Hkv, d = k.shape
    _shape(v, "v", (T, Hkv, d))
    _shape(pos, "pos", (T,))
    n = rows.numel()
    _shape(rows, "rows", (n,))
    if k_past is None:
        k_past = torch.empty(n, Hkv, d, dtype=k.dtype, device=k.device)
    if v_past is None:
        v_past = torch.empty(n, Hkv, d, dtype=k.dtype, device=k.device)
    _shape(k_past, "k_past", (n, Hkv, d))
    _shape(v_past, "v_past", (n, Hkv, d))
    dev = k.device
    _check(_lib.tree_attn_gw_export(_dev_ptr(k, "k"), _dev_ptr(v, "v", k.dtype, dev), _dt(k), T, Hkv, d,
                                    _dev_ptr(pos, "pos", torch.int32, dev), int(pos_offset), float(rope_theta),
                                    _dev_ptr(rows, "rows", torch.int32, dev), n,
                                    _dev_ptr(k_past, "k_past", k.dtype, dev), _dev_ptr(v_past, "v_past", k.dtype, dev),
                                    _stream(dev)))
    return k_past, v_past


def tree_attn_gw_relay(dk_past, dv_past, rows, pos, dk, dv, pos_offset=0, rope_theta=10000.0):
    """Adds the float32 gradients of cached rows back into one partition's
    dk / dv [T, Hkv, d] (in place): dk[rows[r]] += R^T dk_past[r],
    dv[rows[r]] += dv_past[r], rotated at pos_offset + pos[rows[r]]."""
    torch = _torch()
    if dk.dim() != 3:
        raise ValueError(f"dk must be [T, Hkv, d] (got {tuple(dk.shape)})")
    T, Hkv, d = dk.shape
    _shape(dv, "dv", (T, Hkv, d))
    _shape(pos, "pos", (T,))
    n = rows.numel()
    _shape(rows, "rows", (n,))
    _shape(dk_past, "dk_past", (n, Hkv, d))
    _shape(dv_past, "dv_past", (n, Hkv, d))
    dev = dk.device
    _check(_lib.tree_attn_gw_relay(_dev_ptr(dk_past, "dk_past", torch.float32, dev),
                                   _dev_ptr(dv_past, "dv_past", torch.float32, dev),
                                   _dev_ptr(rows, "rows", torch.int32, dev), n, _dt(dk), T, Hkv, d,
                                   _dev_ptr(pos, "pos", torch.int32, dev), int(pos_offset), float(rope_theta),
                                   _dev_ptr(dk, "dk"), _dev_ptr(dv, "dv", dk.dtype, dev), _stream(dev)))


def tree_logprob(logits, src_row, target, weight, grad_scale=1.0, with_grad=True, with_row_lse=True,
                 workspace=None):
    """Returns (logp [M] f32, row_lse [R] f32 or None, loss [] f32, dlogits [R,V] or None)."""
    torch = _torch()
    R, V = _check_logprob(logits, src_row, target, weight)
    M = src_row.numel()
    dev = logits.device
    if workspace is None:
        nbytes = _lib.tree_logprob_workspace_bytes(R, M)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    logp = torch.empty(max(M, 1), dtype=torch.float32, device=dev)
    row_lse = torch.empty(R, dtype=torch.float32, device=dev) if with_row_lse else None
    loss = torch.empty((), dtype=torch.float32, device=dev)
    dlogits = torch.empty_like(logits) if with_grad else None
    null = ctypes.c_void_p(None)
    rc = _lib.tree_logprob(_dev_ptr(logits, "logits"), _dt(logits), R, V,
                           _dev_ptr(src_row, "src_row", torch.int32, dev) if M else null,
                           _dev_ptr(target, "target", torch.int32, dev) if M else null,
                           _dev_ptr(weight, "weight", torch.float32, dev) if M else null, M,
                           _dev_ptr(logp, "logp"), _dev_ptr(row_lse, "row_lse") if with_row_lse else null,
                           _dev_ptr(loss, "loss"), _dev_ptr(dlogits, "dlogits") if with_grad else null,
                           float(grad_scale), _dev_ptr(workspace, "workspace"), workspace.numel(), _stream(dev))
    _check(rc)
    return logp[:M], row_lse, loss, dlogits


def tree_logprob_ppo(logits, src_row, target, weight, advantage, old_logp, mask=None, eps_low=0.2, eps_high=0.2,
                     grad_scale=1.0, with_grad=True, with_row_lse=True, workspace=None):
    """Clipped policy loss per occurrence. Returns (logp [M] f32, row_lse [R] f32 or None, loss [] f32,
    dlogits [R,V] or None)."""
    torch = _torch()
    R, V = _check_logprob(logits, src_row, target, weight, ("advantage", advantage), ("old_logp", old_logp),
                          ("mask", mask))
    M = src_row.numel()
    dev = logits.device
    if workspace is None:
        nbytes = _lib.tree_logprob_workspace_bytes(R, M)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    logp = torch.empty(max(M, 1), dtype=torch.float32, device=dev)
    row_lse = torch.empty(R, dtype=torch.float32, device=dev) if with_row_lse else None
    loss = torch.empty((), dtype=torch.float32, device=dev)
    dlogits = torch.empty_like(logits) if with_grad else None
    null = ctypes.c_void_p(None)
    rc = _lib.tree_logprob_ppo(_dev_ptr(logits, "logits"), _dt(logits), R, V,
                               _dev_ptr(src_row, "src_row", torch.int32, dev) if M else null,
                               _dev_ptr(target, "target", torch.int32, dev) if M else null,
                               _dev_ptr(weight, "weight", torch.float32, dev) if M else null,
                               _dev_ptr(advantage, "advantage", torch.float32, dev) if M else null,
                               _dev_ptr(old_logp, "old_logp", torch.float32, dev) if M else null,
                               _dev_ptr(mask, "mask", torch.uint8, dev) if (M and mask is not None) else null, M,
                               float(eps_low), float(eps_high),
                               _dev_ptr(logp, "logp"), _dev_ptr(row_lse, "row_lse") if with_row_lse else null,
                               _dev_ptr(loss, "loss"), _dev_ptr(dlogits, "dlogits") if with_grad else null,
                               float(grad_scale), _dev_ptr(workspace, "workspace"), workspace.numel(), _stream(dev))
    _check(rc)
    return logp[:M], row_lse, loss, dlogits


def tree_partition(node_start, node_end, node_parent, capacity):
    """Host partition plan: dict(node_part [n], part_tokens [P], part_parent [P], part_cut [P]) as int32 arrays."""
    ns = np.ascontiguousarray(node_start, dtype=np.int32)
    ne = np.ascontiguousarray(node_end, dtype=np.int32)
    npar = np.ascontiguousarray(node_parent, dtype=np.int32)
    n = len(ns)
    node_part = np.zeros(n, np.int32)
    part_tokens = np.zeros(n, np.int32)
    part_parent = np.zeros(n, np.int32)
    part_cut = np.zeros(n, np.int32)
    n_parts = ctypes.c_int32(0)
    _check(_lib.tree_partition(_np_ptr(ns), _np_ptr(ne), _np_ptr(npar), n, int(capacity), _np_ptr(node_part),
                               _np_ptr(part_tokens), _np_ptr(part_parent), _np_ptr(part_cut), ctypes.byref(n_parts)))
    P = n_parts.value
    return {"node_part": node_part, "part_tokens": part_tokens[:P].copy(), "part_parent": part_parent[:P].copy(),
            "part_cut": part_cut[:P].copy()}


def _check_conv(x, weight, bias, parent, pos=None, subtree_end=None, dy=None):
    if x.dim() != 2 or weight.dim() != 2:
        raise ValueError(f"x must be [T, C] and weight [C, K] (got {tuple(x.shape)}, {tuple(weight.shape)})")
    T, C = x.shape
    K = weight.shape[1]
    _shape(weight, "weight", (C, K))
    if bias is not None:
        _shape(bias, "bias", (C,))
    _shape(parent, "parent", (T,))
    for name, t in (("pos", pos), ("subtree_end", subtree_end)):
        if t is not None:
            _shape(t, name, (T,))
    if dy is not None:
        _shape(dy, "dy", (T, C))
    return T, C, K


def tree_conv_fwd(x, weight, bias, parent, activation=1):
    """x [T, C] (bf16 / f32), weight [C, K] f32, bias [C] f32 or None, parent [T] int32 -> y [T, C]."""
    torch = _torch()
    T, C, K = _check_conv(x, weight, bias, parent)
    dev = x.device
    y = torch.empty_like(x)
    rc = _lib.tree_conv_fwd(_dev_ptr(x, "x"), _dt(x), T, C, K, _dev_ptr(weight, "weight", torch.float32, dev),
                            _dev_ptr(bias, "bias", torch.float32, dev) if bias is not None else None,
                            _dev_ptr(parent, "parent", torch.int32, dev), int(activation), _dev_ptr(y, "y"),
                            _stream(dev))
    _check(rc)
    return y


def tree_conv_bwd(x, dy, weight, bias, parent, pos, subtree_end, activation=1, workspace=None):
    """Returns (dx [T, C] like x, dweight [C, K] f32, dbias [C] f32 or None)."""
    torch = _torch()
    T, C, K = _check_conv(x, weight, bias, parent, pos=pos, subtree_end=subtree_end, dy=dy)
    dev = x.device
    if workspace is None:
        workspace = torch.empty(max(_lib.tree_conv_workspace_bytes(T, C, K), 256), dtype=torch.uint8, device=dev)
    dx = torch.empty_like(x)
    dw = torch.empty_like(weight)
    db = torch.empty(C, dtype=torch.float32, device=dev) if bias is not None else None
    rc = _lib.tree_conv_bwd(_dev_ptr(x, "x"), _dev_ptr(dy, "dy", x.dtype, dev), _dt(x), T, C, K,
                            _dev_ptr(weight, "weight", torch.float32, dev),
                            _dev_ptr(bias, "bias", torch.float32, dev) if bias is not None else None,
                            _dev_ptr(parent, "parent", torch.int32, dev), _dev_ptr(pos, "pos", torch.int32, dev),
                            _dev_ptr(subtree_end, "subtree_end", torch.int32, dev), int(activation),
                            _dev_ptr(dx, "dx"), _dev_ptr(dw, "dweight"), _dev_ptr(db, "dbias") if db is not None else None,
                            _dev_ptr(workspace, "workspace"), workspace.numel(), _stream(dev))
    _check(rc)
    return dx, dw, db


def tree_gdn_plan(node_start, node_end, node_parent, chunk=64):
    """Host chunk schedule (int32 numpy array) for tree_gdn_fwd."""
    ns = np.ascontiguousarray(node_start, dtype=np.int32)
    ne = np.ascontiguousarray(node_end, dtype=np.int32)
    npar = np.ascontiguousarray(node_parent, dtype=np.int32)
    sz = GdnPlanSizes()
    rc = _lib.tree_gdn_plan(_np_ptr(ns), _np_ptr(ne), _np_ptr(npar), len(ns), int(chunk), None, 0, ctypes.byref(sz))
    if rc != TA_ECAPACITY:
        _check(rc)
    plan = np.zeros(sz.plan_ints, dtype=np.int32)
    _check(_lib.tree_gdn_plan(_np_ptr(ns), _np_ptr(ne), _np_ptr(npar), len(ns), int(chunk), _np_ptr(plan), len(plan),
                              ctypes.byref(sz)))
    return plan


def gdn_workspace(q, v, plan, backward=False):
    """Device workspace for tree_gdn_fwd; with backward=True also large
    enough for tree_gdn_bwd (pass the same buffer to both)."""
    torch = _torch()
    H, dk = q.shape[1], q.shape[2]
    Hv, dv = v.shape[1], v.shape[2]
    if backward:
        nbytes = _lib.tree_gdn_bwd_workspace_bytes(H, Hv, dk, dv, int(plan[0]), int(plan[1]))
    else:
        nbytes = _lib.tree_gdn_workspace_bytes(H, Hv, dk, dv, int(plan[0]))
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)


def _check_gdn(q, k, v, g, beta, do=None):
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError(f"q must be [T, H, dk] and v [T, Hv, dv] (got {tuple(q.shape)}, {tuple(v.shape)})")
    T, H, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    _shape(k, "k", (T, H, dk))
    _shape(v, "v", (T, Hv, dv))
    _shape(g, "g", (T, Hv))
    _shape(beta, "beta", (T, Hv))
    if do is not None:
        _shape(do, "do", (T, Hv, dv))
    return T, H, dk, Hv, dv


def tree_gdn_fwd(q, k, v, g, beta, plan, plan_dev=None, workspace=None):
    """q, k [T, H, dk]; v [T, Hv, dv] (bf16 / f32); g, beta [T, Hv] f32; plan from tree_gdn_plan -> o [T, Hv, dv]."""
    torch = _torch()
    T, H, dk, Hv, dv = _check_gdn(q, k, v, g, beta)
    dev = q.device
    plan = np.ascontiguousarray(plan, dtype=np.int32)
    if plan_dev is None:
        plan_dev = torch.from_numpy(plan).to(dev)
    if workspace is None:
        nbytes = _lib.tree_gdn_workspace_bytes(H, Hv, dk, dv, int(plan[0]))
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    o = torch.empty_like(v)
    rc = _lib.tree_gdn_fwd(_dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype, dev), _dev_ptr(v, "v", q.dtype, dev), _dt(q),
                           _dev_ptr(g, "g", torch.float32, dev), _dev_ptr(beta, "beta", torch.float32, dev), T, H, Hv,
                           dk, dv, _dev_ptr(plan_dev, "plan", torch.int32, dev), _np_ptr(plan), _dev_ptr(o, "o"),
                           _dev_ptr(workspace, "workspace"), workspace.numel(), _stream(dev))
    _check(rc)
    return o


def tree_gdn_bwd(q, k, v, g, beta, do, plan, workspace, plan_dev=None):
    """Gradients of sum(do * o) for the tree_gdn_fwd call that filled
    `workspace` (from gdn_workspace(..., backward=True)) with the same inputs
    and plan -> (dq, dk, dv, dg, dbeta)."""
    torch = _torch()
    T, H, dk, Hv, dv = _check_gdn(q, k, v, g, beta, do=do)
    dev = q.device
    plan = np.ascontiguousarray(plan, dtype=np.int32)
    if plan_dev is None:
        plan_dev = torch.from_numpy(plan).to(dev)
    dq, dk_, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty((T, Hv), dtype=torch.float32, device=dev)
    dbeta = torch.empty((T, Hv), dtype=torch.float32, device=dev)
    rc = _lib.tree_gdn_bwd(_dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype, dev), _dev_ptr(v, "v", q.dtype, dev), _dt(q),
                           _dev_ptr(g, "g", torch.float32, dev), _dev_ptr(beta, "beta", torch.float32, dev),
                           _dev_ptr(do, "do", q.dtype, dev), T, H, Hv, dk, dv,
                           _dev_ptr(plan_dev, "plan", torch.int32, dev), _np_ptr(plan), _dev_ptr(dq, "dq"),
                           _dev_ptr(dk_, "dk"), _dev_ptr(dv_, "dv"), _dev_ptr(dg, "dg"), _dev_ptr(dbeta, "dbeta"),
                           _dev_ptr(workspace, "workspace"), workspace.numel(), _stream(dev))
    _check(rc)
    return dq, dk_, dv_, dg, dbeta


def _make_autograd():
    torch = _torch()

    class _TreeAttention(torch.autograd.Function):
        """o = TreeAttention.apply(q, k, v, pos, subtree_end, scale, theta)."""

        @staticmethod
        def forward(ctx, q, k, v, pos, subtree_end, softmax_scale=0.0, rope_theta=10000.0):
            o, lse, ws = tree_attn_fwd(q, k, v, pos, subtree_end, softmax_scale, rope_theta,
                                       with_bwd_workspace=True)
            ctx.save_for_backward(q, k, v, o, lse, pos, subtree_end)
            ctx.ws = ws
            ctx.cfg = (softmax_scale, rope_theta)
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse, pos, se = ctx.saved_tensors
            dq, dk, dv = tree_attn_bwd(q, k, v, o, lse, do.contiguous(), pos, se, *ctx.cfg, workspace=ctx.ws,
                                       reuse_prep=True)
            ctx.ws = None
            return dq, dk, dv, None, None, None, None

    return _TreeAttention


TreeAttention = _make_autograd()
