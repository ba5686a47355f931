"""The Python binding checks every tensor's shape against the sizes it passes
to the C ABI and raises ValueError before any device pointer is taken, so a
mismatched tensor can never make a kernel read or write past a buffer. CPU
tensors suffice: the shape check comes first."""
import pytest
import torch

import tree_packed_attention_amd as ta


def _attn(T=10, Hq=4, Hkv=2, d=16):
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    i = lambda *s: torch.zeros(*s, dtype=torch.int32)
    return dict(q=z(T, Hq, d), k=z(T, Hkv, d), v=z(T, Hkv, d), pos=i(T), se=i(T), o=z(T, Hq, d),
                lse=torch.zeros(Hq, T), do=z(T, Hq, d))


@pytest.mark.parametrize("bad,shape", [("k", (9, 2, 16)), ("v", (10, 2, 8)), ("v", (10, 1, 16)), ("pos", (11,)),
                                       ("se", (10, 1))])
def test_attention_forward_shapes(bad, shape):
    a = _attn()
    a[bad] = torch.zeros(*shape, dtype=a[bad].dtype)
    with pytest.raises(ValueError):
        ta.tree_attn_fwd(a["q"], a["k"], a["v"], a["pos"], a["se"])


@pytest.mark.parametrize("bad,shape", [("o", (10, 4, 8)), ("lse", (10, 4)), ("do", (10, 2, 16)), ("k", (10, 3, 16))])
def test_attention_backward_shapes(bad, shape):
    a = _attn()
    a[bad] = torch.zeros(*shape, dtype=a[bad].dtype)
    with pytest.raises(ValueError):
        ta.tree_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["pos"], a["se"])


def test_gateway_shapes():
    a = _attn()
    kp = torch.zeros(5, 2, 16, dtype=torch.bfloat16)
    vis = torch.ones(5, dtype=torch.uint8)
    with pytest.raises(ValueError):
        ta.tree_attn_gw_fwd(a["q"], a["k"], a["v"], a["pos"], a["se"], 3, kp, kp[:4], vis)
    with pytest.raises(ValueError):
        ta.tree_attn_gw_fwd(a["q"], a["k"], a["v"], a["pos"], a["se"], 3, kp, kp, vis[:4])
    with pytest.raises(ValueError):
        ta.tree_attn_gw_fwd(a["q"], a["k"], a["v"], a["pos"], a["se"], 3, kp[:, :1], kp[:, :1], vis)
    with pytest.raises(ValueError):
        ta.tree_attn_gw_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["pos"], a["se"], 3, kp, kp, vis,
                            dk_past=torch.zeros(4, 2, 16), dv_past=torch.zeros(5, 2, 16))


def test_logprob_shapes():
    z = torch.zeros(4, 32, dtype=torch.bfloat16)
    s, t, w = torch.zeros(6, dtype=torch.int32), torch.zeros(6, dtype=torch.int32), torch.zeros(6)
    with pytest.raises(ValueError):
        ta.tree_logprob(z, s, t[:5], w)
    with pytest.raises(ValueError):
        ta.tree_logprob(z, s, t, w[:5])
    with pytest.raises(ValueError):
        ta.tree_logprob(z.view(-1), s, t, w)
    with pytest.raises(ValueError):
        ta.tree_logprob_ppo(z, s, t, w, torch.zeros(6), torch.zeros(5))
    with pytest.raises(ValueError):
        ta.tree_logprob_ppo(z, s, t, w, torch.zeros(6), torch.zeros(6), torch.zeros(7, dtype=torch.uint8))


def test_conv_and_gdn_shapes():
    x = torch.zeros(10, 16, dtype=torch.bfloat16)
    w = torch.zeros(16, 4)
    par = torch.zeros(10, dtype=torch.int32)
    with pytest.raises(ValueError):
        ta.tree_conv_fwd(x, torch.zeros(8, 4), None, par)
    with pytest.raises(ValueError):
        ta.tree_conv_fwd(x, w, torch.zeros(15), par)
    with pytest.raises(ValueError):
        ta.tree_conv_fwd(x, w, None, par[:9])
    with pytest.raises(ValueError):
        ta.tree_conv_bwd(x, x[:9], w, None, par, par, par)
    q = torch.zeros(10, 2, 64, dtype=torch.bfloat16)
    v = torch.zeros(10, 4, 64, dtype=torch.bfloat16)
    g = torch.zeros(10, 4)
    with pytest.raises(ValueError):
        ta.tree_gdn_fwd(q, q[:, :1], v, g, g, plan=[0] * 8)
    with pytest.raises(ValueError):
        ta.tree_gdn_fwd(q, q, v, g[:, :3], g, plan=[0] * 8)
