"""Metadata guards of the attention kernels, checked on the host.

The kernels read subtree_end on the device only, so a malformed value cannot
be rejected before launch. The RoPE prep clamps every own row's subtree end
into (i, T] (and flags it); the tile bounds the dK/dV pass derives from it
must then stay inside the padded workspace rows. This is a replica of that
index arithmetic (the clamp, the per-128-key-tile maximum, the first and
last 64-row query block a key tile loads), run over malformed inputs,
including the cached-row layout of a child partition. It checks arithmetic
only; no kernel is launched.
"""
import numpy as np


def _layout(T, Lp):
    Lq = -(-Lp // 128) * 128
    Tc = Lq + T
    Tp = -(-Tc // 256) * 256
    return Lq, Tc, Tp


def _combined_se(se_raw, T, Lp, vis):
    """Subtree ends of the combined sequence as the prep writes them."""
    Lq, Tc, Tp = _layout(T, Lp)
    sep = np.zeros(Tp, np.int64)
    flagged = False
    for t in range(Tc):
        if t >= Lq:
            i = t - Lq
            c = min(max(int(se_raw[i]), i + 1), T)
            flagged |= c != int(se_raw[i])
            sep[t] = c + Lq
        elif t < Lp:
            sep[t] = Tc if vis[t] else t
        else:
            sep[t] = t
    return sep, flagged


def _dkdv_rows(sep, Tc, Lq):
    """Query rows [lo, hi) each 128-key tile's dK/dV loop loads."""
    out = []
    for kt in range(-(-Tc // 128)):
        j0 = kt * 128
        mmy = int(sep[j0:j0 + 128].max())
        qb_lo = max(j0, Lq) // 64
        nqb = max(-(-mmy // 64) - qb_lo, 0)
        out.append((qb_lo * 64, (qb_lo + nqb) * 64))
    return out


def test_clamped_tile_bounds_stay_inside_the_workspace():
    rng = np.random.default_rng(0)
    cases = 0
    for T in (1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000):
        for Lp in (0, 1, 127, 128, 300):
            for kind in ("valid", "huge", "negative", "self", "random"):
                i = np.arange(T)
                if kind == "valid":
                    se = np.full(T, T)
                elif kind == "huge":
                    se = np.full(T, 2 ** 31 - 1)
                elif kind == "negative":
                    se = np.full(T, -(2 ** 31))
                elif kind == "self":
                    se = i.copy()
                else:
                    se = rng.integers(-5 * T, 5 * T + 3, T)
                vis = rng.integers(0, 2, Lp)
                Lq, Tc, Tp = _layout(T, Lp)
                sep, flagged = _combined_se(se, T, Lp, vis)
                assert flagged == (kind not in ("valid",)) or kind == "random"
                own = sep[Lq:Tc] - Lq
                assert np.all(own >= i + 1) and np.all(own <= T)
                for lo, hi in _dkdv_rows(sep, Tc, Lq):
                    assert 0 <= lo and hi <= Tp
                # every own row sees at least its own key
                assert all(sep[t] > t for t in range(Lq, Tc))
                cases += 1
    assert cases == 12 * 5 * 5


def test_valid_metadata_is_left_unchanged():
    import workloads
    from oracle import pack as OP

    p = OP.pack(*workloads.sequences("short"))
    sep, flagged = _combined_se(p["se"], p["T"], 0, [])
    assert not flagged and np.array_equal(sep[:p["T"]], p["se"])
