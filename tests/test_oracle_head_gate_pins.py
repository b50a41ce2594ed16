"""Pins of the oracle's scalar-gate form (one gate per head and token, the
Gated DeltaNet operator that FLA's chunk_gdn computes; "KDA at the production
shape...", sections 1.1 and 1.2) against facts that do not come from the
oracle: a closed form of the recurrence at orthogonal keys with gates that
switch between exactly 0 and exactly the bound, central finite differences
of every input, and the per-head gate's independence across heads.
"""
import numpy as np
import pytest

import oracle

L_BOUND = -5.0
EPS = 1e-6


def rand_problem(seed, seqlens, H, K, V):
    rng = np.random.default_rng(seed)
    T = int(sum(seqlens))
    p = dict(
        q=rng.standard_normal((T, H, K)), k=rng.standard_normal((T, H, K)),
        v=rng.standard_normal((T, H, V)), raw_g=rng.standard_normal((T, H)),
        raw_beta=rng.standard_normal((T, H)),
        A_log=rng.standard_normal(H) * 0.5, dt_bias=rng.standard_normal(H) * 0.5,
        cu_seqlens=np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64),
    )
    return p, rng.standard_normal((T, H, V))


def loss(p, dO, **kw):
    return float(np.sum(oracle.kda(**p, **kw)["o"] * dO))


@pytest.mark.parametrize("gate_mode", [0, 1])
def test_orthogonal_keys_switching_scalar_gates(gate_mode):
    # With orthogonal keys and beta = 1 every write lands in an empty row of
    # the state, so the delta rule's erase term never acts and
    #   o_t = sum_{s<=t} exp(sum_{s<u<=t} g_u) (qh_t . kh_s) v_s,
    # one scalar decay per head. A raw gate of -1e4 gives g = 0 and +40 gives
    # g = L exactly, under either gate map; the two heads get different
    # switching patterns.
    T, H, K, V = 8, 2, 8, 5
    p, _ = rand_problem(31, [T], H, K, V)
    p["k"][:] = 0
    for h in range(H):
        for t in range(T):
            p["k"][t, h, (t + 3 * h) % K] = 0.5 + t
    p["raw_beta"][:] = 40.0  # beta = 1 exactly in double
    on = np.random.default_rng(5).random((T, H)) < 0.5
    p["raw_g"] = np.where(on, 40.0, -1e4)
    p["A_log"][:] = 0
    p["dt_bias"][:] = 0
    o = oracle.kda(**p, gate_mode=gate_mode)["o"]
    g = np.where(on, L_BOUND, 0.0)
    qh = p["q"] / np.sqrt(np.sum(p["q"] ** 2, -1, keepdims=True) + EPS)
    kh = p["k"] / np.sqrt(np.sum(p["k"] ** 2, -1, keepdims=True) + EPS)
    for h in range(H):
        for t in range(T):
            want = sum(np.exp(g[s + 1:t + 1, h].sum()) * (qh[t, h] @ kh[s, h]) * p["v"][s, h]
                       for s in range(t + 1))
            assert np.allclose(o[t, h], want, rtol=1e-12, atol=1e-300), (h, t)


@pytest.mark.parametrize("gate_mode", [0, 1])
def test_scalar_gate_finite_differences(gate_mode):
    p, dO = rand_problem(12, [6, 11], 2, 4, 3)
    if gate_mode == 1:
        p["A_log"] = p["A_log"] * 0.2 - 1.0  # keep most gates off the clamp
    r = oracle.kda(**p, dO=dO, gate_mode=gate_mode)
    assert r["draw_g"].shape == p["raw_g"].shape and r["ddt_bias"].shape == p["dt_bias"].shape
    rng = np.random.default_rng(13)
    step = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("raw_g", "draw_g"),
                        ("raw_beta", "draw_beta"), ("A_log", "dA_log"), ("dt_bias", "ddt_bias")):
        x = p[name]
        g = r[gname]
        scale_g = np.sqrt(np.mean(g ** 2)) + 1e-12
        for _ in range(8):
            ix = tuple(rng.integers(0, s) for s in x.shape)
            orig = x[ix]
            x[ix] = orig + step
            lp = loss(p, dO, gate_mode=gate_mode)
            x[ix] = orig - step
            lm = loss(p, dO, gate_mode=gate_mode)
            x[ix] = orig
            fd = (lp - lm) / (2 * step)
            assert abs(fd - g[ix]) <= 1e-6 * (abs(g[ix]) + scale_g), (name, ix, fd, g[ix])


def test_scalar_gate_of_one_head_leaves_the_other_alone():
    p, dO = rand_problem(14, [9, 4], 2, 4, 4)
    a = oracle.kda(**p, dO=dO)
    p["raw_g"][:, 1] += 0.7
    p["dt_bias"][1] -= 0.3
    b = oracle.kda(**p, dO=dO)
    for name in ("o", "dq", "dk", "dv", "draw_g", "draw_beta"):
        assert np.array_equal(a[name][:, 0], b[name][:, 0]), name
        assert not np.allclose(a[name][:, 1], b[name][:, 1]), name
    assert a["dA_log"][0] == b["dA_log"][0] and a["ddt_bias"][0] == b["ddt_bias"][0]
