"""Pins of the FP64 oracle against facts that do not come from the oracle.

Each test fixes a property that the pages or the mathematics determine:
the chunk form of the per-chunk operation table equals the token recurrence;
closed forms at special inputs (beta = 0, beta -> 0, beta = 1 with orthogonal
keys, a single write followed by per-channel decay, a single token); central
finite differences for all seven inputs; packing, causality, linearity and
the invariances of the L2 normalisation and of the gate map.
"""
import numpy as np
import pytest

import oracle
from oracle import chunked_ref

L_BOUND = -5.0
EPS = 1e-6


def rand_problem(seed, seqlens, H, K, V, a_scale=0.5, b_scale=0.5):
    rng = np.random.default_rng(seed)
    T = int(sum(seqlens))
    p = dict(
        q=rng.standard_normal((T, H, K)), k=rng.standard_normal((T, H, K)),
        v=rng.standard_normal((T, H, V)), raw_g=rng.standard_normal((T, H, K)),
        raw_beta=rng.standard_normal((T, H)),
        A_log=rng.standard_normal(H) * a_scale, dt_bias=rng.standard_normal((H, K)) * b_scale,
        cu_seqlens=np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64),
    )
    dO = rng.standard_normal((T, H, V))
    return p, dO


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def loss(p, dO, **kw):
    return float(np.sum(oracle.kda(**p, **kw)["o"] * dO))


# ---------------------------------------------------------------- P1: chunk form


@pytest.mark.parametrize("chunk", [1, 5, 16, 64])
def test_chunk_form_equals_recurrence_forward(chunk):
    p, _ = rand_problem(1, [1, 17, 23, 64], 2, 6, 5)
    ref = oracle.kda(**p)["o"]
    got = chunked_ref.chunk_fwd(**p, chunk=chunk)
    assert rel(got, ref) < 1e-12


@pytest.mark.parametrize("chunk", [1, 7, 16])
def test_chunk_adjoint_equals_token_adjoint(chunk):
    p, dO = rand_problem(2, [9, 20, 1], 2, 5, 4)
    ref = oracle.kda(**p, dO=dO)
    got = chunked_ref.chunk_bwd(**p, dO=dO, chunk=chunk)
    for name in ("dq", "dk", "dv", "draw_g", "draw_beta", "dA_log", "ddt_bias"):
        assert rel(got[name], ref[name]) < 1e-11, name


def test_chunk_form_slow_decay_long_sequence():
    # dt_bias = -8 gives g ~ -2e-3: long memory, many chunks carry state.
    p, dO = rand_problem(3, [150], 1, 8, 8)
    p["A_log"][:] = 0.0
    p["dt_bias"][:] = -8.0
    ref = oracle.kda(**p, dO=dO)
    assert rel(chunked_ref.chunk_fwd(**p, chunk=16), ref["o"]) < 1e-12
    got = chunked_ref.chunk_bwd(**p, dO=dO, chunk=16)
    for name in ("dq", "dk", "dv", "draw_g", "draw_beta", "dA_log", "ddt_bias"):
        assert rel(got[name], ref[name]) < 1e-11, name


# ---------------------------------------------------------------- P2/P3: beta -> 0


def _prologue_np(p, scale=1.0):
    """Prologue restated from the input description (L2 norm, sigmoid, gate map)."""
    qh = scale * p["q"] / np.sqrt(np.sum(p["q"] ** 2, -1, keepdims=True) + EPS)
    kh = p["k"] / np.sqrt(np.sum(p["k"] ** 2, -1, keepdims=True) + EPS)
    z = np.exp(p["A_log"])[None, :, None] * (p["raw_g"] + p["dt_bias"][None])
    with np.errstate(over="ignore"):
        g = L_BOUND / (1 + np.exp(-z))
    return qh, kh, g


def test_beta_zero_gives_zero_output_and_gradients():
    p, dO = rand_problem(4, [11, 6], 2, 5, 4)
    p["raw_beta"][:] = -1e4  # sigmoid is exactly 0 in double
    r = oracle.kda(**p, dO=dO)
    assert np.all(r["o"] == 0)
    for name in ("dq", "dk", "dv", "draw_g", "draw_beta", "dA_log", "ddt_bias"):
        assert np.all(r[name] == 0), name


def test_beta_gradient_at_zero_is_gated_linear_attention_form():
    # At beta -> 0 the state is sum_s beta_s Diag(e^{G_t-G_s}) k_s v_s^T to first
    # order, so dL/dbeta_t = sum_{r>=t} (qh_r . e^{G_r-G_t} kh_t)(v_t . dO_r).
    p, dO = rand_problem(5, [13], 2, 5, 4)
    p["raw_beta"][:] = -25.0  # beta ~ 1.4e-11
    r = oracle.kda(**p, dO=dO)
    beta = 1 / (1 + np.exp(25.0))
    dbeta = r["draw_beta"] / (beta * (1 - beta))
    qh, kh, g = _prologue_np(p)
    T, H = p["raw_beta"].shape
    for h in range(H):
        G = np.cumsum(g[:, h], axis=0)
        for t in range(T):
            want = sum((qh[rr, h] * np.exp(G[rr] - G[t]) * kh[t, h]).sum()
                       * (p["v"][t, h] @ dO[rr, h]) for rr in range(t, T))
            assert abs(dbeta[t, h] - want) <= 1e-8 * (abs(want) + 1e-3)


def test_small_beta_no_decay_is_linear_attention():
    p, _ = rand_problem(6, [24], 2, 6, 5)
    eps_b = 1e-7
    p["raw_beta"][:] = np.log(eps_b / (1 - eps_b))
    p["raw_g"][:] = -1e4
    p["A_log"][:] = 0
    p["dt_bias"][:] = 0
    o = oracle.kda(**p)["o"]
    qh, kh, _ = _prologue_np(p)
    lin = np.zeros_like(o)
    for t in range(o.shape[0]):
        for s in range(t + 1):
            lin[t] += np.sum(qh[t] * kh[s], -1)[:, None] * p["v"][s]
    assert rel(o / eps_b, lin) < 1e-5


# ---------------------------------------------------------------- P4/P5: exact closed forms


@pytest.mark.parametrize("raw_gate,gval", [(-1e4, 0.0), (40.0, L_BOUND)])
def test_orthogonal_keys_beta_one_closed_form(raw_gate, gval):
    T, K, V = 8, 8, 5
    p, _ = rand_problem(7, [T], 1, K, V)
    p["k"][:] = 0
    for t in range(T):
        p["k"][t, 0, t] = 1.0 + t  # orthogonal keys, any positive length
    p["raw_beta"][:] = 40.0  # beta = 1 exactly in double
    p["raw_g"][:] = raw_gate
    p["A_log"][:] = 0
    p["dt_bias"][:] = 0
    o = oracle.kda(**p)["o"]
    qh, kh, _ = _prologue_np(p)
    for t in range(T):
        want = sum(np.exp(gval * (t - s)) * (qh[t, 0] @ kh[s, 0]) * p["v"][s, 0]
                   for s in range(t + 1))
        assert np.allclose(o[t, 0], want, rtol=1e-12, atol=0)


@pytest.mark.parametrize("decay_all", [False, True])
def test_single_write_then_per_channel_decay(decay_all):
    T, K, V = 64, 8, 3
    p, _ = rand_problem(8, [T], 1, K, V)
    p["raw_beta"][:] = -1e4
    p["raw_beta"][0] = 40.0
    p["q"][:] = p["k"][0]
    D = np.ones(K, bool) if decay_all else (np.arange(K) % 2 == 0)
    p["raw_g"][:] = np.where(D, 40.0, -1e4)[None, None, :]
    p["A_log"][:] = 0
    p["dt_bias"][:] = 0
    o = oracle.kda(**p)["o"]
    qh, kh, _ = _prologue_np(p)
    for t in range(T):
        want = np.sum(qh[t, 0] * kh[0, 0] * np.exp(-5.0 * t * D)) * p["v"][0, 0]
        assert np.allclose(o[t, 0], want, rtol=1e-12, atol=0), t


def test_single_token():
    p, dO = rand_problem(9, [1], 3, 6, 4)
    r = oracle.kda(**p, dO=dO)
    qh, kh, _ = _prologue_np(p)
    beta = 1 / (1 + np.exp(-p["raw_beta"]))
    for h in range(3):
        qk = qh[0, h] @ kh[0, h]
        vd = p["v"][0, h] @ dO[0, h]
        assert np.allclose(r["o"][0, h], beta[0, h] * qk * p["v"][0, h], rtol=1e-13)
        assert np.allclose(r["dv"][0, h], beta[0, h] * qk * dO[0, h], rtol=1e-13)
        assert np.isclose(r["draw_beta"][0, h], qk * vd * beta[0, h] * (1 - beta[0, h]), rtol=1e-12)
    # the decay acts on an empty state: no gate gradient at all
    assert np.all(r["draw_g"] == 0) and np.all(r["dA_log"] == 0) and np.all(r["ddt_bias"] == 0)


# ---------------------------------------------------------------- P7: finite differences


@pytest.mark.parametrize("gate_mode", [0, 1])
def test_finite_differences_all_seven_inputs(gate_mode):
    p, dO = rand_problem(10, [7, 13], 2, 4, 3)
    if gate_mode == 1:
        p["A_log"] = p["A_log"] * 0.2 - 1.0  # keep most gates off the clamp
    r = oracle.kda(**p, dO=dO, gate_mode=gate_mode)
    rng = np.random.default_rng(11)
    step = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("raw_g", "draw_g"),
                        ("raw_beta", "draw_beta"), ("A_log", "dA_log"), ("dt_bias", "ddt_bias")):
        x = p[name]
        g = r[gname]
        scale_g = np.sqrt(np.mean(g ** 2)) + 1e-12
        idx = [tuple(rng.integers(0, s) for s in x.shape) for _ in range(8)]
        for ix in idx:
            orig = x[ix]
            x[ix] = orig + step
            lp = loss(p, dO, gate_mode=gate_mode)
            x[ix] = orig - step
            lm = loss(p, dO, gate_mode=gate_mode)
            x[ix] = orig
            fd = (lp - lm) / (2 * step)
            assert abs(fd - g[ix]) <= 1e-6 * (abs(g[ix]) + scale_g), (name, ix, fd, g[ix])


# ---------------------------------------------------------------- P8/P9: structure


def test_packing_equals_separate_runs():
    seqlens = [5, 9, 3, 0, 12]
    p, dO = rand_problem(12, seqlens, 2, 5, 4)
    packed = oracle.kda(**p, dO=dO)
    cu = p["cu_seqlens"]
    dA = np.zeros(2)
    dtb = np.zeros((2, 5))
    for n in range(len(seqlens)):
        a, b = cu[n], cu[n + 1]
        sub = {k_: (v_[a:b] if k_ in ("q", "k", "v", "raw_g", "raw_beta") else v_)
               for k_, v_ in p.items() if k_ != "cu_seqlens"}
        one = oracle.kda(**sub, cu_seqlens=[0, b - a], dO=dO[a:b])
        for name in ("o", "dq", "dk", "dv", "draw_g", "draw_beta"):
            assert np.array_equal(one[name], packed[name][a:b]), name
        dA += one["dA_log"]
        dtb += one["ddt_bias"]
    assert np.allclose(packed["dA_log"], dA, rtol=1e-13, atol=1e-15)
    assert np.allclose(packed["ddt_bias"], dtb, rtol=1e-13, atol=1e-15)


def test_causality_and_sequence_isolation():
    p, _ = rand_problem(13, [10, 10], 2, 4, 4)
    o1 = oracle.kda(**p)["o"]
    for name in ("q", "k", "v", "raw_g", "raw_beta"):
        p2 = {k_: v_.copy() for k_, v_ in p.items()}
        p2[name][6:] += 1.0  # perturb tokens 6.. (inside sequence 0 and all of sequence 1)
        o2 = oracle.kda(**p2)["o"]
        assert np.array_equal(o1[:6], o2[:6]), name
    p3 = {k_: v_.copy() for k_, v_ in p.items()}
    p3["q"][10:] *= -2.0
    p3["v"][10:] += 3.0
    assert np.array_equal(oracle.kda(**p3)["o"][:10], o1[:10])


def test_linear_in_v_and_columns_independent():
    p, _ = rand_problem(14, [17], 2, 4, 6)
    o1 = oracle.kda(**p)["o"]
    rng = np.random.default_rng(15)
    v2 = rng.standard_normal(p["v"].shape)
    p2 = dict(p, v=v2)
    o2 = oracle.kda(**p2)["o"]
    p3 = dict(p, v=2.5 * p["v"] - 0.5 * v2)
    assert np.allclose(oracle.kda(**p3)["o"], 2.5 * o1 - 0.5 * o2, rtol=1e-12, atol=1e-12)
    p4 = dict(p, v=p["v"].copy())
    p4["v"][:, :, 3] += 1.0
    o4 = oracle.kda(**p4)["o"]
    keep = [0, 1, 2, 4, 5]
    assert np.array_equal(o4[:, :, keep], o1[:, :, keep])


# ---------------------------------------------------------------- P10/P11: invariances


def test_norm_scale_invariance_and_orthogonal_gradients():
    p, dO = rand_problem(16, [12], 2, 5, 4)
    r = oracle.kda(**p, dO=dO, eps=0.0)
    for c in (0.3, 7.0):
        pc = dict(p, q=c * p["q"], k=c * p["k"])
        assert rel(oracle.kda(**pc, eps=0.0)["o"], r["o"]) < 1e-13
    assert np.max(np.abs(np.sum(p["q"] * r["dq"], -1))) < 1e-12
    assert np.max(np.abs(np.sum(p["k"] * r["dk"], -1))) < 1e-12


def test_scale_argument_multiplies_output():
    p, _ = rand_problem(17, [9], 1, 4, 3)
    o1 = oracle.kda(**p)["o"]
    o2 = oracle.kda(**p, scale=0.125)["o"]
    assert np.allclose(o2, 0.125 * o1, rtol=1e-13, atol=1e-15)


def test_gate_parameter_gradients_follow_the_gate_map():
    # z = exp(A_log) (raw_g + dt_bias) implies, for every input:
    #   ddt_bias[h,k] = sum_t draw_g[t,h,k],  dA_log[h] = sum_{t,k} draw_g * (raw_g + dt_bias)
    p, dO = rand_problem(18, [8, 11], 3, 4, 3)
    r = oracle.kda(**p, dO=dO)
    assert np.allclose(r["ddt_bias"], r["draw_g"].sum(0), rtol=1e-12, atol=1e-14)
    want = np.sum(r["draw_g"] * (p["raw_g"] + p["dt_bias"][None]), axis=(0, 2))
    assert np.allclose(r["dA_log"], want, rtol=1e-12, atol=1e-14)


def test_long_sequence_crosses_oracle_checkpoint_blocks():
    # The reverse sweep recomputes blocks of 256 tokens from stored states;
    # a 600-token sequence (plus a short one) crosses two block boundaries.
    p, dO = rand_problem(19, [600, 3], 1, 3, 2)
    p["dt_bias"][:] = -6.0  # slow decay so early tokens still matter late
    ref = chunked_ref.chunk_bwd(**p, dO=dO, chunk=64)
    r = oracle.kda(**p, dO=dO)
    assert rel(r["o"], chunked_ref.chunk_fwd(**p, chunk=64)) < 1e-12
    for name in ("dq", "dk", "dv", "draw_g", "draw_beta", "dA_log", "ddt_bias"):
        assert rel(r[name], ref[name]) < 1e-11, name


def test_prologue_entry_matches_its_definition():
    # gcum restarts every chunk from each sequence start; qh,kh unit-norm
    # (up to eps) rows; beta in (0, 1); g in (L, 0) so gcum is decreasing.
    p, _ = rand_problem(20, [5, 40, 0, 17], 2, 6, 4)
    r = oracle.prologue(p["q"], p["k"], p["raw_g"], p["raw_beta"], p["A_log"], p["dt_bias"],
                        p["cu_seqlens"], chunk=16)
    qh, kh, g = _prologue_np(p)
    assert np.allclose(r["qh"], qh, rtol=1e-14) and np.allclose(r["kh"], kh, rtol=1e-14)
    assert np.allclose(r["beta"], 1 / (1 + np.exp(-p["raw_beta"])), rtol=1e-14)
    cu = p["cu_seqlens"]
    for n in range(len(cu) - 1):
        for t in range(cu[n], cu[n + 1]):
            c0 = cu[n] + (t - cu[n]) // 16 * 16
            assert np.allclose(r["gcum"][t], g[c0:t + 1].sum(0), rtol=1e-13, atol=1e-15)
    assert np.all(g < 0) and np.all(g > L_BOUND)
