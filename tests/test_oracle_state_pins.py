"""Pins of the oracle's state input and output (initial state h0, final state
ht, and the gradients dh0 of h0 given a loss term on ht through dht).

The measured operator has neither (the FROST page's configuration starts every
sequence from zero and returns no final state); these are the first extension
the recurrence admits. Each test fixes a property that holds for any correct
implementation: the chunk form started from h0 agrees with the token
recurrence; running a sequence in two parts, with the first part's final
state as the second part's initial state, equals one run (forward and
backward); beta = 0 leaves only the decay of h0, a closed form; and central
finite differences of sum(O * dO) + sum(ht * dht) match dh0 and the input
gradients.
"""
import numpy as np
import pytest

import oracle
from oracle import chunked_ref

L_BOUND = -5.0
EPS = 1e-6
GRADS = ("dq", "dk", "dv", "draw_g", "draw_beta")


def rand_problem(seed, seqlens, H, K, V):
    rng = np.random.default_rng(seed)
    T = int(sum(seqlens))
    N = len(seqlens)
    p = dict(
        q=rng.standard_normal((T, H, K)), k=rng.standard_normal((T, H, K)),
        v=rng.standard_normal((T, H, V)), raw_g=rng.standard_normal((T, H, K)),
        raw_beta=rng.standard_normal((T, H)),
        A_log=rng.standard_normal(H) * 0.5, dt_bias=rng.standard_normal((H, K)) * 0.5,
        cu_seqlens=np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64),
    )
    h0 = rng.standard_normal((N, H, K, V))
    dht = rng.standard_normal((N, H, K, V))
    dO = rng.standard_normal((T, H, V))
    return p, h0, dht, dO


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def part(p, a, b):
    """Tokens [a, b) of a one-sequence problem as a problem of its own."""
    sub = {k_: (v_[a:b] if k_ in ("q", "k", "v", "raw_g", "raw_beta") else v_)
           for k_, v_ in p.items() if k_ != "cu_seqlens"}
    sub["cu_seqlens"] = np.array([0, b - a], dtype=np.int64)
    return sub


@pytest.mark.parametrize("chunk", [1, 6, 16])
def test_chunk_form_from_initial_state_equals_recurrence(chunk):
    p, h0, _, _ = rand_problem(31, [13, 1, 0, 29], 2, 5, 4)
    ref = oracle.kda(**p, h0=h0)
    o, ht = chunked_ref.chunk_fwd(**p, chunk=chunk, h0=h0, return_state=True)
    assert rel(o, ref["o"]) < 1e-12
    assert rel(ht, ref["ht"]) < 1e-12
    # the empty third sequence passes its initial state through unchanged
    assert np.array_equal(ref["ht"][2], h0[2])


def test_final_state_without_initial_state_matches_chunk_form():
    p, _, _, _ = rand_problem(32, [21, 8], 2, 4, 6)
    ref = oracle.kda(**p, final_state=True)
    o, ht = chunked_ref.chunk_fwd(**p, chunk=5, return_state=True)
    assert rel(o, ref["o"]) < 1e-12
    assert rel(ht, ref["ht"]) < 1e-12


@pytest.mark.parametrize("cut", [1, 9, 22])
def test_two_part_run_equals_one_run(cut):
    p, h0, dht, dO = rand_problem(33, [23], 2, 5, 4)
    full = oracle.kda(**p, dO=dO, h0=h0, dht=dht)
    second_in = oracle.kda(**part(p, 0, cut), h0=h0)["ht"]
    second = oracle.kda(**part(p, cut, 23), dO=dO[cut:], h0=second_in, dht=dht)
    first = oracle.kda(**part(p, 0, cut), dO=dO[:cut], h0=h0, dht=second["dh0"])
    assert rel(np.concatenate([first["o"], second["o"]]), full["o"]) < 1e-12
    assert rel(second["ht"], full["ht"]) < 1e-12
    for name in GRADS:
        got = np.concatenate([first[name], second[name]])
        assert rel(got, full[name]) < 1e-11, name
    for name in ("dA_log", "ddt_bias"):
        assert rel(first[name] + second[name], full[name]) < 1e-11, name
    assert rel(first["dh0"], full["dh0"]) < 1e-11


def test_beta_zero_only_decays_the_initial_state():
    p, h0, dht, dO = rand_problem(34, [9, 14], 2, 5, 3)
    p["raw_beta"][:] = -1e4  # sigmoid is exactly 0 in double
    r = oracle.kda(**p, dO=dO, h0=h0, dht=dht)
    qh = p["q"] / np.sqrt(np.sum(p["q"] ** 2, -1, keepdims=True) + EPS)
    z = np.exp(p["A_log"])[None, :, None] * (p["raw_g"] + p["dt_bias"][None])
    g = L_BOUND / (1 + np.exp(-z))
    cu = p["cu_seqlens"]
    for n in range(2):
        a, b = cu[n], cu[n + 1]
        G = np.cumsum(g[a:b], axis=0)  # [L, H, K], inclusive
        for hh in range(2):
            S = np.exp(G[:, hh, :])[:, :, None] * h0[n, hh][None]  # S_t = Diag(e^G_t) h0
            o = np.einsum("tkv,tk->tv", S, qh[a:b, hh])
            assert rel(r["o"][a:b, hh], o) < 1e-12
            assert rel(r["ht"][n, hh], S[-1]) < 1e-12
            # dh0 = sum_t Diag(e^G_t) qh_t dO_t^T + Diag(e^G_last) dht
            dh0 = np.einsum("tk,tk,tv->kv", np.exp(G[:, hh, :]), qh[a:b, hh], dO[a:b, hh])
            dh0 += np.exp(G[-1, hh, :])[:, None] * dht[n, hh]
            assert rel(r["dh0"][n, hh], dh0) < 1e-12
    for name in ("dv", "draw_beta"):
        assert np.all(np.isfinite(r[name])), name


def test_finite_differences_with_state_terms():
    p, h0, dht, dO = rand_problem(35, [6, 11], 2, 4, 3)
    r = oracle.kda(**p, dO=dO, h0=h0, dht=dht)

    def loss():
        s = oracle.kda(**p, h0=h0)
        return float(np.sum(s["o"] * dO) + np.sum(s["ht"] * dht))

    rng = np.random.default_rng(36)
    step = 1e-6
    cases = [("h0", h0, r["dh0"])] + [(n_, p[n_], r[g_]) for n_, g_ in (
        ("q", "dq"), ("k", "dk"), ("v", "dv"), ("raw_g", "draw_g"), ("raw_beta", "draw_beta"),
        ("A_log", "dA_log"), ("dt_bias", "ddt_bias"))]
    for name, x, g in cases:
        scale_g = np.sqrt(np.mean(g ** 2)) + 1e-12
        for _ in range(6):
            ix = tuple(rng.integers(0, s) for s in x.shape)
            orig = x[ix]
            x[ix] = orig + step
            lp = loss()
            x[ix] = orig - step
            lm = loss()
            x[ix] = orig
            fd = (lp - lm) / (2 * step)
            assert abs(fd - g[ix]) <= 1e-6 * (abs(g[ix]) + scale_g), (name, ix, fd, g[ix])


def test_zero_initial_state_is_the_stateless_operator():
    p, h0, _, dO = rand_problem(37, [7, 12], 2, 4, 4)
    a = oracle.kda(**p, dO=dO)
    b = oracle.kda(**p, dO=dO, h0=np.zeros_like(h0), dht=np.zeros_like(h0))
    for name in ("o",) + GRADS + ("dA_log", "ddt_bias"):
        assert np.array_equal(a[name], b[name]), name
