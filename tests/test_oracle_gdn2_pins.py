"""Pins of the GDN-2 oracle (oracle/gdn2_oracle.c: a per-channel erase gate
b = sigmoid(raw_b) [K] and write gate w = sigmoid(raw_w) [V] in place of
KDA's scalar beta; "KDA at the production shape...", section 1.6 and the
per-chunk operation table of section 2.1).

- KDA is the special case b = w = beta in every channel (the same page): with
  raw_b and raw_w set to raw_beta broadcast over the channels the GDN-2
  oracle must reproduce the separately written KDA oracle (kda_oracle.c) in
  O and every shared gradient, and the KDA beta gradient must equal the sum
  of the b and w gradients over their channels (chain rule of a broadcast).
- Central finite differences of all eight inputs.
- Closed forms that isolate each new gate: a single write, read back later,
  scales every value column j by w_j; an erase of the same key removes the
  part b projects onto.
- Packing: a packed batch equals its sequences run one by one.
- Planted mistakes in a copy of gdn2_oracle.c are each caught.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn2_oracle.c")


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def problem(rng, seqlens, H, K, V, A_scale=0.5):
    T = sum(seqlens)
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    return dict(q=rng.standard_normal((T, H, K)), k=rng.standard_normal((T, H, K)),
                v=rng.standard_normal((T, H, V)), raw_g=rng.standard_normal((T, H, K)),
                raw_b=rng.standard_normal((T, H, K)), raw_w=rng.standard_normal((T, H, V)),
                A_log=rng.standard_normal(H) * A_scale,
                dt_bias=rng.standard_normal((H, K)) * A_scale, cu_seqlens=cu)


@pytest.mark.parametrize("gate_mode", [0, 1])
def test_reduces_to_kda_when_both_gates_are_beta(gate_mode):
    rng = np.random.default_rng(81)
    H, K, V = 3, 8, 6
    p = problem(rng, [19, 0, 33, 1], H, K, V)
    T = p["q"].shape[0]
    raw_beta = rng.standard_normal((T, H))
    p["raw_b"] = np.repeat(raw_beta[:, :, None], K, axis=2)
    p["raw_w"] = np.repeat(raw_beta[:, :, None], V, axis=2)
    dO = rng.standard_normal((T, H, V))
    g = oracle.gdn2(**p, dO=dO, gate_mode=gate_mode, scale=0.7)
    kw = {n: p[n] for n in ("q", "k", "v", "raw_g", "A_log", "dt_bias", "cu_seqlens")}
    r = oracle.kda(**kw, raw_beta=raw_beta, dO=dO, gate_mode=gate_mode, scale=0.7)
    assert rel(g["o"], r["o"]) < 1e-13
    for name in ("dq", "dk", "dv", "draw_g", "dA_log", "ddt_bias"):
        assert rel(g[name], r[name]) < 1e-12, name
    assert rel(g["draw_b"].sum(axis=2) + g["draw_w"].sum(axis=2), r["draw_beta"]) < 1e-12


def loss(p, dO, **kw):
    return float(np.sum(oracle.gdn2(**p, **kw)["o"] * dO))


@pytest.mark.parametrize("gate_mode", [0, 1])
def test_finite_differences_all_inputs(gate_mode):
    rng = np.random.default_rng(82 + gate_mode)
    H, K, V = 2, 4, 3
    p = problem(rng, [13, 9], H, K, V)
    if gate_mode == 1:
        p["raw_g"] = rng.standard_normal(p["raw_g"].shape) - 2.0  # mostly above the clamp
    dO = rng.standard_normal(p["v"].shape)
    g = oracle.gdn2(**p, dO=dO, gate_mode=gate_mode)
    step = 1e-6
    checked = 0
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("raw_g", "draw_g"),
                        ("raw_b", "draw_b"), ("raw_w", "draw_w"), ("A_log", "dA_log"),
                        ("dt_bias", "ddt_bias")):
        x = p[name]
        flat = x.reshape(-1)
        for ix in rng.choice(flat.size, size=min(6, flat.size), replace=False):
            x0 = flat[ix]
            flat[ix] = x0 + step
            lp = loss(p, dO, gate_mode=gate_mode)
            flat[ix] = x0 - step
            lm = loss(p, dO, gate_mode=gate_mode)
            flat[ix] = x0
            fd = (lp - lm) / (2 * step)
            an = g[gname].reshape(-1)[ix]
            assert abs(fd - an) <= 1e-6 * (abs(an) + 1e-2), (name, ix, fd, an)
            checked += 1
    assert checked == 6 * 6 + 2 + 6


def test_single_write_scales_each_value_column_by_its_write_gate():
    # token 0 writes kh0 (w0 * v0)^T into the empty state; later tokens neither
    # erase (b = 0) nor write (w = 0), so o_t[j] = w0_j v0_j sum_k qh_tk kh0_k
    # exp(G_tk - G_0k), with per-channel decay
    rng = np.random.default_rng(84)
    T, H, K, V = 9, 1, 5, 4
    p = problem(rng, [T], H, K, V, A_scale=0.0)
    p["raw_b"][1:] = -1e4
    p["raw_w"][1:] = -1e4
    o = oracle.gdn2(**p)["o"][:, 0]
    q, k = p["q"][:, 0], p["k"][:, 0]
    qh = q / np.sqrt((q * q).sum(1, keepdims=True) + 1e-6)
    kh = k / np.sqrt((k * k).sum(1, keepdims=True) + 1e-6)
    g = -5.0 / (1.0 + np.exp(-p["raw_g"][:, 0]))
    w0 = 1.0 / (1.0 + np.exp(-p["raw_w"][0, 0]))
    G = np.cumsum(g, axis=0)
    for t in range(T):
        s = np.sum(qh[t] * kh[0] * np.exp(G[t] - G[0]))
        np.testing.assert_allclose(o[t], w0 * p["v"][0, 0] * s, rtol=1e-13, atol=1e-300)


def test_erase_removes_what_the_erase_gate_projects():
    # token 0 writes kh v0^T (w = 1); token 1 reuses the key, writes nothing
    # (w = 0), does not decay (g = 0 exactly) and erases with b in {0, 1} per
    # channel: S_1 = kh v0^T (1 - sum_{k in E} kh_k^2), o_1 = S_1^T qh_1
    rng = np.random.default_rng(85)
    H, K, V = 1, 6, 3
    p = problem(rng, [2], H, K, V, A_scale=0.0)
    p["k"][1] = p["k"][0]
    p["raw_w"][0] = 1e4
    p["raw_w"][1] = -1e4
    p["raw_g"][:] = -1e4
    E = np.array([1, 0, 1, 1, 0, 0], dtype=bool)
    p["raw_b"][1, 0] = np.where(E, 1e4, -1e4)
    o1 = oracle.gdn2(**p)["o"][1, 0]
    k0, q1 = p["k"][0, 0], p["q"][1, 0]
    kh = k0 / np.sqrt(k0 @ k0 + 1e-6)
    qh = q1 / np.sqrt(q1 @ q1 + 1e-6)
    want = p["v"][0, 0] * (qh @ kh) * (1.0 - np.sum(kh[E] ** 2))
    np.testing.assert_allclose(o1, want, rtol=1e-12)
    # erasing every channel with the write gate of that key empties the state
    p["raw_b"][1, 0] = 1e4
    np.testing.assert_allclose(oracle.gdn2(**p)["o"][1, 0], 0.0, atol=1e-6 * np.abs(want).max())


def test_packing_equals_separate_runs():
    rng = np.random.default_rng(86)
    H, K, V = 2, 4, 5
    lens = [7, 0, 12]
    p = problem(rng, lens, H, K, V)
    dO = rng.standard_normal(p["v"].shape)
    r = oracle.gdn2(**p, dO=dO)
    cu = p["cu_seqlens"]
    dA = np.zeros(H)
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        s = {k_: (v_[a:b] if v_.ndim == 3 else v_) for k_, v_ in p.items() if k_ != "cu_seqlens"}
        part = oracle.gdn2(**s, dO=dO[a:b])
        for name in ("o", "dq", "dk", "dv", "draw_g", "draw_b", "draw_w"):
            np.testing.assert_allclose(r[name][a:b], part[name], rtol=1e-13, atol=1e-300)
        dA += part["dA_log"]
    np.testing.assert_allclose(r["dA_log"], dA, rtol=1e-12)


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "erase_without_gate": ("acc -= S[(size_t)i * V + j] * (x->b[i] * x->kh[i]);",
                           "acc -= S[(size_t)i * V + j] * x->kh[i];"),
    "write_without_gate": ("double acc = x->w[j] * vt[j];", "double acc = vt[j];"),
    "write_key_gated": ("for (int j = 0; j < V; ++j) S[(size_t)i * V + j] += x->kh[i] * u[j];",
                        "for (int j = 0; j < V; ++j) S[(size_t)i * V + j] += x->b[i] * x->kh[i] * u[j];"),
    "dw_without_v": ("drw[j] = du[j] * vt[j] * x.w[j] * (1.0 - x.w[j]);",
                     "drw[j] = du[j] * x.w[j] * (1.0 - x.w[j]);"),
    "db_without_key": ("db[i] = de * x.kh[i];", "db[i] = de;"),
    "dkh_missing_erase": ("dkh[i] += de * x.b[i];", ";"),
    "dSd_missing_erase": ("dSd[(size_t)i * V + j] = dS[(size_t)i * V + j] - e * du[j];",
                          "dSd[(size_t)i * V + j] = dS[(size_t)i * V + j];"),
    "dv_without_gate": ("dvt[j] = du[j] * x.w[j];", "dvt[j] = du[j];"),
}


def _battery(lib_path) -> bool:
    rng = np.random.default_rng(87)
    H, K, V = 2, 4, 3
    p = problem(rng, [6, 9], H, K, V)
    T = p["q"].shape[0]
    dO = rng.standard_normal((T, H, V))
    # the reduction to KDA
    raw_beta = rng.standard_normal((T, H))
    pk = dict(p, raw_b=np.repeat(raw_beta[:, :, None], K, 2), raw_w=np.repeat(raw_beta[:, :, None], V, 2))
    g = oracle.gdn2(**pk, dO=dO, lib_path=lib_path)
    kw = {n: p[n] for n in ("q", "k", "v", "raw_g", "A_log", "dt_bias", "cu_seqlens")}
    r = oracle.kda(**kw, raw_beta=raw_beta, dO=dO)
    if rel(g["o"], r["o"]) > 1e-12:
        return False
    for name in ("dq", "dk", "dv", "draw_g", "dA_log", "ddt_bias"):
        if rel(g[name], r[name]) > 1e-11:
            return False
    if rel(g["draw_b"].sum(2) + g["draw_w"].sum(2), r["draw_beta"]) > 1e-11:
        return False
    # finite differences on the first entry of every input, with distinct gates
    g = oracle.gdn2(**p, dO=dO, lib_path=lib_path)
    step = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("raw_g", "draw_g"),
                        ("raw_b", "draw_b"), ("raw_w", "draw_w"), ("A_log", "dA_log"),
                        ("dt_bias", "ddt_bias")):
        x = p[name]
        ix = tuple(0 for _ in x.shape)
        x0 = x[ix]
        x[ix] = x0 + step
        lp = np.sum(oracle.gdn2(**p, lib_path=lib_path)["o"] * dO)
        x[ix] = x0 - step
        lm = np.sum(oracle.gdn2(**p, lib_path=lib_path)["o"] * dO)
        x[ix] = x0
        if abs((lp - lm) / (2 * step) - g[gname][ix]) > 1e-6 * (abs(g[gname][ix]) + 1e-2):
            return False
    return True


def test_unmutated_gdn2_oracle_passes_the_battery():
    assert _battery(None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_gdn2_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must match exactly once"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-std=c11", "-o", lib, str(mpath), "-lm"],
                   check=True)
    assert not _battery(lib), "planted mistake %s went unnoticed" % name
