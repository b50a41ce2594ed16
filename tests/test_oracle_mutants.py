"""Plant plausible mistakes in a copy of the oracle and check the pins catch each.

Every mutant is a textual edit of ``oracle/kda_oracle.c`` compiled into a
temporary library on the CPU; the pins then run against that library. A
mutant that no pin rejects would mean the pins leave that part of the oracle
unchecked.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import chunked_ref

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

MUTANTS = {
    "no_erase_term": ("u_out[j] -= S[(size_t)i * V + j] * w->kh[i];", ";"),
    "output_reads_key": ("o_out[j] += S[(size_t)i * V + j] * w->qh[i];",
                         "o_out[j] += S[(size_t)i * V + j] * w->kh[i];"),
    "write_without_beta": ("const double c = w->beta * w->kh[i];", "const double c = w->kh[i];"),
    "decay_missing": ("const double d = exp(w->g[i]);\n    for (int j = 0; j < V; ++j) S[(size_t)i * V + j] *= d;",
                      "const double d = 1.0 + 0 * exp(w->g[i]);\n    for (int j = 0; j < V; ++j) S[(size_t)i * V + j] *= d;"),
    "norm_without_eps": ("w->rq = 1.0 / sqrt(sq + p->eps);", "w->rq = 1.0 / sqrt(sq);"),
    "gate_sign": ("w->g[i] = p->lower_bound * sigmoid(w->z[i]);",
                  "w->g[i] = -p->lower_bound * sigmoid(w->z[i]) - 5.0;"),
    "dg_sign": ("s.dg[i] = a;", "s.dg[i] = -a;"),
    "du_missing_beta": ("for (int j = 0; j < V; ++j) s.du[j] *= w.beta;", ";"),
    "dkh_missing_erase_path": ("s.dkh[i] -= a;", ";"),
    "dq_no_projection": ("dqt[i] = p->scale * w.rq * (s.dqh[i] - w.qbar[i] * qd);",
                         "dqt[i] = p->scale * w.rq * s.dqh[i];"),
    "dbeta_no_sigmoid_grad": ("p->draw_beta[th] = dbeta * w.beta * (1.0 - w.beta);",
                              "p->draw_beta[th] = dbeta * w.beta;"),
    "dA_log_wrong": ("dA = dz * w.z[i];", "dA = dz;"),
    "dS_not_decayed": ("s.dS[(size_t)i * V + j] = d * s.dSt[(size_t)i * V + j];",
                       "s.dS[(size_t)i * V + j] = s.dSt[(size_t)i * V + j];"),
    "dv_extra_factor": ("for (int j = 0; j < V; ++j) dvt[j] = s.du[j];",
                        "for (int j = 0; j < V; ++j) dvt[j] = s.du[j] / w.beta;"),
    "ddt_bias_missing_scale": ("dx = dz * ea;", "dx = dz;"),
}


def _pins_pass(lib_path) -> bool:
    rng = np.random.default_rng(3)
    T_list = [6, 11]
    H, K, V = 2, 4, 3
    T = sum(T_list)
    p = dict(q=rng.standard_normal((T, H, K)), k=rng.standard_normal((T, H, K)),
             v=rng.standard_normal((T, H, V)), raw_g=rng.standard_normal((T, H, K)),
             raw_beta=rng.standard_normal((T, H)), A_log=rng.standard_normal(H) * 0.5,
             dt_bias=rng.standard_normal((H, K)) * 0.5,
             cu_seqlens=np.array([0, 6, 17], dtype=np.int64))
    dO = rng.standard_normal((T, H, V))
    r = oracle.kda(**p, dO=dO, lib_path=lib_path)
    # forward against the chunk form
    ref_o = chunked_ref.chunk_fwd(**p, chunk=4)
    if np.linalg.norm(r["o"] - ref_o) > 1e-12 * np.linalg.norm(ref_o):
        return False
    # backward against the chunk-form adjoint
    ref = chunked_ref.chunk_bwd(**p, dO=dO, chunk=4)
    for name in ("dq", "dk", "dv", "draw_g", "draw_beta", "dA_log", "ddt_bias"):
        if np.linalg.norm(r[name] - ref[name]) > 1e-10 * np.linalg.norm(ref[name]):
            return False
    # finite differences on a few entries of every input
    step = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("raw_g", "draw_g"),
                        ("raw_beta", "draw_beta"), ("A_log", "dA_log"), ("dt_bias", "ddt_bias")):
        x = p[name]
        ix = tuple(0 for _ in x.shape)
        o0 = x[ix]
        x[ix] = o0 + step
        lp = np.sum(oracle.kda(**p, lib_path=lib_path)["o"] * dO)
        x[ix] = o0 - step
        lm = np.sum(oracle.kda(**p, lib_path=lib_path)["o"] * dO)
        x[ix] = o0
        if abs((lp - lm) / (2 * step) - r[gname][ix]) > 1e-6 * (abs(r[gname][ix]) + 1):
            return False
    return True


def test_unmutated_oracle_passes_the_battery():
    assert _pins_pass(None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must match exactly once"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    import subprocess
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-std=c11", "-o", lib, str(mpath), "-lm"],
                   check=True)
    assert not _pins_pass(lib), "planted mistake %s went unnoticed" % name


# Mistakes in the state input / output path, against the state pins: the chunk
# form from h0, the two-part run, and a finite difference on h0.
STATE_MUTANTS = {
    "h0_ignored": ("if (p->h0) memcpy(s.S, p->h0 + soff, sizeof(double) * KV);", ";"),
    "h0_wrong_sequence": ("const size_t soff = ((size_t)n * H + h) * KV;",
                          "const size_t soff = ((size_t)0 * n + h) * KV;"),
    "ht_not_written": ("if (p->ht) memcpy(p->ht + soff, s.S, sizeof(double) * KV);", ";"),
    "dht_ignored": ("    memcpy(s.dS, p->dht + soff, sizeof(double) * KV);",
                    "    memset(s.dS, 0, sizeof(double) * KV);"),
    "dh0_before_last_decay": ("if (p->dh0) memcpy(p->dh0 + soff, s.dS, sizeof(double) * KV);",
                              "if (p->dh0) memcpy(p->dh0 + soff, s.dSt, sizeof(double) * KV);"),
}


def _state_pins_pass(lib_path) -> bool:
    rng = np.random.default_rng(5)
    H, K, V = 2, 4, 3
    seqlens = [7, 10]
    T = sum(seqlens)
    p = dict(q=rng.standard_normal((T, H, K)), k=rng.standard_normal((T, H, K)),
             v=rng.standard_normal((T, H, V)), raw_g=rng.standard_normal((T, H, K)),
             raw_beta=rng.standard_normal((T, H)), A_log=rng.standard_normal(H) * 0.5,
             dt_bias=rng.standard_normal((H, K)) * 0.5,
             cu_seqlens=np.array([0, 7, 17], dtype=np.int64))
    h0 = rng.standard_normal((2, H, K, V))
    dht = rng.standard_normal((2, H, K, V))
    dO = rng.standard_normal((T, H, V))

    def rel(a, b):
        return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)

    r = oracle.kda(**p, dO=dO, h0=h0, dht=dht, lib_path=lib_path)
    o, ht = chunked_ref.chunk_fwd(**p, chunk=4, h0=h0, return_state=True)
    if rel(r["o"], o) > 1e-12 or rel(r["ht"], ht) > 1e-12:
        return False
    # two-part run of the second sequence, cut after 4 of its 10 tokens
    def sub(a, b):
        s = {k_: (v_[a:b] if k_ in ("q", "k", "v", "raw_g", "raw_beta") else v_)
             for k_, v_ in p.items() if k_ != "cu_seqlens"}
        s["cu_seqlens"] = np.array([0, b - a], dtype=np.int64)
        return s
    mid = oracle.kda(**sub(7, 11), h0=h0[1:], lib_path=lib_path)["ht"]
    tail = oracle.kda(**sub(11, 17), dO=dO[11:], h0=mid, dht=dht[1:], lib_path=lib_path)
    head = oracle.kda(**sub(7, 11), dO=dO[7:11], h0=h0[1:], dht=tail["dh0"], lib_path=lib_path)
    if rel(np.concatenate([head["dk"], tail["dk"]]), r["dk"][7:]) > 1e-11:
        return False
    if rel(head["dh0"][0], r["dh0"][1]) > 1e-11:
        return False
    # finite difference on one h0 entry, loss sum(O dO) + sum(ht dht)
    ix = (1, 0, 2, 1)
    step = 1e-6
    vals = []
    for sgn in (1, -1):
        h = h0.copy()
        h[ix] += sgn * step
        s = oracle.kda(**p, h0=h, lib_path=lib_path)
        vals.append(np.sum(s["o"] * dO) + np.sum(s["ht"] * dht))
    fd = (vals[0] - vals[1]) / (2 * step)
    return abs(fd - r["dh0"][ix]) <= 1e-6 * (abs(r["dh0"][ix]) + 1)


def test_unmutated_oracle_passes_the_state_battery():
    assert _state_pins_pass(None)


@pytest.mark.parametrize("name", sorted(STATE_MUTANTS))
def test_state_mutant_is_caught(name, tmp_path):
    old, new = STATE_MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must match exactly once"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    import subprocess
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-std=c11", "-o", lib, str(mpath), "-lm"],
                   check=True)
    assert not _state_pins_pass(lib), "planted mistake %s went unnoticed" % name
