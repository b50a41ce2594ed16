"""GPU parity of the extensions beyond the measured setting, against the FP64
oracle (needs an MI355X): the softplus-clamp gate map, initial and final
states with their gradients, forward-saved segment checkpoints, and the
scalar gate per head through all of them.

Tolerances as for the operator itself (normalised L2 over a whole tensor):
fp32 problems 1e-5; bf16 problems 5e-3 for O and the final state, 2e-2 for
every gradient including that of the initial state.
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from recompute_kda_chunked_amd import kda, kda_backward, kda_forward

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "raw_g", "raw_beta", "A_log", "dt_bias")
GRADS = ("dq", "dk", "dv", "draw_g", "draw_beta", "dA_log", "ddt_bias")
TOL = {torch.float32: (1e-5, 1e-5), torch.bfloat16: (5e-3, 2e-2)}
RAGGED_EMPTY = [1, 17, 0, 63, 64, 65, 200]


def announce(msg):
    print("\n[case] " + msg, flush=True)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.max(np.abs(a))) if a.size else 0.0
    return float(np.linalg.norm(a - b) / nb)


def to_np(t):
    return t.detach().double().cpu().numpy()


def check(got, ref, dtype, label):
    tol_o, tol_g = TOL[dtype]
    errs = {name: rel(to_np(got[name]), r) for name, r in ref.items()}
    print(label, " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    for name, e in errs.items():
        tol = tol_o if name in ("o", "ht") else tol_g
        assert np.isfinite(e) and e <= tol, (name, e, tol)


def gpu_run(x, chunk, seg_chunks=0, gate_mode=0, st=None, checkpoints=False):
    args = [x[n] for n in NAMES]
    kw = dict(cu_seqlens_host=x["cu_seqlens_host"], chunk=chunk, seg_chunks=seg_chunks,
              gate_mode=gate_mode)
    out = {}
    h0 = st["h0"] if st is not None else None
    if st is not None or checkpoints:
        o, ht, ck = kda_forward(*args, x["cu_seqlens"], initial_state=h0,
                                output_final_state=st is not None,
                                save_checkpoints=checkpoints, **kw)
        out["o"] = o
        if ht is not None:
            out["ht"] = ht
    else:
        out["o"], ck = kda_forward(*args, x["cu_seqlens"], **kw), None
    g = kda_backward(*args, x["dO"], x["cu_seqlens"], initial_state=h0,
                     d_final_state=st["dht"] if st is not None else None, checkpoints=ck, **kw)
    out.update(zip(GRADS, g[:7]))
    if st is not None:
        out["dh0"] = g[7]
    torch.cuda.synchronize()
    return out


def oracle_run(x, gate_mode=0, st=None):
    kw = {}
    if st is not None:
        kw = dict(h0=st["h0"], dht=st["dht"])
    return oracle.kda(*[x[n] for n in NAMES], cu_seqlens=x["cu_seqlens_host"], dO=x["dO"],
                      gate_mode=gate_mode, **kw)


# ------------------------------------------------------------------ gate map R2


@pytest.mark.parametrize("dtype,D,chunk,A_log", [(torch.float32, 64, 32, 0.3),
                                                 (torch.float32, 128, 16, 1.0),
                                                 (torch.bfloat16, 128, 64, 1.0),
                                                 (torch.bfloat16, 64, 32, 0.3)])
def test_softplus_clamp_gate(dtype, D, chunk, A_log):
    announce("gate mode 1 %s D%d C%d A_log %.1f" % (dtype, D, chunk, A_log))
    x = kda_inputs.make_inputs([1, 17, 63, 64, 65, 200], 2, D, D, dtype, seed=41,
                               device="cuda", A_log=A_log, dt_bias=0.2)
    # part of the gates sit at the clamp (no gradient there), part above it
    frac = (torch.nn.functional.softplus(x["raw_g"].float() + 0.2) * np.exp(A_log) >= 5).float()
    print("clamped fraction %.3f" % frac.mean().item(), flush=True)
    check(gpu_run(x, chunk, seg_chunks=2, gate_mode=1), oracle_run(x, gate_mode=1), dtype,
          label="gate1")


# ------------------------------------------------------------------ state ends


@pytest.mark.parametrize("dtype,D,chunk,seg", [(torch.float32, 64, 32, 0),
                                               (torch.float32, 64, 16, 3),
                                               (torch.float32, 128, 32, 2),
                                               (torch.bfloat16, 128, 64, 0),
                                               (torch.bfloat16, 128, 64, 2),
                                               (torch.bfloat16, 64, 32, 3)])
def test_initial_and_final_state(dtype, D, chunk, seg):
    announce("states %s D%d C%d seg %d" % (dtype, D, chunk, seg))
    x = kda_inputs.make_inputs(RAGGED_EMPTY, 2, D, D, dtype, seed=42, device="cuda",
                               A_log=0.2, dt_bias=-1.0)
    st = kda_inputs.make_states(len(RAGGED_EMPTY), 2, D, D, seed=42, device="cuda")
    got = gpu_run(x, chunk, seg_chunks=seg, st=st)
    ref = oracle_run(x, st=st)
    check(got, ref, dtype, label="states")
    # the empty sequence passes its state through in both directions
    assert torch.equal(got["ht"][2], st["h0"][2])
    assert torch.equal(got["dh0"][2], st["dht"][2])


def test_final_state_alone_and_zero_initial_state():
    announce("final state only; zero initial state equals none")
    x = kda_inputs.make_inputs([90, 0, 33], 2, 64, 64, torch.float32, seed=43, device="cuda")
    args = [x[n] for n in NAMES]
    kw = dict(cu_seqlens_host=x["cu_seqlens_host"], chunk=32)
    o, ht, _ = kda_forward(*args, x["cu_seqlens"], output_final_state=True, **kw)
    ref = oracle.kda(*args, cu_seqlens=x["cu_seqlens_host"], final_state=True)
    assert rel(to_np(o), ref["o"]) <= 1e-5 and rel(to_np(ht), ref["ht"]) <= 1e-5
    assert torch.count_nonzero(ht[1]).item() == 0
    z = torch.zeros((3, 2, 64, 64), dtype=torch.float32, device="cuda")
    a = kda_backward(*args, x["dO"], x["cu_seqlens"], **kw)
    b = kda_backward(*args, x["dO"], x["cu_seqlens"], initial_state=z, d_final_state=z, **kw)
    for name, ga, gb in zip(GRADS, a, b):
        assert torch.equal(ga, gb), name


# ------------------------------------------------------------------ checkpoints


@pytest.mark.parametrize("dtype,D,chunk,seg", [(torch.float32, 64, 32, 2),
                                               (torch.bfloat16, 128, 64, 3)])
def test_forward_checkpoints_give_the_same_gradients(dtype, D, chunk, seg):
    announce("checkpoints %s D%d C%d seg %d" % (dtype, D, chunk, seg))
    x = kda_inputs.make_inputs([300, 0, 77, 129], 2, D, D, dtype, seed=44, device="cuda")
    st = kda_inputs.make_states(4, 2, D, D, seed=44, device="cuda")
    for s in (None, st):
        plain = gpu_run(x, chunk, seg_chunks=seg, st=s)
        saved = gpu_run(x, chunk, seg_chunks=seg, st=s, checkpoints=True)
        for name in plain:
            assert torch.equal(plain[name], saved[name]), name
    check(saved, oracle_run(x, st=st), dtype, label="checkpoints")


@pytest.mark.parametrize("dtype,D,chunk,lens,budget_mb,per_head", [
    (torch.float32, 64, 32, [640, 640, 500, 0, 700], 2, False),
    (torch.bfloat16, 128, 64, [900, 0, 1000, 777, 1000], 6, False),
    (torch.float32, 64, 32, [640, 640, 500, 0, 700], 2, True)])
def test_windowed_segments_match_one_segment(dtype, D, chunk, lens, budget_mb, per_head,
                                             monkeypatch):
    # A workspace budget small enough that both directions stream a packed
    # batch of several long sequences in windows of the same chunk positions
    # in every sequence: the backward in windows of 2 (fp32) or 3 (bf16)
    # chunks, the forward in windows of 6, which writes the checkpoints of
    # the backward's windows from inside its own. In fp32 the per-token
    # results are bit-identical to one segment holding every chunk (the
    # states cross the boundaries in fp32); only the gate-parameter sums add
    # their per-chunk partials in another order. In bf16 the backward's
    # recording scan advances the state with U rounded to bf16 inside a
    # segment while each segment starts from the state of the forward's
    # recurrence (fp32 U), so the gradients depend on where the segments
    # start by rounding; they are held to the oracle.
    announce("windows %s D%d C%d budget %d MB%s" % (dtype, D, chunk, budget_mb,
                                                    ", gate per head" if per_head else ""))
    x = kda_inputs.make_inputs(lens, 2, D, D, dtype, seed=47, device="cuda",
                               gate_per_head=per_head)
    if per_head:
        x["A_log"].copy_(torch.tensor([0.3, -0.5]))
        x["dt_bias"].copy_(torch.tensor([-1.0, 0.6]))
    st = kda_inputs.make_states(len(lens), 2, D, D, seed=47, device="cuda")
    whole = gpu_run(x, chunk, seg_chunks=100000, st=st)
    monkeypatch.setenv("KDA_WS_BUDGET_MB", str(budget_mb))
    plain = gpu_run(x, chunk, st=st)
    saved = gpu_run(x, chunk, st=st, checkpoints=True)
    for name in plain:
        assert torch.equal(plain[name], saved[name]), name
        if dtype != torch.float32 and name not in ("o", "ht"):
            continue
        if name in ("dA_log", "ddt_bias"):
            e = rel(to_np(plain[name]), to_np(whole[name]))
            assert e <= 1e-6, (name, e)
        else:
            assert torch.equal(plain[name], whole[name]), name
    ref = oracle_run(x, st=st)
    check(whole, ref, dtype, label="one segment")
    check(saved, ref, dtype, label="windows")


# ------------------------------------------------------------------ autograd


def test_autograd_with_states():
    announce("autograd: initial state and final state")
    x = kda_inputs.make_inputs([40, 70], 2, 64, 64, torch.float32, seed=45, device="cuda")
    st = kda_inputs.make_states(2, 2, 64, 64, seed=45, device="cuda")
    leaves = {n: x[n].clone().requires_grad_(True) for n in NAMES}
    h0 = st["h0"].clone().requires_grad_(True)
    o, ht = kda(*[leaves[n] for n in NAMES], x["cu_seqlens"],
                cu_seqlens_host=x["cu_seqlens_host"], chunk=32, initial_state=h0,
                output_final_state=True, save_checkpoints=True, seg_chunks=1)
    ((o * x["dO"]).sum() + (ht * st["dht"]).sum()).backward()
    ref = oracle_run(x, st=st)
    got = {"o": o, "ht": ht, "dh0": h0.grad}
    got.update({g: leaves[n].grad for n, g in zip(NAMES, GRADS)})
    check(got, ref, torch.float32, label="autograd")


# ------------------------------------------------------------------ scalar gate per head


@pytest.mark.parametrize("chunk,seg", [(32, 2), (64, 0)])
def test_head_gate_with_states_and_checkpoints(chunk, seg):
    # one gate per head and token, each head with its own A_log and dt_bias,
    # through initial/final states, forward-saved checkpoints and autograd
    announce("per-head gate, states and checkpoints, fp32 D64 C%d seg %d" % (chunk, seg))
    x = kda_inputs.make_inputs(RAGGED_EMPTY, 3, 64, 64, torch.float32, seed=46, device="cuda",
                               gate_per_head=True)
    x["A_log"].copy_(torch.tensor([0.3, -0.5, 0.1]))
    x["dt_bias"].copy_(torch.tensor([-1.0, 0.6, 2.0]))
    st = kda_inputs.make_states(len(RAGGED_EMPTY), 3, 64, 64, seed=46, device="cuda")
    ref = oracle_run(x, st=st)
    plain = gpu_run(x, chunk, seg_chunks=seg, st=st)
    check(plain, ref, torch.float32, label="head states")
    saved = gpu_run(x, chunk, seg_chunks=seg, st=st, checkpoints=True)
    for name in plain:
        assert torch.equal(plain[name], saved[name]), name
    leaves = {n: x[n].clone().requires_grad_(True) for n in NAMES}
    h0 = st["h0"].clone().requires_grad_(True)
    o, ht = kda(*[leaves[n] for n in NAMES], x["cu_seqlens"],
                cu_seqlens_host=x["cu_seqlens_host"], chunk=chunk, seg_chunks=seg,
                initial_state=h0, output_final_state=True)
    ((o * x["dO"]).sum() + (ht * st["dht"]).sum()).backward()
    got = {"o": o, "ht": ht, "dh0": h0.grad}
    got.update({g: leaves[n].grad for n, g in zip(NAMES, GRADS)})
    assert got["draw_g"].shape == x["raw_g"].shape and got["ddt_bias"].shape == (3,)
    check(got, ref, torch.float32, label="head autograd")
