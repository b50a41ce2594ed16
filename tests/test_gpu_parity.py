"""GPU parity of the HIP path against the FP64 oracle (needs an MI355X).

Tolerances (normalised L2 error, ||x - ref|| / ||ref|| over a whole tensor):
fp32 problems 1e-5 for O and every gradient; bf16 problems 5e-3 for O and
2e-2 for every gradient (bf16 inputs, fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from recompute_kda_chunked_amd import kda_backward, kda_forward, kda_prologue

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "raw_g", "raw_beta", "A_log", "dt_bias")
GRADS = ("dq", "dk", "dv", "draw_g", "draw_beta", "dA_log", "ddt_bias")
TOL = {torch.float32: (1e-5, 1e-5), torch.bfloat16: (5e-3, 2e-2)}
# Worst single (token, head) row: ||x_row - ref_row|| over the RMS row norm of
# the reference tensor. A row that is wrong (a dropped term, a row from the
# wrong chunk, sequence or head) is off by about its own norm, i.e. of order
# 1 here. Rounding alone keeps the worst row of every tested tensor below
# 9.4e-2 (bf16; the [T,H] tensors, one value per row, have the longest tails
# over millions of rows) and 4e-6 (fp32); the bounds sit between the two.
ROW_TOL = {torch.float32: 1e-4, torch.bfloat16: 0.25}


def announce(msg):
    print("\n[case] " + msg, flush=True)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.max(np.abs(a))) if a.size else 0.0
    return float(np.linalg.norm(a - b) / nb)


def row_stats(a, b):
    """(sum of squared errors, sum of squared reference values, largest row
    error, number of rows) of a [T, H, D] or [T, H] tensor pair, rows being
    (token, head) pairs."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    d2 = (a - b) ** 2
    if a.ndim == 3:
        rows = np.sqrt(d2.sum(axis=2))
    else:
        rows = np.sqrt(d2)
    return float(d2.sum()), float((b * b).sum()), float(rows.max()) if rows.size else 0.0, rows.size


def worst_row(a, b):
    """Largest row error over the RMS row norm (0 for an all-zero reference)."""
    e2, r2, mx, n = row_stats(a, b)
    rms = np.sqrt(r2 / n) if n else 0.0
    return mx / rms if rms > 0 else mx


def gpu_run(x, chunk, seg_chunks=0, scale=1.0, with_bwd=True, gate_mode=0):
    args = [x[n] for n in NAMES]
    kw = dict(cu_seqlens_host=x["cu_seqlens_host"], chunk=chunk, seg_chunks=seg_chunks,
              scale=scale, gate_mode=gate_mode)
    out = {"o": kda_forward(*args, x["cu_seqlens"], **kw)}
    if with_bwd:
        out.update(zip(GRADS, kda_backward(*args, x["dO"], x["cu_seqlens"], **kw)))
    torch.cuda.synchronize()
    return out


def to_np(t):
    return t.detach().double().cpu().numpy()


def check(got, ref, dtype, heads=None, label="", sum_scales=None):
    """Normalised L2 error of every output against the stated tolerance.
    sum_scales: for the gate-parameter gradients of a per-head gate in bf16,
    {name: per-head L2 norms of the per-token terms each one sums}; those are
    checked per head as |error| <= tolerance * norm instead."""
    tol_o, tol_g = TOL[dtype]
    errs, sums, rows = {}, {}, {}
    for name, r in ref.items():
        t = got[name]
        if heads is not None:  # select on the device: full tensors can be GBs
            t = t[heads] if name in ("dA_log", "ddt_bias") else t[:, heads]
        a = to_np(t)
        errs[name] = rel(a, r)
        if name not in ("dA_log", "ddt_bias"):
            rows[name] = worst_row(a, r)
        if sum_scales is not None and name in sum_scales:
            # where every term is exactly zero the error itself is compared,
            # as the normalised error takes max|x| when the reference is 0
            scale = sum_scales[name]
            sums[name] = np.abs(to_np(t) - r) / np.where(scale > 0, scale, 1.0)
    print(label, " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    print("  worst row / rms row:", " ".join("%s=%.2e" % kv for kv in rows.items()), flush=True)
    for name, e in rows.items():
        assert np.isfinite(e) and e <= ROW_TOL[dtype], (name, "worst row", e, ROW_TOL[dtype])
    for name, e in errs.items():
        tol = tol_o if name == "o" else tol_g
        if name in sums:
            print("  %s error over the L2 norm of its terms: %s" % (name, np.array2string(
                sums[name], precision=2)), flush=True)
            assert np.all(sums[name] <= tol), (name, sums[name], tol)
        else:
            assert np.isfinite(e) and e <= tol, (name, e, tol)
    return errs


def gate_sum_scales(x, ref, heads=None, gate_mode=0):
    """The L2 norms of the per-token terms that ddt_bias and dA_log sum, from
    the oracle's draw_g: ddt_bias sums draw_g over tokens; dA_log sums
    draw_g * (raw_g + dt_bias) (smooth gate map) or draw_g * softplus(z) /
    sigmoid(z), z = raw_g + dt_bias (softplus-clamp map), over tokens and
    channels. A sum of terms whose errors are independent at a relative level
    e has an error near e times the L2 norm of its terms; its error relative
    to the sum itself grows with the cancellation among the terms, which
    these sums over every token of a head have in plenty. Works for a gate
    per channel ([T,H,K]) and per head ([T,H])."""
    sel = slice(None) if heads is None else heads
    xg = x["raw_g"][:, sel].double().cpu().numpy()
    b = x["dt_bias"][sel].double().cpu().numpy()
    dg = ref["draw_g"]
    z = xg + b[None]
    if gate_mode == 0:
        ta = dg * z
    else:
        with np.errstate(over="ignore"):
            ta = dg * np.logaddexp(0.0, z) * (1.0 + np.exp(-z))
        ta = np.where(dg == 0, 0.0, ta)
    red = tuple(range(2, dg.ndim))
    return {"ddt_bias": np.sqrt(np.sum(dg ** 2, axis=0)),
            "dA_log": np.sqrt(np.sum(ta ** 2, axis=(0,) + red))}


def oracle_run(x, heads=None, scale=1.0, with_bwd=True, gate_mode=0):
    sel = (lambda t: t) if heads is None else (lambda t: t[:, heads])
    args = [sel(x[n]) for n in ("q", "k", "v", "raw_g", "raw_beta")]
    A = x["A_log"] if heads is None else x["A_log"][heads]
    B = x["dt_bias"] if heads is None else x["dt_bias"][heads]
    return oracle.kda(*args, A, B, cu_seqlens=x["cu_seqlens_host"],
                      dO=sel(x["dO"]) if with_bwd else None, scale=scale, gate_mode=gate_mode)


# ------------------------------------------------------------------ small, full comparison


@pytest.mark.parametrize("name", ["tiny_f32", "small_f32"])
def test_fp32_workloads_full(name):
    w = kda_inputs.WORKLOADS[name]
    announce("%s full vs oracle" % name)
    x = kda_inputs.workload_inputs(w, device="cuda")
    check(gpu_run(x, w.chunk), oracle_run(x), torch.float32, label=name)


RAGGED = [1, 17, 63, 64, 65, 200]


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_fp32_ragged_varlen_every_chunk_size(chunk):
    announce("fp32 ragged D64 chunk %d" % chunk)
    x = kda_inputs.make_inputs(RAGGED, 3, 64, 64, torch.float32, seed=11, device="cuda",
                               A_log=0.3, dt_bias=0.2)
    check(gpu_run(x, chunk), oracle_run(x), torch.float32, label="C%d" % chunk)


@pytest.mark.parametrize("D,chunk", [(128, 64), (128, 32), (64, 64), (64, 32)])
def test_bf16_ragged_varlen(D, chunk):
    announce("bf16 ragged D%d chunk %d" % (D, chunk))
    x = kda_inputs.make_inputs(RAGGED + [130], 2, D, D, torch.bfloat16, seed=12, device="cuda")
    check(gpu_run(x, chunk), oracle_run(x), torch.bfloat16, label="bf16 D%d C%d" % (D, chunk))


@pytest.mark.parametrize("D,dtype,chunk", [(64, torch.bfloat16, 64), (128, torch.bfloat16, 64),
                                           (64, torch.float32, 32), (128, torch.float32, 32)])
def test_wide_value_tiles(D, dtype, chunk):
    # enough (sequence, head) pairs that N*H*V/32 scan blocks exceed the CU
    # count (256 on MI355X): both scans switch to 64-column value tiles
    H = 96 if D == 64 else 48
    announce("wide value tiles D%d %s chunk %d, N=3 H=%d" % (D, dtype, chunk, H))
    x = kda_inputs.make_inputs([40, 9, 77], H, D, D, dtype, seed=21, device="cuda")
    check(gpu_run(x, chunk), oracle_run(x), dtype, label="wide D%d C%d" % (D, chunk))


def test_fp32_d128_and_segment_streaming():
    announce("fp32 D128 chunk 32, one-chunk segments")
    x = kda_inputs.make_inputs([70, 1, 130], 2, 128, 128, torch.float32, seed=13, device="cuda")
    ref = oracle_run(x)
    check(gpu_run(x, 32), ref, torch.float32, label="seg auto")
    check(gpu_run(x, 32, seg_chunks=1), ref, torch.float32, label="seg 1")
    check(gpu_run(x, 32, seg_chunks=3), ref, torch.float32, label="seg 3")


def test_slow_decay_long_memory():
    announce("slow decay dt_bias=-8, fp32 and bf16")
    for dt, D, C in ((torch.float32, 64, 64), (torch.bfloat16, 128, 64)):
        x = kda_inputs.make_inputs([700, 300], 2, D, D, dt, seed=14, device="cuda", dt_bias=-8.0)
        check(gpu_run(x, C, seg_chunks=3), oracle_run(x), dt, label=str(dt))


def test_scale_argument():
    announce("scale 1/sqrt(K)")
    x = kda_inputs.make_inputs([90, 33], 2, 64, 64, torch.float32, seed=15, device="cuda")
    s = 64 ** -0.5
    check(gpu_run(x, 32, scale=s), oracle_run(x, scale=s), torch.float32, label="scale")


# ------------------------------------------------------------------ special inputs


def test_beta_zero_gives_exact_zeros():
    announce("beta = 0")
    x = kda_inputs.make_inputs([100, 28], 2, 64, 64, torch.float32, seed=16, device="cuda")
    x["raw_beta"].fill_(-1e4)
    got = gpu_run(x, 64)
    for name in ("o",) + GRADS:
        assert torch.count_nonzero(got[name]).item() == 0, name


def test_gate_at_bound_stays_finite():
    # Single write at token 0, then beta = 0 and every channel decaying at the
    # bound: the chunk's cumulative gate runs down to -5 * 63. Any unsafe split
    # of exp(G_r - G_s) overflows here.
    announce("gate at the -5 bound, single write")
    for dt, D in ((torch.float32, 64), (torch.bfloat16, 128)):
        x = kda_inputs.make_inputs([128], 1, D, D, dt, seed=17, device="cuda")
        x["raw_beta"].fill_(-1e4)
        x["raw_beta"][0] = 40.0
        x["q"].copy_(x["k"][0:1].expand_as(x["q"]))
        x["raw_g"].fill_(40.0)
        x["raw_g"][:, :, ::2] = -1e4  # half the channels hold, half decay at -5
        got = gpu_run(x, 64)
        for name in ("o",) + GRADS:
            assert torch.isfinite(got[name]).all(), (dt, name)
        ref = oracle_run(x)
        check(got, ref, dt, label="bound " + str(dt))



def test_large_qk_magnitudes():
    # The in-kernel L2 normalisation makes the operator invariant to the scale
    # of q and k, and the kernels form some products from unnormalised rows
    # (the row side of the chunk-local pair products). q and k scaled by 1e4,
    # with every second channel decaying at the -5 bound so that gate factors
    # inside a chunk reach e^75, must stay finite and match the oracle.
    announce("q and k scaled by 1e4, half the channels at the gate bound")
    for dt, D in ((torch.float32, 64), (torch.bfloat16, 128)):
        x = kda_inputs.make_inputs([200, 77], 2, D, D, dt, seed=23, device="cuda")
        x["q"].mul_(1e4)
        x["k"].mul_(1e4)
        x["raw_g"][:, :, ::2] = 40.0
        got = gpu_run(x, 64)
        for name in ("o",) + GRADS:
            assert torch.isfinite(got[name]).all(), (dt, name)
        ref = oracle_run(x)
        check(got, ref, dt, label="large q, k " + str(dt))

# ------------------------------------------------------------------ structure


def test_prologue_step():
    announce("prologue step")
    x = kda_inputs.make_inputs(RAGGED, 3, 128, 128, torch.bfloat16, seed=18, device="cuda",
                               A_log=-0.4, dt_bias=0.7)
    qh, kh, be, gc = kda_prologue(x["q"], x["k"], x["raw_g"], x["raw_beta"], x["A_log"],
                                  x["dt_bias"], x["cu_seqlens"],
                                  cu_seqlens_host=x["cu_seqlens_host"], chunk=64)
    torch.cuda.synchronize()
    ref = oracle.prologue(x["q"], x["k"], x["raw_g"], x["raw_beta"], x["A_log"], x["dt_bias"],
                          x["cu_seqlens_host"], chunk=64)
    for name, t in (("qh", qh), ("kh", kh), ("beta", be), ("gcum", gc)):
        e = rel(to_np(t), ref[name])
        print("prologue", name, "%.2e" % e, flush=True)
        assert e <= 1e-6, (name, e)


def test_many_short_sequences():
    # 300 sequences (more than the chunk table's 256 threads, so each thread
    # takes two), lengths 1..130 with empty ones among them, three segments
    announce("many short sequences, N=300")
    rng = np.random.default_rng(23)
    lens = [int(v) for v in rng.integers(0, 131, size=300)]
    lens[0], lens[7], lens[299] = 0, 1, 0
    x = kda_inputs.make_inputs(lens, 2, 64, 64, torch.float32, seed=23, device="cuda")
    ref = oracle_run(x)
    check(gpu_run(x, 32), ref, torch.float32, label="N300 C32")
    check(gpu_run(x, 64, seg_chunks=97), ref, torch.float32, label="N300 C64 seg97")


def test_many_sequences_in_windows():
    # 300 sequences of 0..400 tokens, at most 600 chunks per segment: the
    # plan takes windows of 2 chunks of every sequence (7 segments, 246
    # sequences carrying their state across window starts, 800 checkpoints),
    # so the chunk table's per-segment scans run over more sequences than
    # its threads. fp32 results are bit-identical to one segment except the
    # gate-parameter sums, which add their per-chunk partials in another order.
    announce("300 sequences in windows of 2 chunks")
    rng = np.random.default_rng(29)
    lens = [int(v) for v in rng.integers(0, 401, size=300)]
    lens[0], lens[5], lens[299] = 0, 0, 0
    x = kda_inputs.make_inputs(lens, 2, 64, 64, torch.float32, seed=29, device="cuda")
    win = gpu_run(x, 32, seg_chunks=600)
    whole = gpu_run(x, 32, seg_chunks=100000)
    for name in win:
        if name in ("dA_log", "ddt_bias"):
            assert rel(to_np(win[name]), to_np(whole[name])) <= 1e-6, name
        else:
            assert torch.equal(win[name], whole[name]), name
    check(win, oracle_run(x), torch.float32, label="N300 windows")


def test_bitwise_deterministic():
    announce("run-to-run determinism")
    x = kda_inputs.make_inputs([300, 77], 4, 128, 128, torch.bfloat16, seed=19, device="cuda")
    a = gpu_run(x, 64, seg_chunks=2)
    b = gpu_run(x, 64, seg_chunks=2)
    for name in a:
        assert torch.equal(a[name], b[name]), name


def test_chunk_size_invariance_bf16():
    announce("C32 vs C64, bf16")
    x = kda_inputs.make_inputs([257, 64], 2, 128, 128, torch.bfloat16, seed=20, device="cuda")
    ref = oracle_run(x)
    check(gpu_run(x, 32), ref, torch.bfloat16, label="C32")
    check(gpu_run(x, 64), ref, torch.bfloat16, label="C64")


# ------------------------------------------------------------------ scalar gate per head


def head_gate_inputs(seqlens, H, D, dtype, seed, per_head_params=True):
    """raw_g [T,H] ~ N(0,1); a different A_log and dt_bias for every head, or
    both zero as in the measured workloads."""
    x = kda_inputs.make_inputs(seqlens, H, D, D, dtype, seed=seed, device="cuda",
                               gate_per_head=True)
    if per_head_params:
        x["A_log"].copy_(torch.linspace(-0.6, 0.4, H))
        x["dt_bias"].copy_(torch.linspace(0.5, -0.9, H))
    return x


@pytest.mark.parametrize("gate_mode", [0, 1])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_head_gate_fp32_ragged(chunk, gate_mode):
    announce("per-head gate fp32 ragged D64 chunk %d mode %d" % (chunk, gate_mode))
    x = head_gate_inputs(RAGGED, 3, 64, torch.float32, seed=51)
    check(gpu_run(x, chunk, gate_mode=gate_mode), oracle_run(x, gate_mode=gate_mode),
          torch.float32, label="head C%d m%d" % (chunk, gate_mode))


@pytest.mark.parametrize("D,chunk", [(128, 64), (128, 32), (64, 64), (64, 32)])
def test_head_gate_bf16_ragged_segments(D, chunk):
    # dA_log and ddt_bias of a per-head gate are sums over all tokens of
    # terms that cancel heavily (28-fold for head 1's dA_log at D = 64); the
    # bf16 operands move them by up to 2.6e-2 of their value, and the
    # per-channel path with the same gate repeated over K moves them the
    # same way. They are held to the tolerance against the scale of their
    # terms (gate_sum_scales).
    announce("per-head gate bf16 ragged D%d chunk %d, segments of 2 chunks" % (D, chunk))
    x = head_gate_inputs(RAGGED + [130], 2, D, torch.bfloat16, seed=52)
    ref = oracle_run(x)
    sc = gate_sum_scales(x, ref)
    check(gpu_run(x, chunk), ref, torch.bfloat16, label="head bf16 D%d C%d" % (D, chunk),
          sum_scales=sc)
    check(gpu_run(x, chunk, seg_chunks=2), ref, torch.bfloat16, label="seg 2", sum_scales=sc)


def test_head_gate_fp32_d128_slow_decay():
    announce("per-head gate fp32 D128 chunk 32, slow decay")
    x = head_gate_inputs([300, 1, 97], 2, 128, torch.float32, seed=53)
    x["dt_bias"].fill_(-8.0)
    check(gpu_run(x, 32, seg_chunks=3), oracle_run(x), torch.float32, label="head slow")


def test_head_gate_switching_at_the_bound():
    # gates switch per token between exactly 0 and exactly the bound, a
    # different pattern in each head, under both gate maps
    announce("per-head gate switching between 0 and the bound")
    for dt, D in ((torch.float32, 64), (torch.bfloat16, 128)):
        x = head_gate_inputs([128, 77], 2, D, dt, seed=54)
        on = torch.rand(x["raw_g"].shape, generator=torch.Generator().manual_seed(54)) < 0.5
        x["raw_g"].copy_(torch.where(on, 40.0, -1e4).to(dt))
        x["A_log"].zero_()
        x["dt_bias"].zero_()
        for mode in (0, 1):
            got = gpu_run(x, 64, gate_mode=mode)
            for name in ("o",) + GRADS:
                assert torch.isfinite(got[name]).all(), (dt, mode, name)
            # saturated gates: the gate-parameter gradients are exactly 0
            check(got, oracle_run(x, gate_mode=mode), dt, label="switch %s m%d" % (dt, mode))


def test_head_gate_prologue_step():
    announce("per-head gate prologue step")
    x = head_gate_inputs(RAGGED, 3, 128, torch.bfloat16, seed=55)
    qh, kh, be, gc = kda_prologue(x["q"], x["k"], x["raw_g"], x["raw_beta"], x["A_log"],
                                  x["dt_bias"], x["cu_seqlens"],
                                  cu_seqlens_host=x["cu_seqlens_host"], chunk=64)
    torch.cuda.synchronize()
    ref = oracle.prologue(x["q"], x["k"], x["raw_g"], x["raw_beta"], x["A_log"], x["dt_bias"],
                          x["cu_seqlens_host"], chunk=64)
    for name, t in (("qh", qh), ("kh", kh), ("beta", be), ("gcum", gc)):
        e = rel(to_np(t), ref[name])
        print("head prologue", name, "%.2e" % e, flush=True)
        assert e <= 1e-6, (name, e)
