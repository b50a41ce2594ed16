"""GDN-2 on the GPU (kda_gdn2_fwd / kda_gdn2_bwd) against the FP64 GDN-2
oracle (needs an MI355X).

GDN-2 ("KDA at the production shape...", section 1.6): per-channel erase
gate b = sigmoid(raw_b) [T,H,K] and write gate w = sigmoid(raw_w) [T,H,V]
in place of KDA's beta. Tolerances as for KDA (normalised L2 per tensor):
fp32 1e-5; bf16 5e-3 for O, 2e-2 for every gradient; plus the worst
(token, head) row bound of test_gpu_parity.
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from recompute_kda_chunked_amd import (KdaError, gdn2_backward, gdn2_forward, kda_backward,
                                       kda_forward)
from test_gpu_parity import ROW_TOL, TOL, rel, row_stats, to_np

pytestmark = pytest.mark.gpu

INS = ("q", "k", "v", "raw_g", "raw_b", "raw_w", "A_log", "dt_bias")
GRADS = ("dq", "dk", "dv", "draw_g", "draw_b", "draw_w", "dA_log", "ddt_bias")


def gpu(x, chunk, seg=0, gate_mode=0, scale=1.0):
    kw = dict(cu_seqlens_host=x["cu_seqlens_host"], chunk=chunk, seg_chunks=seg,
              gate_mode=gate_mode, scale=scale)
    args = [x[n] for n in INS]
    out = {"o": gdn2_forward(*args, x["cu_seqlens"], **kw)}
    out.update(zip(GRADS, gdn2_backward(*args, x["dO"], x["cu_seqlens"], **kw)))
    torch.cuda.synchronize()
    return out


def ref(x, heads=None, gate_mode=0, scale=1.0):
    sel = (lambda t: t) if heads is None else (lambda t: t[:, heads])
    A = x["A_log"] if heads is None else x["A_log"][heads]
    B = x["dt_bias"] if heads is None else x["dt_bias"][heads]
    return oracle.gdn2(*(sel(x[n]) for n in INS[:6]), A, B, cu_seqlens=x["cu_seqlens_host"],
                       dO=sel(x["dO"]), gate_mode=gate_mode, scale=scale)


def check(got, r, dtype, label, heads=None):
    tol_o, tol_g = TOL[dtype]
    errs, rows = {}, {}
    for name, rv in r.items():
        t = got[name]
        if heads is not None:
            t = t[heads] if name in ("dA_log", "ddt_bias") else t[:, heads]
        a = to_np(t)
        errs[name] = rel(a, rv)
        if name not in ("dA_log", "ddt_bias"):
            e2, r2, mx, n = row_stats(a, rv)
            rows[name] = mx / np.sqrt(r2 / n) if r2 > 0 else mx
    print(label, " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    print("  worst row / rms row:", " ".join("%s=%.2e" % kv for kv in rows.items()), flush=True)
    for name, e in rows.items():
        assert np.isfinite(e) and e <= ROW_TOL[dtype], (name, "worst row", e)
    for name, e in errs.items():
        assert np.isfinite(e) and e <= (tol_o if name == "o" else tol_g), (name, e)


RAGGED = [1, 17, 63, 64, 65, 200]
BUILT = [(torch.float32, 64, 16), (torch.float32, 64, 32), (torch.float32, 128, 16),
         (torch.float32, 128, 32), (torch.bfloat16, 64, 32), (torch.bfloat16, 64, 64),
         (torch.bfloat16, 128, 32), (torch.bfloat16, 128, 64)]


@pytest.mark.parametrize("dtype,D,chunk", BUILT)
def test_gdn2_ragged_every_built_size(dtype, D, chunk):
    print("\n[case] GDN-2 ragged %s D%d C%d" % (dtype, D, chunk), flush=True)
    x = kda_inputs.make_inputs(RAGGED, 2, D, D, dtype, seed=91, device="cuda", A_log=0.3,
                               dt_bias=-0.4, gdn2=True)
    check(gpu(x, chunk), ref(x), dtype, "gdn2 %s D%d C%d" % (dtype, D, chunk))


def test_gdn2_segments_gate_map_scale_and_slow_decay():
    print("\n[case] GDN-2 segments, softplus-clamp gate, scale, slow decay", flush=True)
    for dtype, D, C in ((torch.float32, 64, 32), (torch.bfloat16, 128, 64)):
        x = kda_inputs.make_inputs([300, 0, 129], 2, D, D, dtype, seed=92, device="cuda",
                                   gdn2=True)
        r = ref(x, gate_mode=1, scale=D ** -0.5)
        check(gpu(x, C, seg=2, gate_mode=1, scale=D ** -0.5), r, dtype, "clamp seg2 %s" % dtype)
        x["dt_bias"].fill_(-8.0)
        check(gpu(x, C, seg=3), ref(x), dtype, "slow seg3 %s" % dtype)


def test_gdn2_with_gates_at_beta_matches_kda():
    # raw_b = raw_w = raw_beta broadcast: the GDN-2 path computes KDA
    print("\n[case] GDN-2 with both gates at beta vs the KDA path", flush=True)
    x = kda_inputs.make_inputs([90, 1, 160], 2, 64, 64, torch.float32, seed=93, device="cuda",
                               A_log=0.2, dt_bias=0.1, gdn2=True)
    x["raw_b"].copy_(x["raw_beta"][:, :, None].expand_as(x["raw_b"]))
    x["raw_w"].copy_(x["raw_beta"][:, :, None].expand_as(x["raw_w"]))
    g = gpu(x, 32)
    kw = dict(cu_seqlens_host=x["cu_seqlens_host"], chunk=32)
    kargs = [x[n] for n in ("q", "k", "v", "raw_g", "raw_beta", "A_log", "dt_bias")]
    o = kda_forward(*kargs, x["cu_seqlens"], **kw)
    dq, dk, dv, dg, dbeta, dA, ddt = kda_backward(*kargs, x["dO"], x["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    for name, a, b in (("o", g["o"], o), ("dq", g["dq"], dq), ("dk", g["dk"], dk),
                       ("dv", g["dv"], dv), ("draw_g", g["draw_g"], dg), ("dA_log", g["dA_log"], dA),
                       ("ddt_bias", g["ddt_bias"], ddt),
                       ("draw_beta", g["draw_b"].sum(2) + g["draw_w"].sum(2), dbeta)):
        e = rel(to_np(a), to_np(b))
        print("  %s %.2e" % (name, e), flush=True)
        assert e <= 1e-5, (name, e)


def test_gdn2_workload_every_head():
    w = kda_inputs.WORKLOADS["gdn2_t8k_h64_bf16"]
    print("\n[case] %s, every head against the GDN-2 oracle" % w.name, flush=True)
    x = kda_inputs.workload_inputs(w, device="cuda")
    got = gpu(x, w.chunk)
    check(got, ref(x), torch.bfloat16, w.name)


def test_gdn2_unbuilt_combinations_are_refused():
    x = kda_inputs.make_inputs([64], 1, 64, 64, torch.float32, seed=94, device="cuda", gdn2=True)
    with pytest.raises(KdaError, match="unsupported"):
        gdn2_forward(*(x[n] for n in INS), x["cu_seqlens"], cu_seqlens_host=x["cu_seqlens_host"],
                     chunk=64)
