#!/usr/bin/env python3
"""KDA forward + recompute-backward throughput on one MI355X.

One step = kda_fwd + kda_bwd over the whole synthetic batch (inputs resident
in HBM before the timed region). Prints one JSON line: tokens/s, ms per
step, peak allocated memory, the roofline of the dominant kernel (its
algorithmic bytes over its event-timed average duration) and the FP64 CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA fwd+bwd tokens/s at 1×8K×H64×D128 bf16; peak allocated GiB; %HBM roof"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC_GDN = ("GDN (scalar gate per head) fwd+bwd tokens/s at 1×8K×H64×D128 bf16; "
              "peak allocated GiB; %HBM roof")
# Algorithmic bytes per (token, head): what the method itself must move.
#   forward:  read q, k, v (D each), raw_g (G), raw_beta, write O (D)
#   backward: read q, k, v, dO (D each), raw_g (G), raw_beta,
#             write dq, dk, dv (D each), draw_g (G), draw_beta
# with G = D gate values per token-head, or 1 for a gate per head.
def alg_bytes_per_token_head(D: int, esz: int, G: int) -> dict:
    fwd = (3 * D + G + 1 + D) * esz
    bwd = (4 * D + G + 1 + 3 * D + G + 1) * esz
    return {"fwd": fwd, "bwd": bwd, "total": fwd + bwd}


# Algorithmic bytes of each kernel per (token, head) of the launch: the
# compulsory reads/writes of the step it implements (workspace traffic is
# overhead and is not counted).
def kernel_alg_bytes(name: str, D: int, esz: int, G: int) -> float:
    if name == "chunk_grad":      # reads q,k,v,raw_g,raw_beta,dO; writes 5 grads
        return (4 * D + G + 1 + 3 * D + G + 1) * esz
    if name == "chunk_local":     # reads q,k,v,raw_g,raw_beta
        return (3 * D + G + 1) * esz
    if name == "scan_fwd":        # writes O (forward launches)
        return D * esz
    if name == "scan_bwd":        # reads dO
        return D * esz
    return 0.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="t8k_h64_bf16")
    ap.add_argument("--seg-chunks", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--checkpoints", action="store_true",
                    help="the forward saves the states entering the backward's segments "
                         "(the backward skips its checkpoint pass; w, u, h are still "
                         "recomputed per chunk)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def copy_calibration() -> int:
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)
    return 0


def profile_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/traffic_<workload>.txt, or None when that summary was taken from
    a different kernel source than the one built now."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    src = os.path.join(ROOT, "recompute_kda_chunked_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(src)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(open(os.path.join(src, f), "rb").read())
    if rec.get("csrc_sha256") != h.hexdigest():
        return None
    v = rec.get("hbm_bytes_per_launch.%s" % kernel)
    return float(v) if v else None


def cpu_baseline(x, w) -> dict:
    """The FP64 oracle on the first n heads of the same inputs (n = twice the
    host threads, at most H), all tokens, scaled to the full workload."""
    import numpy as np
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    # two heads per thread: about 1 s (8K) to 16 s (128K) of wall time per run
    nh = max(1, min(w.H, 2 * threads))
    sl = slice(0, nh)
    host = {n: x[n][:, sl].double().cpu().numpy() for n in ("q", "k", "v", "raw_g", "raw_beta", "dO")}
    A = x["A_log"][sl].double().cpu().numpy()
    B = x["dt_bias"][sl].double().cpu().numpy()
    cu = np.asarray(x["cu_seqlens_host"], dtype=np.int64)
    oracle.kda(host["q"][:1], host["k"][:1], host["v"][:1], host["raw_g"][:1],
               host["raw_beta"][:1], A, B, cu_seqlens=[0, 1], dO=host["dO"][:1])  # load only
    # repeated until at least 10 s of wall time (at most 20 runs), so that the
    # rate is not a one-second reading
    reps, total = 0, 0.0
    while reps < 20 and (total < 10.0 or reps == 0):
        t0 = time.perf_counter()
        oracle.kda(host["q"], host["k"], host["v"], host["raw_g"], host["raw_beta"], A, B,
                   cu_seqlens=cu, dO=host["dO"], n_threads=threads)
        total += time.perf_counter() - t0
        reps += 1
    dt = total / reps
    full_s = dt * w.H / nh  # the whole workload at the measured per-head rate
    return {"value": w.T / full_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "fwd+bwd of heads 0..%d (all %d tokens, %d sequence(s)) of %d, run %d "
                      "times: %.2f s wall in all, %.2f s per run, scaled by %d/%d to the full "
                      "workload" % (nh - 1, w.T, len(w.seqlens), w.H, reps, total, dt, w.H, nh)}


def main() -> int:
    args = parse()
    if args.copy_calibration:
        return copy_calibration()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d (WORLD_SIZE %d) is not "
              "supported" % (args.gpus, world), file=sys.stderr)
        return 2
    import torch

    import kda_inputs
    from recompute_kda_chunked_amd import _lib, kda_backward, kda_forward

    w = kda_inputs.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    x = kda_inputs.workload_inputs(w, device=dev)
    names = ("q", "k", "v", "raw_g", "raw_beta", "A_log", "dt_bias")
    kw = dict(cu_seqlens_host=x["cu_seqlens_host"], chunk=w.chunk, seg_chunks=args.seg_chunks)

    def step():
        if args.checkpoints:
            o, _, ck = kda_forward(*(x[n] for n in names), x["cu_seqlens"],
                                   save_checkpoints=True, **kw)
        else:
            o, ck = kda_forward(*(x[n] for n in names), x["cu_seqlens"], **kw), None
        g = kda_backward(*(x[n] for n in names), x["dO"], x["cu_seqlens"], checkpoints=ck, **kw)
        return o, g

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    tokens_per_s = w.T / (ms / 1e3)

    # ---- per-kernel durations: HIP events the library records on its launch stream
    _lib.profile_begin()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = _lib.profile_end()
    per_launch = {k: {"launches": n, "avg_ms": t / n, "total_ms_per_step": t / args.steps,
                      "chunk_heads_per_launch": u / n}
                  for k, (n, t, u) in prof.items() if n}
    dominant = max(per_launch, key=lambda k: per_launch[k]["total_ms_per_step"])

    # ---- peak allocated memory over one step (inputs, dO, outputs, grads, workspaces live)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    out = step()
    torch.cuda.synchronize()
    peak_alloc = torch.cuda.max_memory_allocated(dev) / 2**30
    peak_res = torch.cuda.max_memory_reserved(dev) / 2**30
    del out

    esz = 2 if w.dtype == "bf16" else 4
    G = 1 if w.gate_per_head else w.D
    th = w.T * w.H
    alg = alg_bytes_per_token_head(w.D, esz, G)
    e2e_frac = alg["total"] * th / (ms / 1e3) / 1e9 / HBM_PEAK_GBS
    d = per_launch[dominant]
    # one launch covers one segment of chunks for all heads: its unit count is
    # (chunk, head) pairs x chunk length = token-heads (the workloads' sequence
    # lengths are multiples of the chunk, so every chunk is full)
    units = d["chunk_heads_per_launch"] * w.chunk
    kab = kernel_alg_bytes(dominant, w.D, esz, G)
    achieved = kab * units / (d["avg_ms"] / 1e3) / 1e9
    traffic = profile_traffic(dominant, w.name)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else round(traffic / (d["avg_ms"] / 1e3) / 1e9, 1),
                "traffic_bytes_per_launch": traffic,
                "alg_bytes_per_launch": kab * units,
                "kernel": dominant, "alg_bytes_per_token_head": kab}

    line = {
        "metric": METRIC_GDN if w.gate_per_head else METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "n_seqs": len(w.seqlens), "tokens": w.T, "heads": w.H,
                   "head_dim": w.D, "chunk": w.chunk, "gate": "per head" if w.gate_per_head
                   else "per channel", "fwd_checkpoints": bool(args.checkpoints)},
        "peak_alloc_gib": round(peak_alloc, 3), "peak_reserved_gib": round(peak_res, 3),
        "e2e_hbm_roof_frac": round(e2e_frac, 4), "wall_s_timed": round(wall, 3),
        "kernels": {k: {kk: round(vv, 4) if isinstance(vv, float) else vv for kk, vv in v.items()}
                    for k, v in per_launch.items()},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
