#!/usr/bin/env python3
"""KDA forward + recompute-backward throughput on one MI355X.

One step = kda_fwd + kda_bwd over the whole synthetic batch (inputs resident
in HBM before the timed region). By default the forward also keeps the
states entering the backward's segments (FROST's checkpoint_every_n_tokens,
"KDA Memory with Recompute: FLA vs cuDNN Frontend FROST", section "Both sides
really use recomputation"), so the backward skips the pass that recomputes
them; it still recomputes w, u, qg, kg and h of every chunk. --no-checkpoints
times the backward that recomputes those states too (also reported on the
default line).

Prints one JSON line: tokens/s and ms per step (mean over the timed steps;
median, p10 and p90 of the per-step times; the first step of the process
separately), peak allocated memory by the FROST page's protocol, each kernel
kind's event-timed duration and roofline, the roofline of the dominant
kernel, and the FP64 CPU oracle timed on a bounded sample of the workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def metric_label(w) -> str:
    """The metric string of a workload, e.g. 'KDA fwd+bwd tokens/s at
    1×8K×H64×D128 bf16; peak allocated GiB; %HBM roof'."""
    def tok(n):
        return "%dK" % (n // 1024) if n % 1024 == 0 else str(n)
    lens = set(w.seqlens)
    shape = ("%d×%s" % (len(w.seqlens), tok(w.seqlens[0])) if len(lens) == 1
             else "%d seqs×%d tokens" % (len(w.seqlens), w.T))
    if len(w.seqlens) > 1:
        shape += " packed"
    dt = "bf16" if w.dtype == "bf16" else "fp32"
    op = ("GDN (scalar gate per head)" if w.gate_per_head else
          "GDN-2 (per-channel erase and write gates)" if w.gdn2 else "KDA")
    chunk = "" if w.chunk == 64 else " C%d" % w.chunk
    return "%s fwd+bwd tokens/s at %s×H%d×D%d %s%s; peak allocated GiB; %%HBM roof" % (
        op, shape, w.H, w.D, dt, chunk)


# Algorithmic bytes per (token, head): what the method itself must move.
#   forward:  read q, k, v (D each), raw_g (G), raw_beta, write O (D)
#   backward: read q, k, v, dO (D each), raw_g (G), raw_beta,
#             write dq, dk, dv (D each), draw_g (G), draw_beta
# with G = D gate values per token-head, or 1 for a gate per head. GDN-2
# (B = 2 D) reads raw_b and raw_w (D each) instead of raw_beta and writes
# their gradients instead of draw_beta.
def alg_bytes_per_token_head(D: int, esz: int, G: int, B: int = 1) -> dict:
    fwd = (3 * D + G + B + D) * esz
    bwd = (4 * D + G + B + 3 * D + G + B) * esz
    return {"fwd": fwd, "bwd": bwd, "total": fwd + bwd}


# Algorithmic bytes of each kernel kind per (token, head) of the launch: the
# compulsory reads and writes of its own step (inputs it must read, outputs
# it must write); workspace traffic is overhead and is not counted, so the
# recording and state-only scans, whose inputs and outputs are all
# workspace, have none.
def kernel_alg_bytes(name: str, D: int, esz: int, G: int, B: int = 1) -> float:
    if name == "chunk_grad":      # reads q,k,v,raw_g,raw_beta,dO; writes 5 grads
        return (4 * D + G + B + 3 * D + G + B) * esz
    if name in ("chunk_local", "chunk_local_bwd"):   # reads q,k,v,raw_g,raw_beta
        return (3 * D + G + B) * esz
    if name == "chunk_local_state":                  # reads k,v,raw_g,raw_beta
        return (2 * D + G + B) * esz
    if name == "scan_fwd":        # writes O
        return D * esz
    if name == "scan_bwd":        # reads dO
        return D * esz
    return 0.0


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="t8k_h64_bf16")
    ap.add_argument("--seg-chunks", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peak", action="store_true", help="skip the peak-memory child process")
    ap.add_argument("--no-checkpoints", action="store_true",
                    help="the backward recomputes the states entering its segments itself "
                         "instead of taking them from the forward")
    ap.add_argument("--peak-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the known-size reference kernels for the FETCH_SIZE / "
                         "WRITE_SIZE counters (a 1 GiB device copy and a 1 GiB read)")
    return ap.parse_args(argv)


def copy_calibration() -> int:
    """Kernels of known traffic, five launches each: a 1 GiB device-to-device
    copy (reads and writes 1 GiB), then a sum of the same bytes as int32 in
    int64, which torch runs as a cast (reads 1 GiB, writes 2 GiB) and a
    reduction of the cast (reads 2 GiB, writes 8 bytes)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    v = src.view(torch.int32)
    out = torch.empty((), dtype=torch.int64, device="cuda:0")
    for _ in range(5):
        torch.sum(v, dim=0, dtype=torch.int64, out=out)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "read_bytes_per_launch": n, "launches": 5}),
          flush=True)
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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": "fwd+bwd of heads 0..%d (all %d tokens, %d sequence(s)) of %d, run %d "
                      "times: %.2f s wall in all, %.2f s per run, scaled by %d/%d to the full "
                      "workload" % (nh - 1, w.T, len(w.seqlens), w.H, reps, total, dt, w.H, nh)}


def make_step(x, w, args, checkpoints: bool):
    from recompute_kda_chunked_amd import gdn2_backward, gdn2_forward, kda_backward, kda_forward
    names = ("q", "k", "v", "raw_g", "raw_beta", "A_log", "dt_bias")
    kw = dict(cu_seqlens_host=x["cu_seqlens_host"], chunk=w.chunk, seg_chunks=args.seg_chunks)
    if w.gdn2:  # no forward-saved states on this path: the backward makes them
        g2 = ("q", "k", "v", "raw_g", "raw_b", "raw_w", "A_log", "dt_bias")

        def step_g2():
            o = gdn2_forward(*(x[n] for n in g2), x["cu_seqlens"], **kw)
            g = gdn2_backward(*(x[n] for n in g2), x["dO"], x["cu_seqlens"], **kw)
            return o, g
        return step_g2

    def step():
        if checkpoints:
            o, _, ck = kda_forward(*(x[n] for n in names), x["cu_seqlens"],
                                   save_checkpoints=True, **kw)
        else:
            o, ck = kda_forward(*(x[n] for n in names), x["cu_seqlens"], **kw), None
        g = kda_backward(*(x[n] for n in names), x["dO"], x["cu_seqlens"], checkpoints=ck, **kw)
        return o, g
    return step


def peak_child(args) -> int:
    """Peak allocated memory as the FROST page measures it ("Sources and
    measurement configuration"): a fresh process for the shape, the
    allocator's expandable segments off, warmup excluded and its outputs
    released, then the median of three steady-state fwd+bwd peaks of PyTorch
    allocated bytes (inputs, dO, O, gradients, workspaces and checkpoints)."""
    import torch

    import kda_inputs
    w = kda_inputs.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    x = kda_inputs.workload_inputs(w, device=dev)
    step = make_step(x, w, args, checkpoints=not args.no_checkpoints)
    for _ in range(2):
        out = step()
        del out
    torch.cuda.synchronize()
    alloc, res = [], []
    for _ in range(3):
        torch.cuda.reset_peak_memory_stats(dev)
        out = step()
        torch.cuda.synchronize()
        alloc.append(torch.cuda.max_memory_allocated(dev) / 2**30)
        res.append(torch.cuda.max_memory_reserved(dev) / 2**30)
        del out
    print(json.dumps({"alloc": alloc, "reserved": res}), flush=True)
    return 0


def measure_peak(args):
    env = dict(os.environ)
    env["PYTORCH_HIP_ALLOC_CONF"] = "expandable_segments:False"
    env["PYTORCH_ALLOC_CONF"] = "expandable_segments:False"
    cmd = [sys.executable, os.path.abspath(__file__), "--peak-child", "--workload", args.workload,
           "--seg-chunks", str(args.seg_chunks)]
    if args.no_checkpoints:
        cmd.append("--no-checkpoints")
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=600)
    if r.returncode != 0:
        raise RuntimeError("peak-memory child failed:\n" + r.stderr[-2000:])
    rec = json.loads([ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1])
    return {"peak_alloc_gib": round(statistics.median(rec["alloc"]), 3),
            "peak_reserved_gib": round(statistics.median(rec["reserved"]), 3),
            "peak_alloc_gib_runs": [round(v, 4) for v in rec["alloc"]],
            "peak_protocol": "fresh process, expandable_segments:False, median of 3 "
                             "steady-state fwd+bwd peaks of allocated bytes"}


def timed(step, steps: int):
    """(mean ms per step over the region, per-step ms list, wall seconds): one
    HIP event before the first step and one after each step, on the stream
    the library launches on (torch's current stream)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[steps]) / steps, per, wall


def quantile(v, q):
    s = sorted(v)
    return s[min(len(s) - 1, max(0, int(round(q * (len(s) - 1)))))]


def main() -> int:
    args = parse()
    if args.copy_calibration:
        return copy_calibration()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d (WORLD_SIZE %d) is not "
              "supported" % (args.gpus, world), file=sys.stderr)
        return 2
    if args.peak_child:
        return peak_child(args)
    # the peak-memory measurement runs first, in its own process, before this
    # one touches the GPU
    peak = None if args.no_peak else measure_peak(args)

    import torch

    import kda_inputs
    from recompute_kda_chunked_amd import _lib

    w = kda_inputs.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    x = kda_inputs.workload_inputs(w, device=dev)
    ckpt = not args.no_checkpoints and not w.gdn2
    step = make_step(x, w, args, checkpoints=ckpt)

    # ---- the first step of the process (library and code objects load here)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out = step()
    torch.cuda.synchronize()
    step0_ms = (time.perf_counter() - t0) * 1e3
    del out

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps
    ms, per, wall = timed(step, args.steps)
    tokens_per_s = w.T / (ms / 1e3)

    # the other backward variant, for reference (same inputs, same step count)
    alt = None
    if not w.gdn2:
        alt_step = make_step(x, w, args, checkpoints=not ckpt)
        for _ in range(2):
            alt_step()
        alt_ms, alt_per, _ = timed(alt_step, args.steps)
        alt = {"ms_per_step": round(alt_ms, 4), "median": round(statistics.median(alt_per), 4),
               "tokens_per_s": round(w.T / (alt_ms / 1e3), 1)}

    # ---- per-kernel durations: HIP events the library records on its launch stream
    _lib.profile_begin()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = _lib.profile_end()

    esz = 2 if w.dtype == "bf16" else 4
    G = 1 if w.gate_per_head else w.D
    B = 2 * w.D if w.gdn2 else 1
    th = w.T * w.H
    alg = alg_bytes_per_token_head(w.D, esz, G, B)
    e2e_frac = alg["total"] * th / (ms / 1e3) / 1e9 / HBM_PEAK_GBS
    kernels = {}
    for k, (n, t, u) in prof.items():
        if not n:
            continue
        # one launch covers one segment of chunks for all heads: (chunk, head)
        # pairs x chunk length = token-heads (the workloads' sequence lengths
        # are multiples of the chunk, so every chunk is full)
        units = u / n * w.chunk
        kab = kernel_alg_bytes(k, w.D, esz, G, B) * units
        avg = t / n
        kernels[k] = {"launches_per_step": round(n / args.steps, 3), "avg_ms": round(avg, 4),
                      "total_ms_per_step": round(t / args.steps, 4),
                      "chunk_heads_per_launch": u / n,
                      "alg_bytes_per_launch": kab,
                      "achieved_gbs": round(kab / (avg / 1e3) / 1e9, 1) if kab else 0.0,
                      "frac": round(kab / (avg / 1e3) / 1e9 / HBM_PEAK_GBS, 4) if kab else 0.0}
    dominant = max(kernels, key=lambda k: kernels[k]["total_ms_per_step"])
    d = kernels[dominant]
    traffic = profile_traffic(dominant, w.name)
    roofline = {"bound": "hbm", "achieved": d["achieved_gbs"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": d["frac"],
                "traffic": None if traffic is None else round(traffic / (d["avg_ms"] / 1e3) / 1e9, 1),
                "traffic_bytes_per_launch": traffic,
                "alg_bytes_per_launch": d["alg_bytes_per_launch"],
                "kernel": dominant,
                "alg_bytes_per_token_head": kernel_alg_bytes(dominant, w.D, esz, G, B)}

    line = {
        "metric": metric_label(w), "value": round(tokens_per_s, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "n_seqs": len(w.seqlens), "tokens": w.T, "heads": w.H,
                   "head_dim": w.D, "chunk": w.chunk, "gate": "per head" if w.gate_per_head
                   else "per channel", "beta": "per-channel erase and write gates (GDN-2)"
                   if w.gdn2 else "scalar", "fwd_checkpoints": ckpt,
                   "seg_chunks": args.seg_chunks or "auto"},
        "step_ms": {"median": round(statistics.median(per), 4), "p10": round(quantile(per, 0.1), 4),
                    "p90": round(quantile(per, 0.9), 4), "step0": round(step0_ms, 2)},
        "e2e_hbm_roof_frac": round(e2e_frac, 4), "wall_s_timed": round(wall, 3),
        "kernels": kernels,
        "roofline": roofline,
    }
    if alt:
        line["no_checkpoints" if ckpt else "with_checkpoints"] = alt
    if peak:
        line.update(peak)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
