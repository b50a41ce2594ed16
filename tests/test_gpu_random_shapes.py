"""Seeded random problems against the FP64 oracle (needs an MI355X): packed
batches of 1-5 sequences of 0-150 tokens (empty and one-token sequences
included), 1-3 heads, D 64 or
128, every built chunk size, both gate maps, per-channel and per-head gates,
random scale and streaming segments.

Tolerances as in test_gpu_parity (normalised L2): fp32 1e-5; bf16 5e-3 for
O and 2e-2 for each gradient, for every output of every problem, except the
two gate-parameter gradients of a gate per head: dA_log[h] and ddt_bias[h]
are then single sums over every token and channel of the head, which cancel
heavily with random A_log and dt_bias on short batches (41-fold in one fp32
draw, whose dA_log then reaches 1.001e-5 of its sum at a per-term accuracy of
2.4e-7), so they are held to the tolerance times the L2 norm of their terms.
Each case prints the cancellation ratio of both sums.
"""
import numpy as np
import pytest
import torch

import kda_inputs
from test_gpu_parity import GRADS, NAMES, check, gate_sum_scales, oracle_run

from recompute_kda_chunked_amd import kda_backward, kda_forward

pytestmark = pytest.mark.gpu

BUILT = {(torch.float32, 64): (16, 32, 64), (torch.float32, 128): (16, 32),
         (torch.bfloat16, 64): (32, 64), (torch.bfloat16, 128): (32, 64)}


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 6))
    lens = [int(v) for v in rng.integers(0, 151, size=n)]
    if n > 1 and rng.random() < 0.5:
        lens[int(rng.integers(0, n))] = 1
    if n > 1 and rng.random() < 0.5:
        lens[int(rng.integers(0, n))] = 0
    if sum(lens) == 0:
        lens[-1] = 1
    dtype = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    D = 64 if rng.random() < 0.5 else 128
    chunk = int(rng.choice(BUILT[(dtype, D)]))
    H = int(rng.integers(1, 4))
    return dict(lens=lens, H=H, D=D, dtype=dtype, chunk=chunk,
                per_head=bool(rng.random() < 0.5), gate_mode=int(rng.integers(0, 2)),
                seg=int(rng.integers(0, 4)), scale=float(rng.choice([1.0, D ** -0.5])),
                A_log=float(rng.uniform(-0.5, 0.5)), dt_bias=float(rng.uniform(-1.0, 1.0)))


@pytest.mark.parametrize("seed", range(16))
def test_random_problem(seed):
    c = draw_case(seed)
    print("\n[case] seed %d %s" % (seed, c), flush=True)
    x = kda_inputs.make_inputs(c["lens"], c["H"], c["D"], c["D"], c["dtype"], seed=60 + seed,
                               device="cuda", A_log=c["A_log"], dt_bias=c["dt_bias"],
                               gate_per_head=c["per_head"])
    kw = dict(cu_seqlens_host=x["cu_seqlens_host"], chunk=c["chunk"], seg_chunks=c["seg"],
              scale=c["scale"], gate_mode=c["gate_mode"])
    args = [x[n] for n in NAMES]
    got = {"o": kda_forward(*args, x["cu_seqlens"], **kw)}
    got.update(zip(GRADS, kda_backward(*args, x["dO"], x["cu_seqlens"], **kw)))
    torch.cuda.synchronize()
    ref = oracle_run(x, scale=c["scale"], gate_mode=c["gate_mode"])
    sc = gate_sum_scales(x, ref, gate_mode=c["gate_mode"])
    for name in ("dA_log", "ddt_bias"):
        # cancellation ratio of each sum: L2 norm of its terms over |sum|
        ratio = sc[name] / np.maximum(np.abs(ref[name]), 1e-300)
        print("  %s cancellation (terms' norm / |sum|): max %.1f" % (name, float(np.max(ratio))),
              flush=True)
    # only the sums of a per-head gate (one value per head over every token and
    # channel, cancelling up to 41-fold in these draws) are held against the
    # norm of their terms (see test_gpu_parity.check); the per-channel gate's
    # sums and every other output meet the stated metric as they are
    relaxed = c["per_head"]
    check(got, ref, c["dtype"], label="seed %d" % seed, sum_scales=sc if relaxed else None)
