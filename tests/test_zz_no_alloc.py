"""kda_fwd_noalloc (the forward for callers that cannot allocate) against
kda_fwd on the same inputs, through the C ABI (needs an MI355X).

Two calls in a row, the second with a smaller problem, so the second call
runs on the scratch the first one left behind. The first problem needs
several segments to fit the 64 MiB scratch, so the state crosses segments
through the carry slots; O must equal kda_fwd's bit for bit (same kernels,
same per-chunk arithmetic, the state carried in fp32), which is stricter
than the oracle tolerance both also meet.
"""
import numpy as np
import pytest
import torch

import kda_inputs
from recompute_kda_chunked_amd import _lib, kda_forward, kda_forward_noalloc
from recompute_kda_chunked_amd.ops import Problem
from test_gpu_parity import NAMES, TOL, oracle_run, rel, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # (seqlens, H, D, dtype, chunk): the first needs several segments of the
    # 64 MiB scratch (about 1.4 MB of operands per chunk of 16 heads)
    ([3000, 1, 2500, 0, 700], 16, 128, torch.bfloat16, 64),
    ([500, 77], 4, 64, torch.float32, 32),
]


def segments_needed(seqlens, H, D, dtype, chunk):
    """Longest forward segment whose workspace fits the scratch (the same
    search the entry point makes), and the number of chunks."""
    lib = _lib.load()
    cu = np.concatenate([[0], np.cumsum(seqlens)]).tolist()
    nc = sum((n + chunk - 1) // chunk for n in seqlens)
    best = 0
    for seg in range(1, nc + 1):
        p = Problem(cu[-1], H, D, D, dtype, cu, chunk, seg_chunks=seg)
        if lib.kda_fwd_workspace_bytes(p.ref) <= _lib.NOALLOC_SCRATCH_BYTES:
            best = seg
    return best, nc


def test_noalloc_forward_matches_kda_fwd_twice():
    for it, (lens, H, D, dtype, chunk) in enumerate(CASES):
        seg, nc = segments_needed(lens, H, D, dtype, chunk)
        print("\n[case] call %d: %s H%d D%d %s C%d: %d chunks in segments of %d"
              % (it, lens, H, D, dtype, chunk, nc, seg), flush=True)
        if it == 0:
            assert 1 <= seg < nc, "the first problem must need several segments"
        x = kda_inputs.make_inputs(lens, H, D, D, dtype, seed=70 + it, device="cuda",
                                   A_log=0.2, dt_bias=-0.3)
        args = [x[n] for n in NAMES]
        ref_o = kda_forward(*args, x["cu_seqlens"], cu_seqlens_host=x["cu_seqlens_host"],
                            chunk=chunk)
        o = torch.full_like(ref_o, float("nan"))
        kda_forward_noalloc(*args, x["cu_seqlens"], o, cu_seqlens_host=x["cu_seqlens_host"],
                            chunk=chunk)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all()
        assert torch.equal(o, ref_o), "kda_fwd_noalloc differs from kda_fwd"
        e = rel(to_np(o), oracle_run(x, with_bwd=False)["o"])
        print("  bit-identical to kda_fwd; O vs oracle %.2e" % e, flush=True)
        assert e <= TOL[dtype][0]
