"""Host-side logic of bench.py (no GPU): the algorithmic byte counts behind
the roofline figures, the refusal of more than one GPU, and the traffic
summary's source-hash check."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_per_token_head():
    # bf16, D = 128, a gate per channel: forward reads q, k, v, raw_g (256 B
    # each) and raw_beta (2 B) and writes O (256 B); backward reads q, k, v,
    # raw_g, dO and raw_beta and writes dq, dk, dv, draw_g and draw_beta
    a = bench.alg_bytes_per_token_head(128, 2, 128)
    assert (a["fwd"], a["bwd"], a["total"]) == (1282, 2308, 3590)
    # fp32, D = 64
    assert bench.alg_bytes_per_token_head(64, 4, 64)["total"] == 3596
    # a gate per head: raw_g and draw_g are one value per token-head
    g = bench.alg_bytes_per_token_head(128, 2, 1)
    assert g["total"] == 3590 - 3 * 254


def test_kernel_bytes_add_up_to_the_step():
    D, esz = 128, 2
    for G in (D, 1):
        k = {n: bench.kernel_alg_bytes(n, D, esz, G)
             for n in ("chunk_local", "scan_fwd", "scan_bwd", "chunk_grad")}
        # forward = chunk-local reads + O; backward = the gradient kernel's
        assert k["chunk_local"] + k["scan_fwd"] == bench.alg_bytes_per_token_head(D, esz, G)["fwd"]
        assert k["chunk_grad"] == bench.alg_bytes_per_token_head(D, esz, G)["bwd"]
        assert bench.kernel_alg_bytes("gate_reduce", D, esz, G) == 0.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_summary_needs_matching_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_w.txt").write_text("csrc_sha256 = deadbeef\n"
                                        "hbm_bytes_per_launch.chunk_grad = 123\n")
    csrc = tmp_path / "recompute_kda_chunked_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("// kernel\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profile_traffic("chunk_grad", "w") is None
    import hashlib
    sha = hashlib.sha256((csrc / "k.hip").read_bytes()).hexdigest()
    (prof / "traffic_w.txt").write_text("csrc_sha256 = %s\n"
                                        "hbm_bytes_per_launch.chunk_grad = 123\n" % sha)
    assert bench.profile_traffic("chunk_grad", "w") == pytest.approx(123.0)
    assert bench.profile_traffic("scan_fwd", "w") is None
