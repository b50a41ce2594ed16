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


def test_metric_labels_name_each_workload():
    import json
    import kda_inputs
    W = kda_inputs.WORKLOADS
    base = json.load(open(os.path.join(ROOT, "BASELINE.json")))["metric"]
    assert bench.metric_label(W["t8k_h64_bf16"]) == base
    labels = {n: bench.metric_label(w) for n, w in W.items()}
    assert len(set(labels.values())) == len(labels)  # every workload its own label
    assert "8×8K packed×H16×D128 bf16" in labels["varlen8x8k_h16_bf16"]
    assert "1×128K×H96×D128 bf16" in labels["t128k_h96_bf16"]
    assert "10×512 packed×H12×D64 fp32 C16" in labels["small_f32"]
    assert labels["gdn_t8k_h64_bf16"].startswith("GDN (scalar gate per head)")


def test_every_timed_kernel_kind_has_a_byte_count():
    D, esz = 128, 2
    # the recording and state-only scans move workspace only
    assert bench.kernel_alg_bytes("scan_rec", D, esz, D) == 0.0
    assert bench.kernel_alg_bytes("scan_state", D, esz, D) == 0.0
    assert bench.kernel_alg_bytes("chunk_local_bwd", D, esz, D) == \
        bench.kernel_alg_bytes("chunk_local", D, esz, D) == 1026
    assert bench.kernel_alg_bytes("chunk_local_state", D, esz, D) == 770  # no q rows


def test_quantiles():
    v = [5.0, 1.0, 3.0, 2.0, 4.0]
    assert bench.quantile(v, 0.0) == 1.0 and bench.quantile(v, 1.0) == 5.0
    assert bench.quantile(v, 0.5) == 3.0


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
