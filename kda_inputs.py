"""Seeded synthetic inputs and the named workloads for the KDA operator.

This module holds no arithmetic of the method: it only draws random tensors
and describes shapes. Both the FP64 oracle (through the tests) and the GPU
path are fed from it.

Inputs follow the measurement configuration of "KDA Memory with Recompute:
FLA vs cuDNN Frontend FROST" (section "Sources and measurement
configuration"): Q, K, V, raw gate, raw beta and the output gradient dO drawn
N(0,1) in float32 and rounded (round-to-nearest-even) to the workload dtype;
FP32 A_log and dt_bias initialised to zero; equal-length sequences packed with
boundaries (cu_seqlens).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seqlens: tuple  # lengths of the packed sequences
    H: int
    D: int  # K = V = D
    dtype: str  # "f32" or "bf16"
    chunk: int
    seed: int
    A_log: float = 0.0
    dt_bias: float = 0.0
    gate_per_head: bool = False  # raw_g [T,H], dt_bias [H] (scalar gate)
    gdn2: bool = False  # GDN-2: raw_b [T,H,K] and raw_w [T,H,V] instead of raw_beta

    @property
    def T(self) -> int:
        return int(sum(self.seqlens))

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def cu_seqlens(self) -> list[int]:
        cu = [0]
        for n in self.seqlens:
            cu.append(cu[-1] + int(n))
        return cu


# The five workloads: a tiny fp32 case, the small fp32 preset (10 packed
# sequences of 512), the 8K x H64 bf16 case the headline throughput is quoted
# on, the 8 x 8K packed varlen case and the 128K x H96 long-context case.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", (256,), 2, 64, "f32", 64, seed=1),
    "small_f32": Workload("small_f32", (512,) * 10, 12, 64, "f32", 16, seed=2),
    "t8k_h64_bf16": Workload("t8k_h64_bf16", (8192,), 64, 128, "bf16", 64, seed=3),
    "varlen8x8k_h16_bf16": Workload("varlen8x8k_h16_bf16", (8192,) * 8, 16, 128, "bf16", 64, seed=4),
    "t128k_h96_bf16": Workload("t128k_h96_bf16", (131072,), 96, 128, "bf16", 64, seed=5),
    # the 8K x H64 shape with one scalar gate per head and token (the Gated
    # DeltaNet form)
    "gdn_t8k_h64_bf16": Workload("gdn_t8k_h64_bf16", (8192,), 64, 128, "bf16", 64, seed=6,
                                 gate_per_head=True),
    # the same shape under GDN-2: per-channel erase and write gates
    "gdn2_t8k_h64_bf16": Workload("gdn2_t8k_h64_bf16", (8192,), 64, 128, "bf16", 64, seed=7,
                                  gdn2=True),
}

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "raw_g": 3, "raw_beta": 4, "dO": 5, "h0": 6, "dht": 7,
              "raw_b": 8, "raw_w": 9}


def _randn(shape, seed: int, tensor_id: int, device, dtype) -> torch.Tensor:
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1000003 + tensor_id * 7919 + 17)
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(dtype)


def make_inputs(seqlens, H: int, K: int, V: int, dtype=torch.float32, seed: int = 0,
                device="cpu", A_log: float = 0.0, dt_bias: float = 0.0,
                with_dO: bool = True, gate_per_head: bool = False, gdn2: bool = False) -> dict:
    """Draw one problem. Returns torch tensors on ``device``:
    q,k,raw_g [T,H,K]; v,dO [T,H,V]; raw_beta [T,H] (all ``dtype``);
    A_log [H], dt_bias [H,K] (float32, constant fill); cu_seqlens int32 [N+1]
    on ``device`` plus ``cu_seqlens_host`` (a Python list). gate_per_head:
    raw_g [T,H] and dt_bias [H] instead. gdn2: also raw_b [T,H,K] and raw_w
    [T,H,V] ~ N(0,1) in ``dtype``.
    """
    seqlens = [int(n) for n in seqlens]
    T = sum(seqlens)
    cu = [0]
    for n in seqlens:
        cu.append(cu[-1] + n)
    out = {
        "q": _randn((T, H, K), seed, TENSOR_IDS["q"], device, dtype),
        "k": _randn((T, H, K), seed, TENSOR_IDS["k"], device, dtype),
        "v": _randn((T, H, V), seed, TENSOR_IDS["v"], device, dtype),
        "raw_g": _randn((T, H) if gate_per_head else (T, H, K), seed, TENSOR_IDS["raw_g"],
                        device, dtype),
        "raw_beta": _randn((T, H), seed, TENSOR_IDS["raw_beta"], device, dtype),
        "A_log": torch.full((H,), float(A_log), dtype=torch.float32, device=device),
        "dt_bias": torch.full((H,) if gate_per_head else (H, K), float(dt_bias),
                              dtype=torch.float32, device=device),
        "cu_seqlens": torch.tensor(cu, dtype=torch.int32, device=device),
        "cu_seqlens_host": cu,
    }
    if with_dO:
        out["dO"] = _randn((T, H, V), seed, TENSOR_IDS["dO"], device, dtype)
    if gdn2:
        out["raw_b"] = _randn((T, H, K), seed, TENSOR_IDS["raw_b"], device, dtype)
        out["raw_w"] = _randn((T, H, V), seed, TENSOR_IDS["raw_w"], device, dtype)
    return out


def make_states(n_seqs: int, H: int, K: int, V: int, seed: int = 0, device="cpu") -> dict:
    """Initial states h0 and final-state gradients dht, fp32 [N,H,K,V] ~ N(0,1)."""
    shape = (n_seqs, H, K, V)
    return {"h0": _randn(shape, seed, TENSOR_IDS["h0"], device, torch.float32),
            "dht": _randn(shape, seed, TENSOR_IDS["dht"], device, torch.float32)}


def workload_inputs(w: Workload, device="cpu", with_dO: bool = True) -> dict:
    return make_inputs(w.seqlens, w.H, w.D, w.D, w.torch_dtype, w.seed, device,
                       w.A_log, w.dt_bias, with_dO, w.gate_per_head, w.gdn2)
