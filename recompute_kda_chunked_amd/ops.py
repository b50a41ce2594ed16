"""Python binding of the KDA operator: argument checks and marshalling only.

Every step of the operator runs in the HIP kernels behind ``include/kda.h``;
PyTorch supplies device memory (outputs and workspace, so its allocator
accounts for every byte) and the current stream.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib


class KdaError(RuntimeError):
    pass


_DT = {torch.float32: _lib.KDA_F32, torch.bfloat16: _lib.KDA_BF16}


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class Problem:
    """Host-side description of one packed batch (holds the host cu_seqlens)."""

    def __init__(self, T, H, K, V, dtype, cu_host, chunk=64, scale=1.0, lower_bound=-5.0,
                 eps=1e-6, seg_chunks=0, gate_mode=_lib.KDA_GATE_SIGMOID_BOUND):
        self.cu = (ctypes.c_int32 * len(cu_host))(*[int(x) for x in cu_host])
        self.p = _lib.KdaProblem(
            n_seqs=len(cu_host) - 1, total_tokens=int(T), H=int(H), K=int(K), V=int(V),
            chunk=int(chunk), dtype=_DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype),
            gate_mode=int(gate_mode), scale=float(scale), gate_lower_bound=float(lower_bound),
            l2_eps=float(eps), seg_chunks=int(seg_chunks),
            cu_seqlens_host=ctypes.cast(self.cu, ctypes.POINTER(ctypes.c_int32)))

    @property
    def ref(self):
        return ctypes.byref(self.p)

    def check(self) -> int:
        return _lib.load().kda_check_problem(self.ref)

    def fwd_ws(self) -> int:
        return int(_lib.load().kda_fwd_workspace_bytes(self.ref))

    def bwd_ws(self) -> int:
        return int(_lib.load().kda_bwd_workspace_bytes(self.ref))


def _raise(lib, st: int, what: str):
    if st != _lib.KDA_OK:
        raise KdaError("%s failed: %s (status %d)" % (what, _lib.status_text(lib, st), st))


def _check_inputs(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens, extra=()):
    dev = q.device
    if dev.type != "cuda":
        raise KdaError("inputs must be on a GPU device")
    T, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    if dt not in _DT:
        raise KdaError("dtype must be float32 or bfloat16")
    want = {"q": (q, (T, H, K), dt), "k": (k, (T, H, K), dt), "v": (v, (T, H, V), dt),
            "raw_g": (raw_g, (T, H, K), dt), "raw_beta": (raw_beta, (T, H), dt),
            "A_log": (A_log, (H,), torch.float32), "dt_bias": (dt_bias, (H, K), torch.float32),
            "cu_seqlens": (cu_seqlens, (cu_seqlens.shape[0],), torch.int32)}
    for name, (t, shape, dtype) in list(want.items()) + list(extra):
        if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
            raise KdaError("%s: expected shape %s dtype %s, got %s %s"
                           % (name, shape, dtype, tuple(t.shape), t.dtype))
        if t.device != dev or not t.is_contiguous() or t.data_ptr() % 16:
            raise KdaError("%s must be contiguous, 16-byte aligned and on %s" % (name, dev))
    return T, H, K, V, dt


def _cu_host(cu_seqlens, cu_seqlens_host):
    if cu_seqlens_host is not None:
        return [int(x) for x in cu_seqlens_host]
    return [int(x) for x in cu_seqlens.tolist()]  # device-to-host copy (synchronises)


def _default_cu(T, device):
    return torch.tensor([0, T], dtype=torch.int32, device=device), [0, T]


def kda_forward(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens=None, *,
                cu_seqlens_host=None, scale=1.0, chunk=64, lower_bound=-5.0, eps=1e-6,
                seg_chunks=0, out=None):
    """O [T,H,V] of the KDA operator (no state saved for the backward)."""
    if cu_seqlens is None:
        cu_seqlens, cu_seqlens_host = _default_cu(q.shape[0], q.device)
    T, H, K, V, dt = _check_inputs(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens)
    prob = Problem(T, H, K, V, dt, _cu_host(cu_seqlens, cu_seqlens_host), chunk, scale,
                   lower_bound, eps, seg_chunks)
    lib = _lib.load()
    _raise(lib, prob.check(), "kda_fwd")
    o = torch.empty((T, H, V), dtype=dt, device=q.device) if out is None else out
    ws = torch.empty(prob.fwd_ws(), dtype=torch.uint8, device=q.device)
    st = lib.kda_fwd(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(raw_g), _ptr(raw_beta),
                     _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), _ptr(o), _ptr(ws),
                     ctypes.c_size_t(ws.numel()), _stream(q.device))
    _raise(lib, st, "kda_fwd")
    return o


def kda_backward(q, k, v, raw_g, raw_beta, A_log, dt_bias, dO, cu_seqlens=None, *,
                 cu_seqlens_host=None, scale=1.0, chunk=64, lower_bound=-5.0, eps=1e-6,
                 seg_chunks=0):
    """Gradients (dq, dk, dv, draw_g, draw_beta, dA_log, ddt_bias) of sum(O * dO),
    recomputing every intermediate from the inputs."""
    if cu_seqlens is None:
        cu_seqlens, cu_seqlens_host = _default_cu(q.shape[0], q.device)
    T, H, K, V, dt = _check_inputs(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens,
                                   extra=[("dO", (dO, tuple(v.shape), v.dtype))])
    prob = Problem(T, H, K, V, dt, _cu_host(cu_seqlens, cu_seqlens_host), chunk, scale,
                   lower_bound, eps, seg_chunks)
    lib = _lib.load()
    _raise(lib, prob.check(), "kda_bwd")
    dev = q.device
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dg = torch.empty_like(raw_g)
    db = torch.empty_like(raw_beta)
    dA = torch.empty((H,), dtype=torch.float32, device=dev)
    ddt = torch.empty((H, K), dtype=torch.float32, device=dev)
    ws = torch.empty(prob.bwd_ws(), dtype=torch.uint8, device=dev)
    st = lib.kda_bwd(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(raw_g), _ptr(raw_beta),
                     _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), _ptr(dO), _ptr(dq),
                     _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dA), _ptr(ddt), _ptr(ws),
                     ctypes.c_size_t(ws.numel()), _stream(dev))
    _raise(lib, st, "kda_bwd")
    return dq, dk, dv, dg, db, dA, ddt


def kda_prologue(q, k, raw_g, raw_beta, A_log, dt_bias, cu_seqlens=None, *,
                 cu_seqlens_host=None, scale=1.0, chunk=64, lower_bound=-5.0, eps=1e-6):
    """fp32 (qh, kh, beta, gcum) of the prologue step alone."""
    if cu_seqlens is None:
        cu_seqlens, cu_seqlens_host = _default_cu(q.shape[0], q.device)
    T, H, K, V, dt = _check_inputs(q, k, q, raw_g, raw_beta, A_log, dt_bias, cu_seqlens)
    prob = Problem(T, H, K, K, dt, _cu_host(cu_seqlens, cu_seqlens_host), chunk, scale,
                   lower_bound, eps)
    lib = _lib.load()
    _raise(lib, prob.check(), "kda_prologue")
    dev = q.device
    qh = torch.empty((T, H, K), dtype=torch.float32, device=dev)
    kh = torch.empty_like(qh)
    gc = torch.empty_like(qh)
    be = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(256, int(lib.kda_prologue_workspace_bytes(prob.ref))),
                     dtype=torch.uint8, device=dev)
    st = lib.kda_prologue(prob.ref, _ptr(q), _ptr(k), _ptr(raw_g), _ptr(raw_beta), _ptr(A_log),
                          _ptr(dt_bias), _ptr(cu_seqlens), _ptr(qh), _ptr(kh), _ptr(be),
                          _ptr(gc), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
    _raise(lib, st, "kda_prologue")
    return qh, kh, be, gc


class KDAFunction(torch.autograd.Function):
    """Autograd wrapper: saves references to the caller's inputs only."""

    @staticmethod
    def forward(ctx, q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens, cu_host, opts):
        ctx.save_for_backward(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens)
        ctx.cu_host = cu_host
        ctx.opts = opts
        return kda_forward(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens,
                           cu_seqlens_host=cu_host, **opts)

    @staticmethod
    def backward(ctx, dO):
        q, k, v, raw_g, raw_beta, A_log, dt_bias, cu = ctx.saved_tensors
        grads = kda_backward(q, k, v, raw_g, raw_beta, A_log, dt_bias, dO.contiguous(), cu,
                             cu_seqlens_host=ctx.cu_host, **ctx.opts)
        return (*grads, None, None, None)


def kda(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens=None, *, cu_seqlens_host=None,
        scale=1.0, chunk=64, lower_bound=-5.0, eps=1e-6, seg_chunks=0):
    """Differentiable KDA operator; returns O [T,H,V]."""
    if cu_seqlens is None:
        cu_seqlens, cu_seqlens_host = _default_cu(q.shape[0], q.device)
    cu_host = _cu_host(cu_seqlens, cu_seqlens_host)
    opts = dict(scale=scale, chunk=chunk, lower_bound=lower_bound, eps=eps, seg_chunks=seg_chunks)
    return KDAFunction.apply(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens, cu_host, opts)
