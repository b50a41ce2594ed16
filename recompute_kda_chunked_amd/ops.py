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
    """Shapes, dtypes and placement; a raw_g of two dimensions selects the
    gate per head and token (raw_g [T,H], dt_bias [H])."""
    dev = q.device
    if dev.type != "cuda":
        raise KdaError("inputs must be on a GPU device")
    T, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    if dt not in _DT:
        raise KdaError("dtype must be float32 or bfloat16")
    per_head = raw_g.dim() == 2
    gk = (T, H) if per_head else (T, H, K)
    want = {"q": (q, (T, H, K), dt), "k": (k, (T, H, K), dt), "v": (v, (T, H, V), dt),
            "raw_g": (raw_g, gk, dt), "raw_beta": (raw_beta, (T, H), dt),
            "A_log": (A_log, (H,), torch.float32), "dt_bias": (dt_bias, gk[1:], torch.float32),
            "cu_seqlens": (cu_seqlens, (cu_seqlens.shape[0],), torch.int32)}
    if raw_beta is None:  # GDN-2: the gates come in `extra`
        del want["raw_beta"]
    for name, (t, shape, dtype) in list(want.items()) + list(extra):
        if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
            raise KdaError("%s: expected shape %s dtype %s, got %s %s"
                           % (name, shape, dtype, tuple(t.shape), t.dtype))
        if t.device != dev or not t.is_contiguous() or t.data_ptr() % 16:
            raise KdaError("%s must be contiguous, 16-byte aligned and on %s" % (name, dev))
    return T, H, K, V, dt, per_head


def _gate_flags(gate_mode, per_head):
    return int(gate_mode) | (_lib.KDA_GATE_PER_HEAD if per_head else 0)


def _cu_host(cu_seqlens, cu_seqlens_host):
    if cu_seqlens_host is not None:
        return [int(x) for x in cu_seqlens_host]
    return [int(x) for x in cu_seqlens.tolist()]  # device-to-host copy (synchronises)


def _default_cu(T, device):
    return torch.tensor([0, T], dtype=torch.int32, device=device), [0, T]


class Checkpoints:
    """States a forward saved at the starts of the backward's segments (fp32,
    device) and the segment length, in chunks, they were taken at."""

    def __init__(self, states: torch.Tensor, seg_chunks: int):
        self.states = states
        self.seg_chunks = int(seg_chunks)


def _state_io(h0=None, ht=None, dht=None, dh0=None, ckpt=None):
    io = _lib.KdaStateIO()
    io.h0 = h0.data_ptr() if h0 is not None else None
    io.ht = ht.data_ptr() if ht is not None else None
    io.dht = dht.data_ptr() if dht is not None else None
    io.dh0 = dh0.data_ptr() if dh0 is not None else None
    if ckpt is not None:
        io.ckpt = ckpt.data_ptr()
        io.ckpt_bytes = ckpt.numel() * ckpt.element_size()
    return io


def _check_state(name, t, shape, dev):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != torch.float32:
        raise KdaError("%s: expected shape %s float32, got %s %s"
                       % (name, tuple(shape), tuple(t.shape), t.dtype))
    if t.device != dev or not t.is_contiguous() or t.data_ptr() % 16:
        raise KdaError("%s must be contiguous, 16-byte aligned and on %s" % (name, dev))


def kda_forward(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens=None, *,
                cu_seqlens_host=None, scale=1.0, chunk=64, lower_bound=-5.0, eps=1e-6,
                seg_chunks=0, gate_mode=_lib.KDA_GATE_SIGMOID_BOUND, initial_state=None,
                output_final_state=False, save_checkpoints=False, out=None):
    """O [T,H,V] of the KDA operator. raw_g [T,H] with dt_bias [H] gives one
    scalar gate per head and token (the Gated DeltaNet form).

    initial_state: fp32 [N,H,K,V] state each sequence starts from (zero when
    None). With output_final_state or save_checkpoints the result is
    (O, ht, checkpoints): ht the fp32 [N,H,K,V] state after each sequence
    (None unless output_final_state), checkpoints a Checkpoints for
    kda_backward (None unless save_checkpoints)."""
    if cu_seqlens is None:
        cu_seqlens, cu_seqlens_host = _default_cu(q.shape[0], q.device)
    T, H, K, V, dt, ph = _check_inputs(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens)
    cu_host = _cu_host(cu_seqlens, cu_seqlens_host)
    N = len(cu_host) - 1
    _check_state("initial_state", initial_state, (N, H, K, V), q.device)
    prob = Problem(T, H, K, V, dt, cu_host, chunk, scale, lower_bound, eps, seg_chunks,
                   _gate_flags(gate_mode, ph))
    lib = _lib.load()
    _raise(lib, prob.check(), "kda_fwd")
    dev = q.device
    o = torch.empty((T, H, V), dtype=dt, device=dev) if out is None else out
    ht = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if output_final_state else None
    ck = None
    if save_checkpoints:
        nbytes = int(lib.kda_checkpoint_bytes(prob.ref))
        ck = Checkpoints(torch.empty(max(nbytes, 256) // 4, dtype=torch.float32, device=dev),
                         lib.kda_bwd_segment_chunks(prob.ref))
    io = _state_io(h0=initial_state, ht=ht, ckpt=ck.states if ck is not None else None)
    ws = torch.empty(prob.fwd_ws(), dtype=torch.uint8, device=dev)
    st = lib.kda_fwd_ex(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(raw_g), _ptr(raw_beta),
                        _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), _ptr(o), ctypes.byref(io),
                        _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
    _raise(lib, st, "kda_fwd")
    if output_final_state or save_checkpoints:
        return o, ht, ck
    return o


def kda_forward_noalloc(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens, o, *,
                        cu_seqlens_host, scale=1.0, chunk=64, lower_bound=-5.0, eps=1e-6,
                        gate_mode=_lib.KDA_GATE_SIGMOID_BOUND):
    """kda_fwd_noalloc: O written into the caller's `o` [T,H,V] with the
    library's own device scratch (no allocation by the library, none here
    either: the host copy of cu_seqlens must be given)."""
    T, H, K, V, dt, ph = _check_inputs(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens,
                                       extra=[("o", (o, tuple(v.shape), v.dtype))])
    prob = Problem(T, H, K, V, dt, [int(c) for c in cu_seqlens_host], chunk, scale, lower_bound,
                   eps, 0, _gate_flags(gate_mode, ph))
    lib = _lib.load()
    st = lib.kda_fwd_noalloc(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(raw_g), _ptr(raw_beta),
                             _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), _ptr(o),
                             _stream(q.device))
    _raise(lib, st, "kda_fwd_noalloc")
    return o


def kda_backward(q, k, v, raw_g, raw_beta, A_log, dt_bias, dO, cu_seqlens=None, *,
                 cu_seqlens_host=None, scale=1.0, chunk=64, lower_bound=-5.0, eps=1e-6,
                 seg_chunks=0, gate_mode=_lib.KDA_GATE_SIGMOID_BOUND, initial_state=None,
                 d_final_state=None, checkpoints=None):
    """Gradients (dq, dk, dv, draw_g, draw_beta, dA_log, ddt_bias, each shaped
    as its input) of
    sum(O * dO) + sum(ht * d_final_state), recomputing every chunk's
    intermediates from the inputs; dh0 is appended when initial_state is
    given. checkpoints: the forward's Checkpoints for the same problem (the
    backward then skips the pass that recomputes the segment states)."""
    if cu_seqlens is None:
        cu_seqlens, cu_seqlens_host = _default_cu(q.shape[0], q.device)
    T, H, K, V, dt, ph = _check_inputs(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens,
                                       extra=[("dO", (dO, tuple(v.shape), v.dtype))])
    cu_host = _cu_host(cu_seqlens, cu_seqlens_host)
    N = len(cu_host) - 1
    dev = q.device
    _check_state("initial_state", initial_state, (N, H, K, V), dev)
    _check_state("d_final_state", d_final_state, (N, H, K, V), dev)
    prob = Problem(T, H, K, V, dt, cu_host, chunk, scale, lower_bound, eps, seg_chunks,
                   _gate_flags(gate_mode, ph))
    lib = _lib.load()
    _raise(lib, prob.check(), "kda_bwd")
    if checkpoints is not None and lib.kda_bwd_segment_chunks(prob.ref) != checkpoints.seg_chunks:
        raise KdaError("checkpoints were saved at a segment of %d chunks; this backward "
                       "uses %d" % (checkpoints.seg_chunks, lib.kda_bwd_segment_chunks(prob.ref)))
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dg = torch.empty_like(raw_g)
    db = torch.empty_like(raw_beta)
    dA = torch.empty((H,), dtype=torch.float32, device=dev)
    ddt = torch.empty_like(dt_bias)
    dh0 = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) \
        if initial_state is not None else None
    io = _state_io(h0=initial_state, dht=d_final_state, dh0=dh0,
                   ckpt=checkpoints.states if checkpoints is not None else None)
    ws = torch.empty(prob.bwd_ws(), dtype=torch.uint8, device=dev)
    st = lib.kda_bwd_ex(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(raw_g), _ptr(raw_beta),
                        _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), _ptr(dO), _ptr(dq),
                        _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dA), _ptr(ddt),
                        ctypes.byref(io), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
    _raise(lib, st, "kda_bwd")
    if dh0 is not None:
        return dq, dk, dv, dg, db, dA, ddt, dh0
    return dq, dk, dv, dg, db, dA, ddt


def gdn2_forward(q, k, v, raw_g, raw_b, raw_w, A_log, dt_bias, cu_seqlens=None, *,
                 cu_seqlens_host=None, scale=1.0, chunk=64, lower_bound=-5.0, eps=1e-6,
                 seg_chunks=0, gate_mode=_lib.KDA_GATE_SIGMOID_BOUND):
    """O [T,H,V] of GDN-2: per-channel erase gate sigmoid(raw_b) [T,H,K] and
    write gate sigmoid(raw_w) [T,H,V] in place of KDA's beta (kda_gdn2_fwd)."""
    if cu_seqlens is None:
        cu_seqlens, cu_seqlens_host = _default_cu(q.shape[0], q.device)
    T, H, K, V, dt, ph = _check_inputs(
        q, k, v, raw_g, None, A_log, dt_bias, cu_seqlens,
        extra=[("raw_b", (raw_b, tuple(k.shape), q.dtype)), ("raw_w", (raw_w, tuple(v.shape), q.dtype))])
    prob = Problem(T, H, K, V, dt, _cu_host(cu_seqlens, cu_seqlens_host), chunk, scale,
                   lower_bound, eps, seg_chunks, _gate_flags(gate_mode, ph))
    lib = _lib.load()
    _raise(lib, prob.check(), "kda_gdn2_fwd")
    o = torch.empty((T, H, V), dtype=dt, device=q.device)
    ws = torch.empty(prob.fwd_ws(), dtype=torch.uint8, device=q.device)
    st = lib.kda_gdn2_fwd(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(raw_g), _ptr(raw_b),
                          _ptr(raw_w), _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), _ptr(o),
                          _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(q.device))
    _raise(lib, st, "kda_gdn2_fwd")
    return o


def gdn2_backward(q, k, v, raw_g, raw_b, raw_w, A_log, dt_bias, dO, cu_seqlens=None, *,
                  cu_seqlens_host=None, scale=1.0, chunk=64, lower_bound=-5.0, eps=1e-6,
                  seg_chunks=0, gate_mode=_lib.KDA_GATE_SIGMOID_BOUND):
    """(dq, dk, dv, draw_g, draw_b, draw_w, dA_log, ddt_bias) of
    sum(O * dO) for GDN-2 (kda_gdn2_bwd), each shaped as its input."""
    if cu_seqlens is None:
        cu_seqlens, cu_seqlens_host = _default_cu(q.shape[0], q.device)
    T, H, K, V, dt, ph = _check_inputs(
        q, k, v, raw_g, None, A_log, dt_bias, cu_seqlens,
        extra=[("raw_b", (raw_b, tuple(k.shape), q.dtype)), ("raw_w", (raw_w, tuple(v.shape), q.dtype)),
               ("dO", (dO, tuple(v.shape), v.dtype))])
    prob = Problem(T, H, K, V, dt, _cu_host(cu_seqlens, cu_seqlens_host), chunk, scale,
                   lower_bound, eps, seg_chunks, _gate_flags(gate_mode, ph))
    lib = _lib.load()
    _raise(lib, prob.check(), "kda_gdn2_bwd")
    dev = q.device
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg, db, dw = torch.empty_like(raw_g), torch.empty_like(raw_b), torch.empty_like(raw_w)
    dA = torch.empty((H,), dtype=torch.float32, device=dev)
    ddt = torch.empty_like(dt_bias)
    ws = torch.empty(prob.bwd_ws(), dtype=torch.uint8, device=dev)
    st = lib.kda_gdn2_bwd(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(raw_g), _ptr(raw_b),
                          _ptr(raw_w), _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), _ptr(dO),
                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dw), _ptr(dA),
                          _ptr(ddt), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
    _raise(lib, st, "kda_gdn2_bwd")
    return dq, dk, dv, dg, db, dw, dA, ddt


def kda_prologue(q, k, raw_g, raw_beta, A_log, dt_bias, cu_seqlens=None, *,
                 cu_seqlens_host=None, scale=1.0, chunk=64, lower_bound=-5.0, eps=1e-6,
                 gate_mode=_lib.KDA_GATE_SIGMOID_BOUND):
    """fp32 (qh, kh, beta, gcum) of the prologue step alone."""
    if cu_seqlens is None:
        cu_seqlens, cu_seqlens_host = _default_cu(q.shape[0], q.device)
    T, H, K, V, dt, ph = _check_inputs(q, k, q, raw_g, raw_beta, A_log, dt_bias, cu_seqlens)
    prob = Problem(T, H, K, K, dt, _cu_host(cu_seqlens, cu_seqlens_host), chunk, scale,
                   lower_bound, eps, gate_mode=_gate_flags(gate_mode, ph))
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
    """Autograd wrapper: saves references to the caller's inputs only (plus
    the segment-start states when opts["save_checkpoints"])."""

    @staticmethod
    def forward(ctx, q, k, v, raw_g, raw_beta, A_log, dt_bias, h0, cu_seqlens, cu_host, opts):
        ctx.set_materialize_grads(False)
        ctx.save_for_backward(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens, h0)
        ctx.cu_host = cu_host
        ctx.opts = {k_: v_ for k_, v_ in opts.items()
                    if k_ not in ("output_final_state", "save_checkpoints")}
        final = opts.get("output_final_state", False)
        res = kda_forward(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens,
                          cu_seqlens_host=cu_host, initial_state=h0, output_final_state=final,
                          save_checkpoints=opts.get("save_checkpoints", False), **ctx.opts)
        if isinstance(res, tuple):
            o, ht, ctx.ckpt = res
        else:
            o, ht, ctx.ckpt = res, None, None
        return (o, ht) if final else o

    @staticmethod
    def backward(ctx, dO, dht=None):
        q, k, v, raw_g, raw_beta, A_log, dt_bias, cu, h0 = ctx.saved_tensors
        dO = torch.zeros_like(v) if dO is None else dO.contiguous()
        dht = None if dht is None else dht.contiguous()
        grads = kda_backward(q, k, v, raw_g, raw_beta, A_log, dt_bias, dO, cu,
                             cu_seqlens_host=ctx.cu_host, initial_state=h0, d_final_state=dht,
                             checkpoints=ctx.ckpt, **ctx.opts)
        ctx.ckpt = None
        dh0 = grads[7] if h0 is not None else None
        return (*grads[:7], dh0, None, None, None)


def kda(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens=None, *, cu_seqlens_host=None,
        scale=1.0, chunk=64, lower_bound=-5.0, eps=1e-6, seg_chunks=0,
        gate_mode=_lib.KDA_GATE_SIGMOID_BOUND, initial_state=None, output_final_state=False,
        save_checkpoints=True):
    """Differentiable KDA operator; returns O [T,H,V], or (O, ht) with
    output_final_state. initial_state (fp32 [N,H,K,V]) is differentiable.
    save_checkpoints (default) keeps the states at the backward's segment
    starts (one fp32 [H,K,V] state per segment, when there is more than one)
    from the forward to the backward, which then skips one forward-direction
    pass; every chunk's w, u and h are still recomputed. False recomputes
    those states in the backward too."""
    if cu_seqlens is None:
        cu_seqlens, cu_seqlens_host = _default_cu(q.shape[0], q.device)
    cu_host = _cu_host(cu_seqlens, cu_seqlens_host)
    opts = dict(scale=scale, chunk=chunk, lower_bound=lower_bound, eps=eps, seg_chunks=seg_chunks,
                gate_mode=gate_mode, output_final_state=output_final_state,
                save_checkpoints=save_checkpoints)
    return KDAFunction.apply(q, k, v, raw_g, raw_beta, A_log, dt_bias, initial_state, cu_seqlens,
                             cu_host, opts)
