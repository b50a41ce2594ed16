"""FP64 CPU oracle for the KDA operator (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the GPU path
(``recompute_kda_chunked_amd``) and never imports it.

``kda_oracle.c`` holds the token-by-token recurrence and its hand-derived
reverse sweep (see its header for the equations and the passages of the pages
they follow); ``gdn2_oracle.c`` the same for the gated delta rule with a
per-channel erase gate and a per-channel write gate (GDN-2), written
separately so that the tests can compare the two. This module only marshals
numpy arrays into them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "libkda_oracle.so")
_GDN2_SRC = os.path.join(_HERE, "gdn2_oracle.c")
_GDN2_LIB_PATH = os.path.join(_BUILD, "libgdn2_oracle.so")

GATE_SIGMOID_BOUND = 0  # g = L * sigmoid(exp(A_log) * (raw_g + dt_bias))
GATE_SOFTPLUS_CLAMP = 1  # g = max(L, -exp(A_log) * softplus(raw_g + dt_bias))


def _gcc(src: str, out: str, extra_flags=()) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           *extra_flags, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(extra_flags: tuple[str, ...] = (), out_path: str | None = None) -> str:
    """Compile the oracles with gcc (OpenMP, -O3, no host-specific ISA so the
    libraries run on any x86-64 host). Returns the KDA library path."""
    if out_path is None:
        _gcc(_GDN2_SRC, _GDN2_LIB_PATH, extra_flags)
    return _gcc(_SRC, out_path or _LIB_PATH, extra_flags)


_lib_cache: dict[str, ctypes.CDLL] = {}


def _load(path: str | None = None) -> ctypes.CDLL:
    path = path or _LIB_PATH
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        if path != _LIB_PATH:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    f = lib.kda_oracle_ex
    dp = ctypes.POINTER(ctypes.c_double)
    f.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                  ctypes.c_double, ctypes.c_int] + [dp] * 8 + [dp] * 8 + [dp] * 4 + [ctypes.c_int]
    f.restype = ctypes.c_int
    _lib_cache[path] = lib
    return lib


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: upcast exactly to float64 on the host
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _widen_gate(raw_g, dt_bias, T, H, K):
    """Scalar gate per head and token (raw_g [T,H], dt_bias [H]): the Gated
    DeltaNet form that FLA's chunk_gdn computes ("KDA at the production
    shape...", sections 1.1 and 1.2: KDA differs from it only by a decay per
    key channel). It is the per-channel operator with all K channels of the
    gate equal, so the inputs are repeated over K here."""
    if raw_g.ndim != 2:
        return raw_g, dt_bias, False
    if raw_g.shape != (T, H) or dt_bias.shape != (H,):
        raise ValueError("a per-head gate takes raw_g [T,H] and dt_bias [H]")
    return (np.repeat(raw_g[:, :, None], K, axis=2), np.repeat(dt_bias[:, None], K, axis=1),
            True)


def kda(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens=None, dO=None,
        scale: float = 1.0, lower_bound: float = -5.0, eps: float = 1e-6,
        gate_mode: int = GATE_SIGMOID_BOUND, n_threads: int = 0,
        lib_path: str | None = None, h0=None, dht=None, final_state: bool = False) -> dict:
    """Run the oracle. Shapes: q,k,raw_g [T,H,K]; v [T,H,V]; raw_beta [T,H];
    A_log [H]; dt_bias [H,K]; or, for a gate per head, raw_g [T,H] and
    dt_bias [H] (draw_g and ddt_bias then take those shapes too); cu_seqlens
    [N+1] (defaults to one sequence);
    dO [T,H,V] or None (forward only); h0 [N,H,K,V] or None (each sequence
    starts from zero); dht [N,H,K,V] or None (no loss on the final state).

    Returns a dict of float64 arrays: ``o``; ``ht`` (the final state of every
    sequence) when final_state, h0 or dht is given; and, when dO is given,
    ``dq, dk, dv, draw_g, draw_beta, dA_log, ddt_bias`` plus ``dh0`` when h0
    is given.
    """
    q, k, v, raw_g, raw_beta = map(_f64, (q, k, v, raw_g, raw_beta))
    A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    T, H, K = q.shape
    V = v.shape[2]
    raw_g, dt_bias, per_head = _widen_gate(raw_g, dt_bias, T, H, K)
    if k.shape != (T, H, K) or raw_g.shape != (T, H, K) or v.shape[:2] != (T, H):
        raise ValueError("shape mismatch among q, k, v, raw_g")
    if raw_beta.shape != (T, H) or A_log.shape != (H,) or dt_bias.shape != (H, K):
        raise ValueError("shape mismatch among raw_beta, A_log, dt_bias")
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64))
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be non-decreasing from 0 to T")
    n = len(cu) - 1
    o = np.zeros((T, H, V))
    out = {"o": o}
    grads = [None] * 8
    if dO is not None:
        dO = _f64(dO)
        if dO.shape != (T, H, V):
            raise ValueError("dO shape mismatch")
        out.update(dq=np.zeros((T, H, K)), dk=np.zeros((T, H, K)), dv=np.zeros((T, H, V)),
                   draw_g=np.zeros((T, H, K)), draw_beta=np.zeros((T, H)),
                   dA_log=np.zeros(H), ddt_bias=np.zeros((H, K)))
        grads = [out[n_] for n_ in ("dq", "dk", "dv", "draw_g", "draw_beta", "dA_log", "ddt_bias")]
    sshape = (n, H, K, V)
    if h0 is not None:
        h0 = _f64(h0)
        if h0.shape != sshape:
            raise ValueError("h0 must be [N,H,K,V]")
    if dht is not None:
        dht = _f64(dht)
        if dht.shape != sshape:
            raise ValueError("dht must be [N,H,K,V]")
    ht = np.zeros(sshape) if (final_state or h0 is not None or dht is not None) else None
    if ht is not None:
        out["ht"] = ht
    dh0 = np.zeros(sshape) if (dO is not None and h0 is not None) else None
    if dh0 is not None:
        out["dh0"] = dh0
    lib = _load(lib_path)
    rc = lib.kda_oracle_ex(n, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, K, V,
                           float(scale), float(lower_bound), float(eps), int(gate_mode),
                           _ptr(q), _ptr(k), _ptr(v), _ptr(raw_g), _ptr(raw_beta), _ptr(A_log),
                           _ptr(dt_bias), _ptr(dO), _ptr(o), *[_ptr(g) for g in grads[:7]],
                           _ptr(h0), _ptr(ht), _ptr(dht), _ptr(dh0), int(n_threads))
    if rc != 0:
        raise RuntimeError("kda_oracle failed with status %d" % rc)
    if per_head and dO is not None:
        # each per-head value feeds all K channels: its gradient is their sum
        out["draw_g"] = out["draw_g"].sum(axis=2)
        out["ddt_bias"] = out["ddt_bias"].sum(axis=1)
    return out


def _cu(cu_seqlens, T):
    if cu_seqlens is None:
        return np.array([0, T], dtype=np.int64)
    cu = np.ascontiguousarray(np.asarray(
        cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64))
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be non-decreasing from 0 to T")
    return cu


def gdn2(q, k, v, raw_g, raw_b, raw_w, A_log, dt_bias, cu_seqlens=None, dO=None,
         scale: float = 1.0, lower_bound: float = -5.0, eps: float = 1e-6,
         gate_mode: int = GATE_SIGMOID_BOUND, n_threads: int = 0,
         lib_path: str | None = None) -> dict:
    """GDN-2 oracle (gdn2_oracle.c): the gated delta rule with a per-channel
    erase gate b = sigmoid(raw_b) [T,H,K] and write gate w = sigmoid(raw_w)
    [T,H,V] in place of KDA's scalar beta. Shapes as for kda(); returns a
    dict of float64 arrays: ``o`` and, when dO is given, ``dq, dk, dv,
    draw_g, draw_b, draw_w, dA_log, ddt_bias``."""
    q, k, v, raw_g, raw_b, raw_w = map(_f64, (q, k, v, raw_g, raw_b, raw_w))
    A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    T, H, K = q.shape
    V = v.shape[2]
    if (k.shape != (T, H, K) or raw_g.shape != (T, H, K) or raw_b.shape != (T, H, K)
            or v.shape != (T, H, V) or raw_w.shape != (T, H, V)):
        raise ValueError("shape mismatch among q, k, v, raw_g, raw_b, raw_w")
    if A_log.shape != (H,) or dt_bias.shape != (H, K):
        raise ValueError("shape mismatch among A_log, dt_bias")
    cu = _cu(cu_seqlens, T)
    out = {"o": np.zeros((T, H, V))}
    names = ("dq", "dk", "dv", "draw_g", "draw_b", "draw_w", "dA_log", "ddt_bias")
    grads = [None] * 8
    if dO is not None:
        dO = _f64(dO)
        if dO.shape != (T, H, V):
            raise ValueError("dO shape mismatch")
        shapes = ((T, H, K), (T, H, K), (T, H, V), (T, H, K), (T, H, K), (T, H, V), (H,), (H, K))
        out.update({n_: np.zeros(s_) for n_, s_ in zip(names, shapes)})
        grads = [out[n_] for n_ in names]
    path = lib_path or _GDN2_LIB_PATH
    if path not in _lib_cache:
        if not os.path.exists(path):
            if path != _GDN2_LIB_PATH:
                raise FileNotFoundError(path)
            build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gdn2_oracle.argtypes = ([ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                     ctypes.c_double, ctypes.c_int] + [dp] * 9 + [dp] * 9
                                    + [ctypes.c_int])
        lib.gdn2_oracle.restype = ctypes.c_int
        _lib_cache[path] = lib
    rc = _lib_cache[path].gdn2_oracle(
        len(cu) - 1, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, K, V, float(scale),
        float(lower_bound), float(eps), int(gate_mode), _ptr(q), _ptr(k), _ptr(v), _ptr(raw_g),
        _ptr(raw_b), _ptr(raw_w), _ptr(A_log), _ptr(dt_bias), _ptr(dO), _ptr(out["o"]),
        *[_ptr(g) for g in grads], int(n_threads))
    if rc != 0:
        raise RuntimeError("gdn2_oracle failed with status %d" % rc)
    return out


def prologue(q, k, raw_g, raw_beta, A_log, dt_bias, cu_seqlens=None, chunk: int = 64,
             scale: float = 1.0, lower_bound: float = -5.0, eps: float = 1e-6,
             gate_mode: int = GATE_SIGMOID_BOUND) -> dict:
    """The prologue alone: qh, kh [T,H,K], beta [T,H] and gcum [T,H,K] (the
    cumulative gate restarted every ``chunk`` tokens of each sequence; a
    per-head gate, raw_g [T,H] and dt_bias [H], gives K equal channels)."""
    q, k, raw_g, raw_beta = map(_f64, (q, k, raw_g, raw_beta))
    A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    T, H, K = q.shape
    raw_g, dt_bias, _ = _widen_gate(raw_g, dt_bias, T, H, K)
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64))
    out = dict(qh=np.zeros((T, H, K)), kh=np.zeros((T, H, K)), beta=np.zeros((T, H)),
               gcum=np.zeros((T, H, K)))
    lib = _load()
    f = lib.kda_oracle_prologue
    dp = ctypes.POINTER(ctypes.c_double)
    f.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.c_int, ctypes.c_int,
                  ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_int,
                  ctypes.c_int] + [dp] * 10
    rc = f(len(cu) - 1, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, K, float(scale),
           float(lower_bound), float(eps), int(gate_mode), int(chunk), _ptr(q), _ptr(k),
           _ptr(raw_g), _ptr(raw_beta), _ptr(A_log), _ptr(dt_bias), _ptr(out["qh"]),
           _ptr(out["kh"]), _ptr(out["beta"]), _ptr(out["gcum"]))
    if rc != 0:
        raise RuntimeError("kda_oracle_prologue failed")
    return out
