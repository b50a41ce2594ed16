"""ctypes view of the C ABI in ``include/kda.h`` (``_build/libkda.so``).

Loading fails loudly when the library has not been built: there is no CPU or
PyTorch fallback for any step of the operator.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_build", "libkda.so")

KDA_OK, KDA_ERR_INVALID, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(5)
KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_SIGMOID_BOUND, KDA_GATE_SOFTPLUS_CLAMP, KDA_GATE_PER_HEAD = 0, 1, 16

# Every function the header declares (checked against include/kda.h by the tests).
EXPORTS = ("kda_fwd_workspace_bytes", "kda_bwd_workspace_bytes", "kda_check_problem",
           "kda_prologue_workspace_bytes", "kda_prologue", "kda_fwd", "kda_bwd",
           "kda_checkpoint_bytes", "kda_bwd_segment_chunks", "kda_fwd_ex", "kda_bwd_ex",
           "kda_profile_begin", "kda_profile_end", "kda_kernel_name", "kda_status_string",
           "kda_fwd_noalloc", "kda_gdn2_fwd", "kda_gdn2_bwd")
NOALLOC_SCRATCH_BYTES = 64 << 20  # KDA_NOALLOC_SCRATCH_BYTES
KERNEL_COUNT = 11


class KdaProblem(ctypes.Structure):
    _fields_ = [
        ("n_seqs", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("H", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("V", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("gate_mode", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("gate_lower_bound", ctypes.c_float),
        ("l2_eps", ctypes.c_float),
        ("seg_chunks", ctypes.c_int32),
        ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
    ]


class KdaStateIO(ctypes.Structure):
    _fields_ = [
        ("h0", ctypes.c_void_p),
        ("ht", ctypes.c_void_p),
        ("dht", ctypes.c_void_p),
        ("dh0", ctypes.c_void_p),
        ("ckpt", ctypes.c_void_p),
        ("ckpt_bytes", ctypes.c_size_t),
    ]


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            "the KDA HIP library is not built (%s); run `python -m "
            "recompute_kda_chunked_amd.build` or __graft_entry__.build()" % p)
    lib = ctypes.CDLL(p)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pp = ctypes.POINTER(KdaProblem)
    lib.kda_fwd_workspace_bytes.argtypes = [pp]
    lib.kda_fwd_workspace_bytes.restype = sz
    lib.kda_bwd_workspace_bytes.argtypes = [pp]
    lib.kda_bwd_workspace_bytes.restype = sz
    lib.kda_prologue_workspace_bytes.argtypes = [pp]
    lib.kda_prologue_workspace_bytes.restype = sz
    lib.kda_check_problem.argtypes = [pp]
    lib.kda_check_problem.restype = ctypes.c_int
    lib.kda_prologue.argtypes = [pp] + [vp] * 11 + [vp, sz, vp]
    lib.kda_prologue.restype = ctypes.c_int
    lib.kda_fwd.argtypes = [pp] + [vp] * 9 + [vp, sz, vp]
    lib.kda_fwd.restype = ctypes.c_int
    lib.kda_bwd.argtypes = [pp] + [vp] * 16 + [vp, sz, vp]
    lib.kda_bwd.restype = ctypes.c_int
    iop = ctypes.POINTER(KdaStateIO)
    lib.kda_checkpoint_bytes.argtypes = [pp]
    lib.kda_checkpoint_bytes.restype = sz
    lib.kda_bwd_segment_chunks.argtypes = [pp]
    lib.kda_bwd_segment_chunks.restype = ctypes.c_int32
    lib.kda_fwd_ex.argtypes = [pp] + [vp] * 9 + [iop, vp, sz, vp]
    lib.kda_fwd_ex.restype = ctypes.c_int
    lib.kda_bwd_ex.argtypes = [pp] + [vp] * 16 + [iop, vp, sz, vp]
    lib.kda_bwd_ex.restype = ctypes.c_int
    lib.kda_gdn2_fwd.argtypes = [pp] + [vp] * 10 + [vp, sz, vp]
    lib.kda_gdn2_fwd.restype = ctypes.c_int
    lib.kda_gdn2_bwd.argtypes = [pp] + [vp] * 18 + [vp, sz, vp]
    lib.kda_gdn2_bwd.restype = ctypes.c_int
    lib.kda_fwd_noalloc.argtypes = [pp] + [vp] * 9 + [vp]
    lib.kda_fwd_noalloc.restype = ctypes.c_int
    lib.kda_profile_begin.argtypes = []
    lib.kda_profile_begin.restype = ctypes.c_int
    lib.kda_profile_end.argtypes = [ctypes.POINTER(ctypes.c_int32),
                                    ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
    lib.kda_profile_end.restype = ctypes.c_int
    lib.kda_kernel_name.argtypes = [ctypes.c_int]
    lib.kda_kernel_name.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def status_text(lib, status: int) -> str:
    return lib.kda_status_string(status).decode()


def profile_begin() -> None:
    load().kda_profile_begin()


def profile_end() -> dict:
    """{kernel name: (launches, total ms, (chunk, head) units)} since
    profile_begin() on this thread."""
    lib = load()
    n = KERNEL_COUNT
    launches = (ctypes.c_int32 * n)()
    ms = (ctypes.c_double * n)()
    units = (ctypes.c_int64 * n)()
    st = lib.kda_profile_end(launches, ms, units, n)
    if st != KDA_OK:
        raise RuntimeError("kda_profile_end: " + status_text(lib, st))
    return {lib.kda_kernel_name(k).decode(): (int(launches[k]), float(ms[k]), int(units[k]))
            for k in range(n)}
