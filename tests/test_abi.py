"""C ABI checks that need no GPU: the library loads, exports every function
include/kda.h declares, and rejects bad problems on the host before any HIP
call (null pointers, bad sizes, bad cu_seqlens, unsupported shapes,
workspace too small)."""
import ctypes
import os
import re

import pytest

from recompute_kda_chunked_amd import _lib
from recompute_kda_chunked_amd.ops import Problem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from recompute_kda_chunked_amd import build
        build.build()
    return _lib.load()


def header_functions():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert header_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_function(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def good(**kw):
    args = dict(T=300, H=4, K=128, V=128, dtype=_lib.KDA_BF16, cu_host=[0, 100, 100, 300], chunk=64)
    args.update(kw)
    return Problem(**args)


def test_valid_problem_and_workspace_sizes(lib):
    p = good()
    assert p.check() == _lib.KDA_OK
    assert p.fwd_ws() > 0 and p.bwd_ws() > 0
    # the backward workspace shrinks with the streaming segment
    small = good(seg_chunks=1)
    assert small.check() == _lib.KDA_OK
    assert small.bwd_ws() < p.bwd_ws()


@pytest.mark.parametrize("kw,code", [
    (dict(cu_host=[0, 100, 50, 300]), _lib.KDA_ERR_INVALID),      # decreasing
    (dict(cu_host=[1, 100, 300]), _lib.KDA_ERR_INVALID),          # does not start at 0
    (dict(cu_host=[0, 100, 299]), _lib.KDA_ERR_INVALID),          # does not end at T
    (dict(H=0), _lib.KDA_ERR_INVALID),
    (dict(T=0, cu_host=[0, 0]), _lib.KDA_ERR_INVALID),
    (dict(lower_bound=1.0), _lib.KDA_ERR_INVALID),
    (dict(lower_bound=float("nan")), _lib.KDA_ERR_INVALID),
    (dict(lower_bound=-10.0), _lib.KDA_ERR_UNSUPPORTED),             # exp(15*10) overflows fp32
    (dict(lower_bound=-6.0), _lib.KDA_ERR_UNSUPPORTED),
    (dict(lower_bound=-10.0, dtype=_lib.KDA_F32, K=64, V=64), _lib.KDA_ERR_UNSUPPORTED),
    (dict(eps=-1.0), _lib.KDA_ERR_INVALID),
    (dict(seg_chunks=-2), _lib.KDA_ERR_INVALID),
    (dict(K=96, V=96), _lib.KDA_ERR_UNSUPPORTED),
    (dict(K=128, V=64), _lib.KDA_ERR_UNSUPPORTED),
    (dict(chunk=16), _lib.KDA_ERR_UNSUPPORTED),                    # bf16 needs C >= 32
    (dict(chunk=48), _lib.KDA_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.KDA_ERR_UNSUPPORTED),
    (dict(gate_mode=2), _lib.KDA_ERR_UNSUPPORTED),
    (dict(gate_mode=2 | _lib.KDA_GATE_PER_HEAD), _lib.KDA_ERR_UNSUPPORTED),
    (dict(gate_mode=32), _lib.KDA_ERR_UNSUPPORTED),
])
def test_bad_problems_are_rejected(lib, kw, code):
    p = good(**kw)
    assert p.check() == code
    assert p.fwd_ws() == 0 and p.bwd_ws() == 0
    nul = ctypes.c_void_p(0)
    assert lib.kda_fwd(p.ref, *([nul] * 9), nul, ctypes.c_size_t(0), nul) == code


@pytest.mark.parametrize("lb", [-5.0, -5.9, -0.5])
def test_gate_bounds_within_the_finite_range_are_accepted(lib, lb):
    assert good(lower_bound=lb).check() == _lib.KDA_OK
    assert good(lower_bound=lb, dtype=_lib.KDA_F32, K=64, V=64).check() == _lib.KDA_OK


@pytest.mark.parametrize("mode", [0, 1])
def test_per_head_gate_flag_is_accepted(lib, mode):
    p = good(gate_mode=mode | _lib.KDA_GATE_PER_HEAD)
    assert p.check() == _lib.KDA_OK
    assert p.fwd_ws() == good(gate_mode=mode).fwd_ws() > 0


def test_null_pointers_and_small_workspace_rejected_before_any_launch(lib):
    p = good()
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    assert lib.kda_fwd(p.ref, *([nul] * 9), nul, ctypes.c_size_t(0), nul) == _lib.KDA_ERR_INVALID
    args = [fake] * 9
    assert lib.kda_fwd(p.ref, *args, fake, ctypes.c_size_t(p.fwd_ws() - 1), nul) == _lib.KDA_ERR_WORKSPACE
    args = [fake] * 16
    assert lib.kda_bwd(p.ref, *args, fake, ctypes.c_size_t(p.bwd_ws() - 1), nul) == _lib.KDA_ERR_WORKSPACE
    args[4] = nul
    assert lib.kda_bwd(p.ref, *args, fake, ctypes.c_size_t(p.bwd_ws()), nul) == _lib.KDA_ERR_INVALID
    assert lib.kda_check_problem(None) == _lib.KDA_ERR_INVALID


def test_status_strings(lib):
    for code in range(5):
        assert len(_lib.status_text(lib, code)) > 0


def test_checkpoint_queries_follow_the_backward_segments(lib):
    p = good(seg_chunks=1)  # chunks: 2 + 0 + 4 = 6 segments of one chunk
    slot = 4 * 128 * 128 * 4
    assert lib.kda_bwd_segment_chunks(p.ref) == 1
    assert lib.kda_checkpoint_bytes(p.ref) == 6 * slot
    q = good(seg_chunks=4)
    assert lib.kda_bwd_segment_chunks(q.ref) == 4
    assert lib.kda_checkpoint_bytes(q.ref) == 2 * slot
    bad = good(H=0)
    assert lib.kda_bwd_segment_chunks(bad.ref) == 0 and lib.kda_checkpoint_bytes(bad.ref) == 0


def test_checkpoints_of_a_plan_by_windows(lib):
    # four sequences of five 64-token chunks, at most 8 chunks per segment:
    # runs of the chunk order would give the scans a chain of 5 + 5 + 4
    # chunks over three segments, windows of 2 chunks of every sequence one
    # of 2 + 2 + 1, so the backward takes windows; every sequence then
    # crosses two window starts, each with a checkpoint
    p = good(T=1280, cu_host=[0, 320, 640, 960, 1280], seg_chunks=8)
    slot = 4 * 128 * 128 * 4
    assert lib.kda_bwd_segment_chunks(p.ref) == 2
    assert lib.kda_checkpoint_bytes(p.ref) == 4 * 2 * slot
    # one long and one short sequence (20 + 1 chunks): windows of 3 chunks
    # would leave the chain at 20, so the runs of 4 chunks of the chunk
    # order stay, one checkpoint slot per segment
    q = good(T=1280 + 64, cu_host=[0, 1280, 1344], seg_chunks=4)
    assert lib.kda_bwd_segment_chunks(q.ref) == 4
    assert lib.kda_checkpoint_bytes(q.ref) == 6 * slot
    # a single sequence: runs of the given length
    r = good(T=1280, cu_host=[0, 1280], seg_chunks=6)  # 20 chunks
    assert lib.kda_bwd_segment_chunks(r.ref) == 6
    assert lib.kda_checkpoint_bytes(r.ref) == 4 * slot


def test_windows_only_where_their_states_fit(lib):
    # 300 sequences of 7 chunks at H16, D128, at most 600 chunks per segment:
    # windows of 2 chunks would shorten the scans' chain (7 chunks in all,
    # against 7 in each of the 4 chunk-order segments), but every sequence
    # would cross three window starts,
    # so the backward would hold 900 checkpoint and 600 carry states of 1 MiB
    # on top of its operands: the plan stays in chunk order, one checkpoint
    # slot per segment
    lens = [448] * 300
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    p = good(T=cu[-1], H=16, cu_host=cu, seg_chunks=600)
    slot = 16 * 128 * 128 * 4
    assert lib.kda_bwd_segment_chunks(p.ref) == 600
    assert lib.kda_checkpoint_bytes(p.ref) == 4 * slot
    # the same batch at H2, D64: the states are small and windows are taken
    q = good(T=cu[-1], H=2, K=64, V=64, cu_host=cu, seg_chunks=600)
    assert lib.kda_bwd_segment_chunks(q.ref) == 2
    assert lib.kda_checkpoint_bytes(q.ref) == 300 * 3 * 2 * 64 * 64 * 4


def test_state_io_validation_before_any_launch(lib):
    p = good(seg_chunks=1)
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    io = _lib.KdaStateIO()
    io.ckpt = 0x2000
    io.ckpt_bytes = lib.kda_checkpoint_bytes(p.ref) - 1
    assert lib.kda_fwd_ex(p.ref, *([fake] * 9), ctypes.byref(io), fake,
                          ctypes.c_size_t(p.fwd_ws()), nul) == _lib.KDA_ERR_WORKSPACE
    assert lib.kda_bwd_ex(p.ref, *([fake] * 16), ctypes.byref(io), fake,
                          ctypes.c_size_t(p.bwd_ws()), nul) == _lib.KDA_ERR_WORKSPACE
    args = [fake] * 16
    args[9] = nul  # dq
    assert lib.kda_bwd_ex(p.ref, *args, None, fake, ctypes.c_size_t(p.bwd_ws()),
                          nul) == _lib.KDA_ERR_INVALID


def test_no_fallback_without_the_library(monkeypatch, tmp_path):
    # a missing library is an error, never a silent CPU or PyTorch path
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()


def test_host_tensors_are_refused():
    import torch
    from recompute_kda_chunked_amd import KdaError, kda_forward
    T, H, D = 8, 1, 64
    x = {n: torch.zeros((T, H, D)) for n in ("q", "k", "v", "raw_g")}
    with pytest.raises(KdaError, match="GPU"):
        kda_forward(x["q"], x["k"], x["v"], x["raw_g"], torch.zeros((T, H)), torch.zeros(H),
                    torch.zeros((H, D)), torch.tensor([0, T], dtype=torch.int32),
                    cu_seqlens_host=[0, T])


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    # one chunk of every head plus the two state carry slots must fit the
    # 64 MiB scratch: at H=512, D=128 the carry slots alone take 64 MiB. The
    # check is on the host, before any HIP call (the pointers are never
    # dereferenced).
    fake = ctypes.c_void_p(0x1000)
    nul = ctypes.c_void_p(0)
    big = good(H=512, T=64, cu_host=[0, 64])
    assert big.check() == _lib.KDA_OK
    assert lib.kda_fwd_noalloc(big.ref, *([fake] * 9), nul) == _lib.KDA_ERR_WORKSPACE
    assert lib.kda_fwd_noalloc(good().ref, *([nul] * 9), nul) == _lib.KDA_ERR_INVALID
    assert lib.kda_fwd_noalloc(good(H=0).ref, *([fake] * 9), nul) == _lib.KDA_ERR_INVALID


def test_gdn2_entry_points_validate_before_any_launch(lib):
    fake = ctypes.c_void_p(0x1000)
    nul = ctypes.c_void_p(0)
    p = good()
    # null gate pointers, then the unbuilt combinations
    args = [fake] * 10
    args[5] = nul  # raw_w
    assert lib.kda_gdn2_fwd(p.ref, *args, fake, ctypes.c_size_t(p.fwd_ws()), nul) == _lib.KDA_ERR_INVALID
    ph = good(gate_mode=_lib.KDA_GATE_PER_HEAD)
    assert lib.kda_gdn2_fwd(ph.ref, *([fake] * 10), fake, ctypes.c_size_t(ph.fwd_ws()),
                            nul) == _lib.KDA_ERR_UNSUPPORTED
    f64 = good(dtype=_lib.KDA_F32, K=64, V=64, chunk=64)
    assert f64.check() == _lib.KDA_OK  # KDA is built there
    assert lib.kda_gdn2_bwd(f64.ref, *([fake] * 18), fake, ctypes.c_size_t(f64.bwd_ws()),
                            nul) == _lib.KDA_ERR_UNSUPPORTED
    args = [fake] * 18
    args[15] = nul  # draw_w
    assert lib.kda_gdn2_bwd(p.ref, *args, fake, ctypes.c_size_t(p.bwd_ws()), nul) == _lib.KDA_ERR_INVALID
    assert lib.kda_gdn2_fwd(p.ref, *([fake] * 10), fake, ctypes.c_size_t(p.fwd_ws() - 1),
                            nul) == _lib.KDA_ERR_WORKSPACE
