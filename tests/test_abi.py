"""CPU tests of the C ABI: libgdr.so loads, exports every function that
include/gdr.h declares, and rejects bad arguments on the host before any HIP
call (so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from gated_delta_rule_recurrence_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")


@pytest.fixture(scope="module")
def lib():
    if not _lib.LIB_PATH.exists():
        from gated_delta_rule_recurrence_amd import build
        build.build(verbose=False)
    return _lib.load()


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdr_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("gdr_forward", "gdr_backward", "gdr_checkpoint_bytes",
              "gdr_forward_workspace_bytes", "gdr_backward_workspace_bytes",
              "gdr_num_chunks", "gdr_strerror", "gdr_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", str(_lib.LIB_PATH)],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(gdr_\w+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"not exported: {missing}"
    for n in declared_functions():
        assert getattr(lib, n) is not None


def test_binding_covers_header():
    assert set(declared_functions()) == set(_lib._SIGNATURES)


def test_version_and_strerror(lib):
    assert re.fullmatch(r"\d+\.\d+\.\d+", lib.gdr_version().decode())
    for code in range(0, -14, -1):
        assert "unknown" not in _lib.strerror(code)
    assert "unknown" in _lib.strerror(-999)


def S(B=1, T=4, Hk=2, Hv=4, Dk=8, Dv=8, chunk=2, dtype=_lib.GDR_F32, decay=0):
    return _lib.make_shape(B, T, Hk, Hv, Dk, Dv, chunk, dtype, decay)


@pytest.mark.parametrize("shape,code", [
    (S(B=-1), -2), (S(T=-1), -2), (S(Hk=0), -2), (S(Hv=0), -2), (S(Dk=0), -2),
    (S(Dv=0), -2), (S(Hk=3, Hv=4), -3), (S(Dk=257), -4), (S(Dv=300), -4),
    (S(B=70000), -4), (S(chunk=0), -5), (S(chunk=2**30 + 1), -5), (S(dtype=2), -6),
    (S(dtype=-1), -6), (S(T=2**40), -7), (S(decay=2), -11), (S(decay=-1), -11),
])
def test_shape_errors(lib, shape, code):
    out = ctypes.c_size_t()
    assert lib.gdr_checkpoint_bytes(ctypes.byref(shape), ctypes.byref(out)) == code
    assert lib.gdr_backward_workspace_bytes(ctypes.byref(shape), ctypes.byref(out)) == code
    assert lib.gdr_forward_workspace_bytes(ctypes.byref(shape), ctypes.byref(out)) == code
    assert _lib.forward_raw(shape, *([0] * 10), 0, 0) == code


def test_null_shape(lib):
    out = ctypes.c_size_t()
    assert lib.gdr_checkpoint_bytes(None, ctypes.byref(out)) == -1
    assert lib.gdr_forward(None, *([None] * 11), 0, None) == -1
    assert lib.gdr_backward(None, *([None] * 16), 0, None) == -1


def test_null_out_pointer(lib):
    sh = S()
    assert lib.gdr_checkpoint_bytes(ctypes.byref(sh), None) == -1
    assert lib.gdr_num_chunks(ctypes.byref(sh), None) == -1


def _round256(x):
    return (x + 255) // 256 * 256


def _tile(C):
    """The kernels' tile: C up to 64, else C's largest divisor up to 64."""
    return C if C <= 64 else max(d for d in range(1, 65) if C % d == 0)


@pytest.mark.parametrize("B,T,Hk,Hv,Dk,Dv,C,bf16", [
    (1, 4, 2, 4, 8, 8, 2, 0), (1, 2048, 16, 64, 192, 128, 64, 0),
    (4, 8192, 16, 64, 192, 128, 64, 0), (2, 5, 1, 3, 7, 5, 64, 0), (1, 0, 1, 1, 4, 4, 8, 0),
    (1, 2048, 16, 64, 192, 128, 512, 0), (4, 8192, 16, 64, 192, 128, 256, 0),
    (1, 300, 2, 4, 64, 32, 256, 0), (2, 230, 1, 2, 200, 40, 100, 0), (1, 50, 1, 2, 8, 8, 97, 0),
    (1, 2048, 16, 64, 256, 128, 64, 1), (2, 230, 1, 2, 200, 40, 100, 1),
    (1, 300, 2, 4, 256, 64, 128, 1), (1, 300, 2, 4, 252, 64, 64, 1),
    (1, 300, 2, 4, 256, 66, 64, 1), (1, 300, 2, 4, 256, 64, 64, 0),
    (1, 256, 16, 64, 192, 128, 64, 1), (1, 512, 16, 64, 192, 128, 64, 1),
    (2, 150, 2, 4, 232, 96, 48, 1), (2, 2048, 4, 8, 256, 64, 64, 1),
])
def test_sizes(lib, B, T, Hk, Hv, Dk, Dv, C, bf16):
    sh = S(B, T, Hk, Hv, Dk, Dv, C, dtype=_lib.GDR_BF16 if bf16 else _lib.GDR_F32)
    L = _tile(C)
    ntiles = (T + L - 1) // L
    nseg = (T + C - 1) // C
    assert _lib.num_chunks(sh) == nseg
    state = B * Hv * Dv * Dk * 4
    rows = B * T * Hv * Dv * 4
    # the chunked sweeps (Dk <= 192, or Dk <= 256 with bf16 inputs whose k
    # rows come in 8-element groups and value rows in 4-element blocks; a
    # tile of 16..64 steps, T >= one tile) keep two 64 x 64 matrices (room
    # for three bf16 pieces of each: 3 x 64 x 64 floats) and three 64-vectors
    # per (batch row, value head, tile), plus 64 floats: the whole forward
    # workspace
    wide = bf16 and Dk <= 256 and Dk % 8 == 0 and Dv % 4 == 0
    chunked = (Dk <= 192 or wide) and 16 <= L <= 64 and T >= L
    prep = B * Hv * ntiles * (3 * 64 * 64 + 4 * 64) * 4 if chunked else 0
    assert _lib.forward_workspace_bytes(sh) == prep
    # C <= 64: a state per chunk and the per-step residuals; C > 64: only the
    # state per chunk (the backward replays the rest)
    if C <= 64:
        assert _lib.checkpoint_bytes(sh) == _round256(ntiles * state) + rows
    else:
        assert _lib.checkpoint_bytes(sh) == nseg * state
    # backward: state-gradient tiles, c, (chunked) 256 bytes of store sinks
    # per tile and the reverse records, and for a replay the tile states,
    # residuals and (chunked) forward records
    end = _round256(ntiles * state) + rows
    if chunked:
        end = _round256(end) + B * Hv * ntiles * 256
        end = _round256(end) + prep
    if C > 64:
        end = _round256(end) + ntiles * state
        end = _round256(end) + rows
        if chunked:
            end = _round256(end) + prep
    # bf16 inputs on the eight-wave chunk kernel (Dk, Dv multiples of 8,
    # 48 < Dk <= 256) with a (tile, kv head, batch row) grid under 256 and 2
    # to 16 value heads per kv head: the value heads go to ng groups (the
    # smallest divisor of their count that brings the grid to 256, else one
    # head each), whose fp32 dq, dk terms [2][ng][B][T][Hk][Dk] follow
    rep, wg = Hv // Hk, ntiles * Hk * B
    if (bf16 and Dk % 8 == 0 and Dv % 8 == 0 and 48 < Dk <= 256 and L <= 64
            and 2 <= rep <= 16 and wg < 256):
        ng = 2
        while ng < rep and (rep % ng or wg * ng < 256):
            ng += 1
        end = _round256(end) + B * T * Hk * Dk * 4 * 2 * ng
    assert _lib.backward_workspace_bytes(sh) == end


FAKE = 1 << 20  # a 16-byte aligned address; never dereferenced in these tests


def test_forward_null_required_pointer(lib):
    sh = S()
    for i in range(5):  # q, k, v, g, beta
        ptrs = [FAKE] * 10
        ptrs[i] = 0
        assert _lib.forward_raw(sh, *ptrs, 0, 0) == -1
    ptrs = [FAKE] * 10
    ptrs[6] = 0  # y
    assert _lib.forward_raw(sh, *ptrs, 0, 0) == -1


def test_forward_misaligned_pointer(lib):
    sh = S()
    for i in range(10):  # q .. ckpt, workspace
        ptrs = [FAKE] * 10
        ptrs[i] = FAKE + 4
        assert _lib.forward_raw(sh, *ptrs, 1 << 30, 0) == -9


def test_forward_workspace_errors(lib):
    sh = S(T=64, Dk=64, Dv=32, chunk=32)  # a shape the chunked forward takes
    ws = _lib.forward_workspace_bytes(sh)
    assert ws > 0
    ptrs = [FAKE] * 10
    assert _lib.forward_raw(sh, *ptrs, ws - 1, 0) == -8
    ptrs[9] = 0
    assert _lib.forward_raw(sh, *ptrs, ws, 0) == -8
    # the sequential sweep needs none
    assert _lib.forward_workspace_bytes(S()) == 0


def test_backward_errors(lib):
    sh = S()
    ws = _lib.backward_workspace_bytes(sh)
    args = [FAKE] * 14
    assert _lib.backward_raw(sh, *args, ws - 1, 0) == -8
    for i in (0, 1, 2, 3, 4, 5, 7, 8, 9, 10, 11, 13):
        a = list(args)
        a[i] = 0
        assert _lib.backward_raw(sh, *a, ws, 0) == -1
    a = list(args)
    a[6] = FAKE + 8  # dS_T misaligned
    assert _lib.backward_raw(sh, *a, ws, 0) == -9


def test_backward_needs_v_beyond_64(lib):
    """chunk > 64: the backward replays the tiles, so v is required."""
    sh = S(T=200, Dk=64, Dv=32, chunk=128)
    ws = _lib.backward_workspace_bytes(sh)
    args = [FAKE] * 14
    assert _lib.backward_raw(sh, *args, ws, 0, v=0) == -1
    assert _lib.backward_raw(sh, *args, ws, 0, v=FAKE + 4) == -9
    # chunk <= 64 does not read v, but a non-NULL v must still be aligned
    sh = S(T=200, Dk=64, Dv=32, chunk=64)
    ws = _lib.backward_workspace_bytes(sh)
    assert _lib.backward_raw(sh, *args, ws, 0, v=FAKE + 4) == -9


def test_empty_batch_is_a_no_op(lib):
    # B = 0: nothing to compute, nothing is launched, all pointers may be NULL
    sh = S(B=0)
    assert _lib.forward_raw(sh, *([0] * 10), 0, 0) == 0
    assert _lib.backward_raw(sh, *([0] * 14), 0, 0) == 0
    # T = 0 and no state output requested: also nothing to launch
    sh = S(T=0)
    assert _lib.forward_raw(sh, *([0] * 10), 0, 0) == 0
    assert _lib.backward_raw(sh, *([0] * 14), 0, 0) == 0


# ---- gdr_forward_noalloc: the same host-side checks, plus the scratch limit
def test_noalloc_shape_errors(lib):
    for shape, code in [(S(Hk=3, Hv=4), -3), (S(chunk=0), -5), (S(dtype=2), -6),
                        (S(Dk=257), -4)]:
        assert _lib.forward_noalloc_raw(shape, *([0] * 9), 0) == code
    assert lib.gdr_forward_noalloc(None, *([None] * 11)) == -1


def test_noalloc_scratch_limit(lib):
    """A shape whose forward workspace (the chunked forward's per-chunk
    records) exceeds the scratch array is rejected before anything runs."""
    big = S(1, 4096, 16, 64, 192, 128, 64, _lib.GDR_BF16)
    assert _lib.forward_workspace_bytes(big) > _lib.NOALLOC_SCRATCH_BYTES
    assert _lib.forward_noalloc_raw(big, *([FAKE] * 9), 0) == _lib.GDR_ERR_SCRATCH_LIMIT
    fits = S(1, 2048, 16, 64, 192, 128, 64, _lib.GDR_BF16)
    assert 0 < _lib.forward_workspace_bytes(fits) <= _lib.NOALLOC_SCRATCH_BYTES
    assert "scratch" in _lib.strerror(_lib.GDR_ERR_SCRATCH_LIMIT)


def test_noalloc_pointer_errors(lib):
    sh = S(T=64, Dk=64, Dv=32, chunk=32)  # takes the chunked forward (scratch)
    assert _lib.forward_workspace_bytes(sh) > 0
    for i in (0, 1, 2, 3, 4, 6):  # q, k, v, g, beta, y
        ptrs = [FAKE] * 9
        ptrs[i] = 0
        assert _lib.forward_noalloc_raw(sh, *ptrs, 0) == -1
    for i in range(9):
        ptrs = [FAKE] * 9
        ptrs[i] = FAKE + 4
        assert _lib.forward_noalloc_raw(sh, *ptrs, 0) == -9


def test_noalloc_empty_is_a_no_op(lib):
    assert _lib.forward_noalloc_raw(S(B=0), *([0] * 9), 0) == 0
    assert _lib.forward_noalloc_raw(S(T=0), *([0] * 9), 0) == 0


# ---- gdr_set_launch_events: argument checks (no GPU: nothing is recorded
# until a call launches a kernel, and the hook is cleared again)
def test_launch_events_arguments(lib):
    FAKE_EVENT = 0x1000  # never recorded: no launch happens while it is set
    assert _lib.set_launch_events([FAKE_EVENT] * 9) == _lib.GDR_ERR_BAD_COUNT
    assert lib.gdr_set_launch_events(None, -1) == _lib.GDR_ERR_BAD_COUNT
    assert lib.gdr_set_launch_events(None, 1) == -1  # GDR_ERR_NULL_ARG
    assert _lib.set_launch_events([FAKE_EVENT, 0]) == -1
    assert _lib.set_launch_events([FAKE_EVENT] * _lib.MAX_LAUNCH_EVENTS) == 0
    assert _lib.set_launch_events([]) == 0
    assert lib.gdr_set_launch_events(None, 0) == 0
    assert "launch-event" in _lib.strerror(_lib.GDR_ERR_BAD_COUNT)
