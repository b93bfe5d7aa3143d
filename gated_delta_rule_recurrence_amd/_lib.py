"""ctypes binding of libgdr.so (the C ABI in include/gdr.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the library.  There is no fallback: if libgdr.so is missing or
fails to load, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libgdr.so"

GDR_F32 = 0
GDR_BF16 = 1
GDR_DECAY_G = 0
GDR_DECAY_LOG = 1

# entry points declared in include/gdr.h, with their ctypes signatures
_c_shape_p = None  # set below


class GdrShape(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("Hk", ctypes.c_int64),
        ("Hv", ctypes.c_int64),
        ("Dk", ctypes.c_int64),
        ("Dv", ctypes.c_int64),
        ("chunk", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("decay", ctypes.c_int32),
    ]


_vp = ctypes.c_void_p
_SIGNATURES = {
    "gdr_num_chunks": (ctypes.c_int, [ctypes.POINTER(GdrShape), ctypes.POINTER(ctypes.c_int64)]),
    "gdr_checkpoint_bytes": (ctypes.c_int, [ctypes.POINTER(GdrShape), ctypes.POINTER(ctypes.c_size_t)]),
    "gdr_backward_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(GdrShape), ctypes.POINTER(ctypes.c_size_t)]),
    "gdr_forward_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(GdrShape), ctypes.POINTER(ctypes.c_size_t)]),
    "gdr_forward": (ctypes.c_int, [ctypes.POINTER(GdrShape)] + [_vp] * 11
                    + [ctypes.c_size_t, _vp]),
    "gdr_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(GdrShape)] + [_vp] * 11),
    "gdr_backward": (ctypes.c_int, [ctypes.POINTER(GdrShape)] + [_vp] * 16
                     + [ctypes.c_size_t, _vp]),
    "gdr_set_launch_events": (ctypes.c_int, [ctypes.POINTER(_vp), ctypes.c_int]),
    "gdr_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "gdr_version": (ctypes.c_char_p, []),
}

_lib = None


class GdrError(RuntimeError):
    """A gdr_status other than GDR_OK."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def load() -> ctypes.CDLL:
    """Open libgdr.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m gated_delta_rule_recurrence_amd.build`")
    lib = ctypes.CDLL(os.fspath(LIB_PATH))
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().gdr_strerror(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != 0:
        raise GdrError(status, where)


def make_shape(B, T, Hk, Hv, Dk, Dv, chunk, dtype, decay=0) -> GdrShape:
    return GdrShape(int(B), int(T), int(Hk), int(Hv), int(Dk), int(Dv),
                    int(chunk), int(dtype), int(decay))


def num_chunks(shape: GdrShape) -> int:
    out = ctypes.c_int64()
    check(load().gdr_num_chunks(ctypes.byref(shape), ctypes.byref(out)), "gdr_num_chunks")
    return out.value


def checkpoint_bytes(shape: GdrShape) -> int:
    out = ctypes.c_size_t()
    check(load().gdr_checkpoint_bytes(ctypes.byref(shape), ctypes.byref(out)),
          "gdr_checkpoint_bytes")
    return out.value


def forward_workspace_bytes(shape: GdrShape) -> int:
    out = ctypes.c_size_t()
    check(load().gdr_forward_workspace_bytes(ctypes.byref(shape), ctypes.byref(out)),
          "gdr_forward_workspace_bytes")
    return out.value


def backward_workspace_bytes(shape: GdrShape) -> int:
    out = ctypes.c_size_t()
    check(load().gdr_backward_workspace_bytes(ctypes.byref(shape), ctypes.byref(out)),
          "gdr_backward_workspace_bytes")
    return out.value


def forward_raw(shape, q, k, v, g, beta, S0, y, S_T, ckpt, workspace,
                workspace_bytes, stream, mask=0) -> int:
    """gdr_forward with integer device addresses (0 = NULL); returns the status."""
    ptrs = [_vp(x or None) for x in (q, k, v, g, beta, S0, mask, y, S_T, ckpt, workspace)]
    return load().gdr_forward(ctypes.byref(shape), *ptrs,
                              ctypes.c_size_t(int(workspace_bytes)),
                              _vp(stream or None))


def forward_noalloc_raw(shape, q, k, v, g, beta, S0, y, S_T, ckpt, stream, mask=0) -> int:
    """gdr_forward_noalloc with integer device addresses (0 = NULL); returns
    the status."""
    ptrs = [_vp(x or None) for x in (q, k, v, g, beta, S0, mask, y, S_T, ckpt)]
    return load().gdr_forward_noalloc(ctypes.byref(shape), *ptrs, _vp(stream or None))


NOALLOC_SCRATCH_BYTES = 128 << 20  # GDR_NOALLOC_SCRATCH_BYTES
GDR_ERR_SCRATCH_LIMIT = -12
GDR_ERR_BAD_COUNT = -13
MAX_LAUNCH_EVENTS = 8  # GDR_MAX_LAUNCH_EVENTS


def set_launch_events(handles) -> int:
    """gdr_set_launch_events: the raw hipEvent_t handles (ints) that the
    following calls record after their kernel launches, in order; an empty
    sequence clears the hook.  Returns the status."""
    handles = list(handles)
    arr = (_vp * max(len(handles), 1))(*[_vp(h) for h in handles])
    return load().gdr_set_launch_events(arr, len(handles))


def backward_raw(shape, q, k, g, beta, ckpt, dy, dS_T, dq, dk, dv, dg, dbeta,
                 dS0, workspace, workspace_bytes, stream, mask=0, v=0) -> int:
    """gdr_backward with integer device addresses (0 = NULL); returns the
    status.  v is read only for chunk > 64."""
    ptrs = [_vp(x or None) for x in (q, k, v, g, beta, mask, ckpt, dy, dS_T, dq, dk, dv,
                                     dg, dbeta, dS0, workspace)]
    return load().gdr_backward(ctypes.byref(shape), *ptrs,
                               ctypes.c_size_t(int(workspace_bytes)),
                               _vp(stream or None))
