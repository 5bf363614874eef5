"""Python binding of libboundary (include/boundary.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libboundary.so. Tensors are PyTorch device tensors; the binding checks dtype,
device, shape and row-major layout, passes ``data_ptr()`` and the leading
dimension, and launches on the current HIP stream unless one is given. The
library must be built (``__graft_entry__.build()``): importing the binding on
a machine without it raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libboundary.so")

# bnd_state
BND_INITIAL, BND_WRITTEN, BND_PENDING = 0, 1, 2
# bnd_kind
BND_KIND_NONE, BND_KIND_PARTIALS, BND_KIND_MOE = 0, 1, 2
# bnd_status
BND_OK = 0
BND_ERR_INVALID_ARG = -1
BND_ERR_NOT_STARTED = -2
BND_ERR_FOREIGN_OUTPUT = -3
BND_ERR_PENDING = -4
BND_ERR_WRONG_KIND = -5
BND_ERR_NO_PATH = -6
BND_ERR_UNAVAILABLE = -7
BND_ERR_HIP = -8
BND_OWED_NONE = 0
BND_MAX_SOURCES = 16
BND_MAX_HIDDEN = 32768
# bnd_norm_form
BND_NORM_PLAIN, BND_NORM_GEMMA = 0, 1
# bnd_option
BND_OPT_FUSED_UNAVAILABLE = 1
BND_OPT_THREADS_PER_ROW = 2
BND_OPT_VECTORS_PER_THREAD = 3
BND_OPT_ONE_WAVEFRONT = 4
BND_ONE_WAVEFRONT_AUTO = 0
BND_ONE_WAVEFRONT_ALWAYS = 1
BND_ONE_WAVEFRONT_NEVER = 2
BND_OPT_RING_DEPTH = 5

# exported symbols, in header order
SYMBOLS = [
    "bnd_stream_create", "bnd_stream_destroy", "bnd_stream_state", "bnd_stream_pending_kind",
    "bnd_stream_has_residual", "bnd_stream_set_norm_form", "bnd_publish_partials", "bnd_publish_moe", "bnd_enter_norm",
    "bnd_fold_norm", "bnd_fold_norm_quant_fp8", "bnd_moe_finalize_fold_norm", "bnd_complete_only",
    "bnd_add_to_output", "bnd_snapshot", "bnd_rsv_share", "bnd_written", "bnd_take_output", "bnd_status_str", "bnd_last_error", "bnd_version",
    "bnd_set_option", "bnd_get_option", "bnd_last_launch_shape", "bnd_last_launch_ring_depth",
    "bnd_time_next_launch",
]

_lib = None


class BoundaryError(RuntimeError):
    """A libboundary call returned an error status."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def _declare(lib):
    c = ctypes
    vp, i64, i32, f32, u64 = c.c_void_p, c.c_int64, c.c_int, c.c_float, c.c_uint64
    st = c.c_int
    sig = {
        "bnd_stream_create": (st, [c.POINTER(vp), i64, i64, i64, i64, vp, i64]),
        "bnd_stream_destroy": (st, [vp]),
        "bnd_stream_state": (c.c_int, [vp]),
        "bnd_stream_pending_kind": (c.c_int, [vp]),
        "bnd_stream_has_residual": (c.c_int, [vp]),
        "bnd_stream_set_norm_form": (st, [vp, c.c_int]),
        "bnd_publish_partials": (st, [vp, c.POINTER(vp), i32, i64, c.POINTER(u64)]),
        "bnd_publish_moe": (st, [vp, vp, i64, i64, vp, vp, i32, c.POINTER(u64)]),
        "bnd_enter_norm": (st, [vp, vp, i64, vp, f32, vp, i64, vp]),
        "bnd_fold_norm": (st, [vp, u64, vp, f32, vp, i64, vp]),
        "bnd_fold_norm_quant_fp8": (st, [vp, u64, vp, f32, vp, i64, vp, vp]),
        "bnd_moe_finalize_fold_norm": (st, [vp, u64, vp, f32, vp, i64, vp]),
        "bnd_complete_only": (st, [vp, u64, vp, i64, c.POINTER(u64), vp]),
        "bnd_add_to_output": (st, [vp, u64, vp, i64, vp, i64, c.POINTER(u64), vp]),
        "bnd_snapshot": (st, [vp, u64, vp, i64, vp]),
        "bnd_rsv_share": (st, [c.POINTER(i64), i32, i32, c.POINTER(i64), c.POINTER(i64),
                               c.POINTER(i64)]),
        "bnd_written": (st, [vp, vp, i64]),
        "bnd_take_output": (st, [vp]),
        "bnd_status_str": (c.c_char_p, [st]),
        "bnd_last_error": (c.c_char_p, []),
        "bnd_version": (c.c_char_p, []),
        "bnd_set_option": (st, [c.c_int, i64]),
        "bnd_get_option": (i64, [c.c_int]),
        "bnd_last_launch_shape": (st, [c.POINTER(i64), c.POINTER(i32), c.POINTER(i32), c.POINTER(i32)]),
        "bnd_last_launch_ring_depth": (st, [c.POINTER(i32)]),
        "bnd_time_next_launch": (st, [vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def lib():
    """The loaded libboundary (ctypes). Raises if the library is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _check(status: int) -> None:
    if status != BND_OK:
        raise BoundaryError(status, lib().bnd_last_error().decode())


def status_name(status: int) -> str:
    return lib().bnd_status_str(status).decode()


def set_option(opt: int, value: int) -> None:
    _check(lib().bnd_set_option(opt, value))


def get_option(opt: int) -> int:
    return lib().bnd_get_option(opt)


def last_launch_shape() -> tuple[int, int, int, bool]:
    """(workgroups, threads per workgroup, vectors per thread, one wavefront per row) of this
    thread's last launch."""
    rows, threads, vpt, one = ctypes.c_int64(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().bnd_last_launch_shape(ctypes.byref(rows), ctypes.byref(threads), ctypes.byref(vpt),
                                       ctypes.byref(one)))
    return rows.value, threads.value, vpt.value, bool(one.value)


def last_launch_ring_depth() -> int:
    """Loads in flight per one-wavefront row in this thread's last launch (2, or 4, 6 or 8 for the
    deep ring of that width; 0 for a launch with several wavefronts per row)."""
    depth = ctypes.c_int()
    _check(lib().bnd_last_launch_ring_depth(ctypes.byref(depth)))
    return depth.value


def _hip_stream(hip_stream):
    if hip_stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(hip_stream, torch.cuda.Stream):
        return ctypes.c_void_p(hip_stream.cuda_stream)
    return ctypes.c_void_p(int(hip_stream))


def _rows(t: torch.Tensor, name: str, rows: int, H: int, dtype: torch.dtype):
    """(pointer, leading dimension) of a row-major [>= rows, H] device tensor."""
    if t is None:
        if rows == 0:
            return None, H
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 2 or t.shape[1] != H or t.shape[0] < rows or (rows > 0 and t.stride(1) != 1):
        raise ValueError(f"{name}: expected a row-major [{rows}, {H}] tensor, got "
                         f"{tuple(t.shape)} with strides {t.stride()}")
    return ctypes.c_void_p(t.data_ptr()), t.stride(0) if t.shape[0] > 1 else max(H, t.stride(0))


def _vec(t: torch.Tensor, name: str, n: int, dtype: torch.dtype):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype or not t.is_cuda or t.numel() < n or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {dtype} device tensor of {n} elements")
    return ctypes.c_void_p(t.data_ptr())


class Stream:
    """A bnd_stream: the residual stream of one microbatch at the boundaries.

    Holds references to the tensors of its pending work so they outlive the
    launch that reads them.
    """

    def __init__(self, T: int, H: int, residual: torch.Tensor | None, row_begin: int = 0,
                 rows: int | None = None):
        self.T, self.H, self.row_begin = T, H, row_begin
        self.rows = T - row_begin if rows is None else rows
        ptr, ld = _rows(residual, "residual", self.rows, H, torch.bfloat16)
        handle = ctypes.c_void_p()
        _check(lib().bnd_stream_create(ctypes.byref(handle), T, H, row_begin, self.rows, ptr, ld))
        self._h = handle
        self._keep = [residual]
        self._pending = []

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise RuntimeError("stream destroyed")
        return self._h

    @property
    def state(self) -> int:
        return lib().bnd_stream_state(self.handle)

    @property
    def pending_kind(self) -> int:
        return lib().bnd_stream_pending_kind(self.handle)

    @property
    def has_residual(self) -> bool:
        return bool(lib().bnd_stream_has_residual(self.handle))

    def destroy(self) -> None:
        if self._h is not None:
            lib().bnd_stream_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def bnd_stream_create(T: int, H: int, residual: torch.Tensor | None, row_begin: int = 0,
                      rows: int | None = None) -> Stream:
    return Stream(T, H, residual, row_begin, rows)


def bnd_stream_destroy(s: Stream) -> None:
    s.destroy()


def bnd_stream_set_norm_form(s: Stream, form: int) -> None:
    _check(lib().bnd_stream_set_norm_form(s.handle, form))


def bnd_publish_partials(s: Stream, partials: Sequence[torch.Tensor]) -> int:
    P = len(partials)
    ptrs, ld = [], s.H
    for p, c in enumerate(partials):
        ptr, ld_p = _rows(c, f"partial {p}", s.T if s.rows else 0, s.H, torch.bfloat16)
        if p and ld_p != ld:
            raise ValueError("partials must share one leading dimension")
        ld = ld_p
        ptrs.append(ptr)
    arr = (ctypes.c_void_p * max(P, 1))(*ptrs)
    owed = ctypes.c_uint64()
    _check(lib().bnd_publish_partials(s.handle, arr, P, ld, ctypes.byref(owed)))
    s._pending = list(partials)
    return owed.value


def bnd_publish_moe(s: Stream, expert_rows: torch.Tensor, idx: torch.Tensor, gate: torch.Tensor,
                    k: int) -> int:
    n_rows = expert_rows.shape[0]
    eptr, ld = _rows(expert_rows, "expert_rows", n_rows if s.rows else 0, s.H, torch.bfloat16)
    need = s.T * k if s.rows else 0
    iptr = _vec(idx, "idx", need, torch.int32) if s.rows else None
    gptr = _vec(gate, "gate", need, torch.float32) if s.rows else None
    owed = ctypes.c_uint64()
    _check(lib().bnd_publish_moe(s.handle, eptr, n_rows, ld, iptr, gptr, k, ctypes.byref(owed)))
    s._pending = [expert_rows, idx, gate]
    return owed.value


def bnd_enter_norm(s: Stream, x: torch.Tensor | None, weight: torch.Tensor, eps: float,
                   y: torch.Tensor, hip_stream=None) -> None:
    entering = s.state == BND_INITIAL
    xptr, ld_x = _rows(x, "x", s.rows if entering else 0, s.H, torch.bfloat16)
    yptr, ld_y = _rows(y, "y", s.rows, s.H, torch.bfloat16)
    wptr = _vec(weight, "weight", s.H, torch.float32) if s.rows else None
    _check(lib().bnd_enter_norm(s.handle, xptr, ld_x, wptr, eps, yptr, ld_y, _hip_stream(hip_stream)))
    s._pending = []


def bnd_fold_norm(s: Stream, owed: int, weight: torch.Tensor, eps: float, y: torch.Tensor,
                  hip_stream=None) -> None:
    yptr, ld_y = _rows(y, "y", s.rows, s.H, torch.bfloat16)
    wptr = _vec(weight, "weight", s.H, torch.float32) if s.rows else None
    _check(lib().bnd_fold_norm(s.handle, owed, wptr, eps, yptr, ld_y, _hip_stream(hip_stream)))


def bnd_fold_norm_quant_fp8(s: Stream, owed: int, weight: torch.Tensor, eps: float,
                            q: torch.Tensor, scale: torch.Tensor, hip_stream=None) -> None:
    qptr, ld_q = _rows(q, "q", s.rows, s.H, torch.uint8)
    sptr = _vec(scale, "scale", s.rows, torch.float32) if s.rows else None
    wptr = _vec(weight, "weight", s.H, torch.float32) if s.rows else None
    _check(lib().bnd_fold_norm_quant_fp8(s.handle, owed, wptr, eps, qptr, ld_q, sptr,
                                         _hip_stream(hip_stream)))


def bnd_moe_finalize_fold_norm(s: Stream, owed: int, weight: torch.Tensor, eps: float,
                               y: torch.Tensor, hip_stream=None) -> None:
    yptr, ld_y = _rows(y, "y", s.rows, s.H, torch.bfloat16)
    wptr = _vec(weight, "weight", s.H, torch.float32) if s.rows else None
    _check(lib().bnd_moe_finalize_fold_norm(s.handle, owed, wptr, eps, yptr, ld_y,
                                            _hip_stream(hip_stream)))


def bnd_complete_only(s: Stream, owed: int, out: torch.Tensor, hip_stream=None) -> int:
    optr, ld = _rows(out, "out", s.rows, s.H, torch.bfloat16)
    new = ctypes.c_uint64()
    _check(lib().bnd_complete_only(s.handle, owed, optr, ld, ctypes.byref(new),
                                   _hip_stream(hip_stream)))
    s._pending = s._pending + [out]
    return new.value


def bnd_add_to_output(s: Stream, owed: int, extra: torch.Tensor, out: torch.Tensor,
                      hip_stream=None) -> int:
    eptr, ld_e = _rows(extra, "extra", s.T if s.rows else 0, s.H, torch.bfloat16)
    optr, ld_o = _rows(out, "out", s.rows, s.H, torch.bfloat16)
    new = ctypes.c_uint64()
    _check(lib().bnd_add_to_output(s.handle, owed, eptr, ld_e, optr, ld_o, ctypes.byref(new),
                                   _hip_stream(hip_stream)))
    s._pending = s._pending + [extra, out]
    return new.value


def bnd_snapshot(s: Stream, owed: int, out: torch.Tensor, hip_stream=None) -> None:
    optr, ld_o = _rows(out, "out", s.rows, s.H, torch.bfloat16)
    _check(lib().bnd_snapshot(s.handle, owed, optr, ld_o, _hip_stream(hip_stream)))


def bnd_rsv_share(counts: Sequence[int], r: int):
    """(row_begin, rows, T) of rank r for per-rank row counts."""
    arr = (ctypes.c_int64 * len(counts))(*counts)
    b, n, t = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().bnd_rsv_share(arr, len(counts), r, ctypes.byref(b), ctypes.byref(n),
                               ctypes.byref(t)))
    return b.value, n.value, t.value


def bnd_written(s: Stream, residual: torch.Tensor) -> None:
    ptr, ld = _rows(residual, "residual", s.rows, s.H, torch.bfloat16)
    _check(lib().bnd_written(s.handle, ptr, ld))
    s._keep = [residual]
    s._pending = []


def bnd_take_output(s: Stream) -> None:
    _check(lib().bnd_take_output(s.handle))
    s._pending = []
