"""ctypes wrapper of the fp64 layer-boundary oracle (``oracle.c``).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. Nothing in the
product path (``reduce_residual_rmsnorm_bnd_amd``) imports it, and it shares
no code with that path.

All arrays are host numpy arrays. bf16 tensors travel as their uint16 bit
patterns; fp8 codes as uint8.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
          "-shared", "-fPIC"]


def build(src: str = _SRC, out: str = _LIB_PATH, extra=()) -> str:
    """Compile oracle.c (gcc, single-threaded, no contraction) into a shared library."""
    subprocess.check_call(["gcc", *CFLAGS, *extra, "-o", out, src, "-lm"])
    return out


def _bind(lib):
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
    p = ctypes.c_void_p
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_value.restype = ctypes.c_double
    lib.orc_bf16_round.argtypes = [ctypes.c_double]
    lib.orc_bf16_round.restype = ctypes.c_uint16
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_e4m3_round.argtypes = [ctypes.c_double]
    lib.orc_e4m3_round.restype = ctypes.c_uint8
    lib.orc_enter_norm.argtypes = [i64, i64, p, i64, p, f32, i32, p, i64, p, i64, p]
    lib.orc_written_norm.argtypes = [i64, i64, p, i64, p, f32, i32, p, i64, p]
    lib.orc_fold_norm.argtypes = [i64, i64, i64, i32, p, i64, p, i64, p, f32, i32, p, i64, p,
                                  i64, p, i64, p, p, p, p]
    lib.orc_moe_fold_norm.argtypes = [i64, i64, i64, i32, p, i64, i64, p, p, p, i64, p, f32,
                                      i32, p, i64, p, i64, p, i64, p, p, p, p]
    lib.orc_complete_partials.argtypes = [i64, i64, i64, i32, p, i64, p, i64, p, i64, p, p]
    lib.orc_complete_moe.argtypes = [i64, i64, i64, i32, p, i64, i64, p, p, p, i64, p, i64, p,
                                     p]
    lib.orc_snapshot.argtypes = [i64, i64, i64, i32, p, i64, p, i64, p, i64, p, p]
    for f in ("orc_enter_norm", "orc_written_norm", "orc_fold_norm", "orc_moe_fold_norm",
              "orc_complete_partials", "orc_complete_moe", "orc_snapshot"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def load(path: str | None = None, build_if_missing: bool = True):
    """Load liboracle.so (or another build of oracle.c at ``path``)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            if not build_if_missing:
                raise RuntimeError(f"{_LIB_PATH} is not built")
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _ptr_array(arrs):
    return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


class Oracle:
    """Numpy-level calls of the oracle. ``lib`` may be an alternative build."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    # number formats ----------------------------------------------------
    def bf16_value(self, bits: int) -> float:
        return self.lib.orc_bf16_value(bits)

    def bf16_round(self, v: float) -> int:
        return self.lib.orc_bf16_round(v)

    def e4m3_value(self, code: int) -> float:
        return self.lib.orc_e4m3_value(code)

    def e4m3_round(self, v: float) -> int:
        return self.lib.orc_e4m3_round(v)

    # boundary reads ----------------------------------------------------
    def enter_norm(self, x_in, w, eps, gemma=False):
        x_in = _u16(x_in)
        rows, H = x_in.shape
        w = np.ascontiguousarray(w, dtype=np.float32)
        res = np.empty((rows, H), np.uint16)
        y = np.empty((rows, H), np.uint16)
        y_ex = np.empty((rows, H), np.float64)
        rc = self.lib.orc_enter_norm(rows, H, _p(x_in), H, _p(w), eps, int(gemma), _p(res), H,
                                     _p(y), H, _p(y_ex))
        assert rc == 0
        return {"residual": res, "y": y, "y_exact": y_ex}

    def written_norm(self, residual, w, eps, gemma=False):
        residual = _u16(residual)
        rows, H = residual.shape
        w = np.ascontiguousarray(w, dtype=np.float32)
        y = np.empty((rows, H), np.uint16)
        y_ex = np.empty((rows, H), np.float64)
        rc = self.lib.orc_written_norm(rows, H, _p(residual), H, _p(w), eps, int(gemma), _p(y), H,
                                       _p(y_ex))
        assert rc == 0
        return {"y": y, "y_exact": y_ex}

    def fold_norm(self, partials, residual, w, eps, *, row_begin=0, rows=None, fp8=False,
                  gemma=False):
        """partials: list of [T,H] uint16 (global rows); residual: [rows,H] uint16 slice or None."""
        partials = [_u16(c) for c in partials]
        T, H = partials[0].shape
        rows = T - row_begin if rows is None else rows
        w = np.ascontiguousarray(w, dtype=np.float32)
        if residual is not None:
            residual = _u16(residual)
            assert residual.shape == (rows, H)
        res = np.empty((rows, H), np.uint16)
        x_ex = np.empty((rows, H), np.float64)
        y_ex = np.empty((rows, H), np.float64)
        mag = np.empty((rows, H), np.float64)
        y = q = scale = None
        if fp8:
            q = np.empty((rows, H), np.uint8)
            scale = np.empty((rows,), np.float32)
        else:
            y = np.empty((rows, H), np.uint16)
        rc = self.lib.orc_fold_norm(rows, H, row_begin, len(partials), _ptr_array(partials), H,
                                    _p(residual), H, _p(w), eps, int(gemma), _p(res), H, _p(y), H,
                                    _p(q), H, _p(scale), _p(x_ex), _p(y_ex), _p(mag))
        assert rc == 0
        out = {"residual": res, "x_exact": x_ex, "y_exact": y_ex, "mag": mag}
        if fp8:
            out.update(q=q, scale=scale)
        else:
            out["y"] = y
        return out

    def moe_fold_norm(self, E, idx, gate, k, residual, w, eps, *, row_begin=0, rows=None,
                      fp8=False, gemma=False):
        E = _u16(E)
        n_rows, H = E.shape
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        gate = np.ascontiguousarray(gate, dtype=np.float32)
        T = idx.size // k
        rows = T - row_begin if rows is None else rows
        w = np.ascontiguousarray(w, dtype=np.float32)
        if residual is not None:
            residual = _u16(residual)
            assert residual.shape == (rows, H)
        res = np.empty((rows, H), np.uint16)
        x_ex = np.empty((rows, H), np.float64)
        y_ex = np.empty((rows, H), np.float64)
        mag = np.empty((rows, H), np.float64)
        y = q = scale = None
        if fp8:
            q = np.empty((rows, H), np.uint8)
            scale = np.empty((rows,), np.float32)
        else:
            y = np.empty((rows, H), np.uint16)
        rc = self.lib.orc_moe_fold_norm(rows, H, row_begin, k, _p(E), H, n_rows, _p(idx),
                                        _p(gate), _p(residual), H, _p(w), eps, int(gemma), _p(res), H,
                                        _p(y), H, _p(q), H, _p(scale), _p(x_ex), _p(y_ex), _p(mag))
        assert rc == 0
        out = {"residual": res, "x_exact": x_ex, "y_exact": y_ex, "mag": mag}
        if fp8:
            out.update(q=q, scale=scale)
        else:
            out["y"] = y
        return out

    def complete_partials(self, partials, *, row_begin=0, rows=None, extra=None):
        """complete_output (extra None) or add_to_output (extra: [T,H] uint16, global rows)."""
        partials = [_u16(c) for c in partials]
        T, H = partials[0].shape
        rows = T - row_begin if rows is None else rows
        if extra is not None:
            extra = _u16(extra)
            assert extra.shape == (T, H)
        out = np.empty((rows, H), np.uint16)
        s_ex = np.empty((rows, H), np.float64)
        mag = np.empty((rows, H), np.float64)
        rc = self.lib.orc_complete_partials(rows, H, row_begin, len(partials),
                                            _ptr_array(partials), H, _p(extra), H, _p(out), H,
                                            _p(s_ex), _p(mag))
        assert rc == 0
        return {"out": out, "s_exact": s_ex, "mag": mag}

    def complete_moe(self, E, idx, gate, k, *, row_begin=0, rows=None, extra=None):
        E = _u16(E)
        n_rows, H = E.shape
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        gate = np.ascontiguousarray(gate, dtype=np.float32)
        T = idx.size // k
        rows = T - row_begin if rows is None else rows
        if extra is not None:
            extra = _u16(extra)
            assert extra.shape == (T, H)
        out = np.empty((rows, H), np.uint16)
        s_ex = np.empty((rows, H), np.float64)
        mag = np.empty((rows, H), np.float64)
        rc = self.lib.orc_complete_moe(rows, H, row_begin, k, _p(E), H, n_rows, _p(idx),
                                       _p(gate), _p(extra), H, _p(out), H, _p(s_ex), _p(mag))
        assert rc == 0
        return {"out": out, "s_exact": s_ex, "mag": mag}

    def snapshot(self, partials, residual, *, H=None, row_begin=0, rows=None):
        """bf16(r + sum of partials) for the slice rows; partials may be empty (a copy)."""
        partials = [_u16(c) for c in partials]
        if residual is not None:
            residual = _u16(residual)
        if partials:
            T, H = partials[0].shape
            rows = T - row_begin if rows is None else rows
        else:
            rows, H = residual.shape
        out = np.empty((rows, H), np.uint16)
        x_ex = np.empty((rows, H), np.float64)
        mag = np.empty((rows, H), np.float64)
        arr = _ptr_array(partials) if partials else None
        rc = self.lib.orc_snapshot(rows, H, row_begin, len(partials), arr, H, _p(residual), H,
                                   _p(out), H, _p(x_ex), _p(mag))
        assert rc == 0
        return {"out": out, "x_exact": x_ex, "mag": mag}
