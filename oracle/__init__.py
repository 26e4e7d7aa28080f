"""fp64 CPU oracle for the depthwise causal conv1d — TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The GPU library and its Python
binding never import it, and it never imports them.

The arithmetic lives in ``ccv_oracle.c`` (plain C, fp64); this module only
builds/loads it and marshals numpy arrays.  Every array is in the logical
layout of the cuDNN FE "Causal Conv1d" page's shapes:
x/y/dy/dx ``[B,D,T]``, weight ``[D,W]``, bias ``[D]``, states ``[R,D,W-1]``
(R = B dense, R = N = len(cu_seqlens)-1 packed).

Every function is pinned by ``tests/test_oracle_pins.py`` against closed
forms, invariants, library routines (``torch.nn.functional.conv1d`` in
float64, ``numpy.convolve``) and finite differences.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ccv_oracle.c")
_LIB = os.path.join(_HERE, "libccv_oracle.so")

ACT_NONE = 0
ACT_SILU = 1

CU_FIRST_NONZERO = 1
CU_LAST_MISMATCH = 2
CU_DECREASING = 4
CU_EMPTY = 8


def build(force=False):
    """Compile the oracle with gcc (plain C, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "ccv_oracle.h"))):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall",
                               "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path):
        lib = ctypes.CDLL(path)
        i64, dp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        lib.oracle_fwd.argtypes = [i64, i64, i64, i64, dp, dp, dp, ip, i64, dp, ctypes.c_int, dp, dp]
        lib.oracle_fwd.restype = ctypes.c_int
        lib.oracle_bwd.argtypes = [i64, i64, i64, i64, dp, dp, dp, ip, i64, dp, dp, dp,
                                   ctypes.c_int, dp, dp, dp, dp]
        lib.oracle_bwd.restype = ctypes.c_int
        lib.oracle_fwd_seq.argtypes = [i64, i64, i64, i64, dp, dp, dp, ip, ctypes.c_int, dp]
        lib.oracle_fwd_seq.restype = ctypes.c_int
        lib.oracle_bwd_seq.argtypes = [i64, i64, i64, i64, dp, dp, dp, ip, dp, ctypes.c_int,
                                       dp, dp, dp]
        lib.oracle_bwd_seq.restype = ctypes.c_int
        lib.oracle_update.argtypes = [i64, i64, i64, dp, dp, dp, dp, ctypes.c_int, dp]
        lib.oracle_update.restype = ctypes.c_int
        lib.oracle_validate_cu_seqlens.argtypes = [ip, i64, i64]
        lib.oracle_validate_cu_seqlens.restype = ctypes.c_uint32
        self.lib = lib


_default = None


def _load():
    global _default
    if _default is None:
        _default = _Oracle(build())
    return _default.lib


def compile_variant(source_text, workdir):
    """Compile an edited copy of the oracle source (used by the tests that
    check the pins catch planted mistakes) and return its library handle."""
    src = os.path.join(workdir, "ccv_oracle.c")
    with open(src, "w") as f:
        f.write(source_text)
    with open(os.path.join(_HERE, "ccv_oracle.h")) as f:
        hdr = f.read()
    with open(os.path.join(workdir, "ccv_oracle.h"), "w") as f:
        f.write(hdr)
    lib = os.path.join(workdir, "libvariant.so")
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-o", lib, src, "-lm"])
    return _Oracle(lib).lib


def source_text():
    with open(_SRC) as f:
        return f.read()


_override = None


class use_library:
    """Context manager: route this module's functions to another compiled
    oracle (a planted-mistake variant) for the duration of a test."""

    def __init__(self, lib):
        self.lib = lib

    def __enter__(self):
        global _override
        self.prev, _override = _override, self.lib
        return self

    def __exit__(self, *exc):
        global _override
        _override = self.prev
        return False


def _L():
    return _override if _override is not None else _load()


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _act(activation):
    if activation in (None, "none", ACT_NONE):
        return ACT_NONE
    if activation in ("silu", ACT_SILU):
        return ACT_SILU
    raise ValueError("activation must be None or 'silu'")


def fwd(x, w, bias=None, cu_seqlens=None, initial_states=None, activation="silu",
        return_final_states=True):
    """Forward: returns (y [B,D,T], final_states [R,D,W-1] or None)."""
    x, w, bias, init = _f64(x), _f64(w), _f64(bias), _f64(initial_states)
    cu = _i32(cu_seqlens)
    B, D, T = x.shape
    W = w.shape[1]
    N = 0 if cu is None else cu.shape[0] - 1
    R = B if cu is None else N
    y = np.empty((B, D, T), np.float64)
    fin = np.empty((R, D, W - 1), np.float64) if return_final_states else None
    rc = _L().oracle_fwd(B, D, T, W, _ptr(x), _ptr(w), _ptr(bias), _ptr(cu), N,
                            _ptr(init), _act(activation), _ptr(y), _ptr(fin))
    if rc:
        raise ValueError("oracle_fwd rejected the arguments (%d)" % rc)
    return y, fin


def bwd(x, w, dy, bias=None, cu_seqlens=None, initial_states=None, dfinal_states=None,
        activation="silu"):
    """Backward of L = <dy, y> + <dfinal, final_states>.

    Returns (dx [B,D,T], dw [D,W], dbias [D] or None, dinit [R,D,W-1] or None);
    dinit is returned only when initial_states is given.
    """
    x, w, bias, init = _f64(x), _f64(w), _f64(bias), _f64(initial_states)
    dy, dfin = _f64(dy), _f64(dfinal_states)
    cu = _i32(cu_seqlens)
    B, D, T = x.shape
    W = w.shape[1]
    N = 0 if cu is None else cu.shape[0] - 1
    R = B if cu is None else N
    dx = np.empty((B, D, T), np.float64)
    dw = np.empty((D, W), np.float64)
    db = np.empty((D,), np.float64) if bias is not None else None
    dinit = np.empty((R, D, W - 1), np.float64) if init is not None else None
    rc = _L().oracle_bwd(B, D, T, W, _ptr(x), _ptr(w), _ptr(bias), _ptr(cu), N, _ptr(init),
                            _ptr(dy), _ptr(dfin), _act(activation), _ptr(dx), _ptr(dw),
                            _ptr(db), _ptr(dinit))
    if rc:
        raise ValueError("oracle_bwd rejected the arguments (%d)" % rc)
    return dx, dw, db, dinit


def fwd_seq(x, w, seq_idx, bias=None, activation="silu"):
    """Forward with per-token sequence ids seq_idx [B,T]: returns y [B,D,T]."""
    x, w, bias, seq = _f64(x), _f64(w), _f64(bias), _i32(seq_idx)
    B, D, T = x.shape
    W = w.shape[1]
    if seq.shape != (B, T):
        raise ValueError("seq_idx must be [B,T]")
    y = np.empty((B, D, T), np.float64)
    rc = _L().oracle_fwd_seq(B, D, T, W, _ptr(x), _ptr(w), _ptr(bias), _ptr(seq),
                             _act(activation), _ptr(y))
    if rc:
        raise ValueError("oracle_fwd_seq rejected the arguments (%d)" % rc)
    return y


def bwd_seq(x, w, dy, seq_idx, bias=None, activation="silu"):
    """Backward of <dy, y> for fwd_seq: returns (dx, dw, dbias or None)."""
    x, w, bias, dy, seq = _f64(x), _f64(w), _f64(bias), _f64(dy), _i32(seq_idx)
    B, D, T = x.shape
    W = w.shape[1]
    if seq.shape != (B, T):
        raise ValueError("seq_idx must be [B,T]")
    dx = np.empty((B, D, T), np.float64)
    dw = np.empty((D, W), np.float64)
    db = np.empty((D,), np.float64) if bias is not None else None
    rc = _L().oracle_bwd_seq(B, D, T, W, _ptr(x), _ptr(w), _ptr(bias), _ptr(seq), _ptr(dy),
                             _act(activation), _ptr(dx), _ptr(dw), _ptr(db))
    if rc:
        raise ValueError("oracle_bwd_seq rejected the arguments (%d)" % rc)
    return dx, dw, db


def update(x, state, w, bias=None, activation="silu"):
    """One decode step: returns (y [B,D], new_state [B,D,W-1]); inputs untouched."""
    x, w, bias = _f64(x), _f64(w), _f64(bias)
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    B, D = x.shape
    W = w.shape[1]
    y = np.empty((B, D), np.float64)
    rc = _L().oracle_update(B, D, W, _ptr(x), _ptr(st), _ptr(w), _ptr(bias),
                               _act(activation), _ptr(y))
    if rc:
        raise ValueError("oracle_update rejected the arguments (%d)" % rc)
    return y, st


def update_tokens(x, state, w, bias=None, activation="silu"):
    """L decode tokens x [B,D,L] in order: L single-token steps (the
    definition of a multi-token update).  Returns (y [B,D,L], new state)."""
    x = _f64(x)
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    y = np.empty(x.shape, np.float64)
    for l in range(x.shape[2]):
        y[:, :, l], st = update(x[:, :, l], st, w, bias, activation)
    return y, st


def validate_cu_seqlens(cu_seqlens, total):
    """Bit mask of the four malformed-metadata conditions (uint32)."""
    cu = _i32(cu_seqlens)
    return int(_L().oracle_validate_cu_seqlens(_ptr(cu), cu.shape[0] - 1, int(total)))
