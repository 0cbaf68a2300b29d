"""Plain fp64 CPU oracle for the RWKV-4 WKV operator.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the CPU-baseline
leg of the benchmark are the only callers. The GPU library never imports, links or
calls anything here, and nothing here imports the GPU package.

The arithmetic lives in ``wkv_oracle.c`` (plain C, fp64, OpenMP over (b, c)); this
module builds it with gcc when the shared object is missing or stale and marshals
numpy arrays through ctypes. Every input is upcast to fp64 exactly.

Operator, per batch row and channel (0-based t), from "RWKV解读：在Transformer的时代的新RNN",
section 二.3, formula (8) and its recursive form, and "RWKV についての調査記録",
section 【wkvとは】:

    y_t = (sum_{i<t} e^{-(t-1-i)w + k_i} v_i + e^{u+k_t} v_t)
        / (sum_{i<t} e^{-(t-1-i)w + k_i}     + e^{u+k_t})

Routines: ``forward_direct`` (the O(T^2) definition), ``forward_recurrent`` (plain
recursion), ``forward_rescaled`` / ``decode_step`` (recursion on a rescaled state),
``backward_direct`` (O(T^2) from the softmax form) and ``backward_recurrent``
(linear-time carries). Each is pinned in tests/ against closed forms, invariants,
finite differences and autograd, not against another routine alone. ``token_shift`` and
``token_shift_backward`` (numpy, token_shift.py) are the mix of formula (7) that feeds the
projections.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wkv_oracle.c")
# WKV_ORACLE_SANITIZE=1 builds and loads an AddressSanitizer + UndefinedBehaviorSanitizer
# build instead (its own file; the process must preload gcc's libasan), for the sanitizer
# pass of the oracle's pins.
SANITIZE = os.environ.get("WKV_ORACLE_SANITIZE") == "1"
_LIB_PATH = os.path.join(_HERE, "liboracle_wkv_san.so" if SANITIZE else "liboracle_wkv.so")
_lib = None

_CFLAGS = ["-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c99", "-Wall"]
_SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all"]


def compile_command(src: str, out: str) -> list:
    """The gcc command that builds a copy of the oracle source `src` into `out` (with the
    sanitizers when WKV_ORACLE_SANITIZE=1)."""
    opt = _SAN_FLAGS if SANITIZE else ["-O2"]
    return ["gcc"] + opt + _CFLAGS + [src, "-o", out, "-lm"]

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile wkv_oracle.c into liboracle_wkv.so (gcc, -O2, OpenMP, no FP contraction)."""
    if (not force and os.path.exists(_LIB_PATH)
            and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.run(compile_command(_SRC, tmp), check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _configure(lib):
    lib.wkv_oracle_num_threads.restype = ctypes.c_int
    lib.wkv_oracle_num_threads.argtypes = []
    fwd = [_I64, _I64, _I64, _D, _D, _D, _D, _D]
    lib.wkv_oracle_forward_direct.restype = None
    lib.wkv_oracle_forward_direct.argtypes = fwd
    lib.wkv_oracle_forward_recurrent.restype = ctypes.c_int
    lib.wkv_oracle_forward_recurrent.argtypes = fwd
    lib.wkv_oracle_forward_rescaled.restype = None
    lib.wkv_oracle_forward_rescaled.argtypes = fwd + [_D, _D, _D]
    lib.wkv_oracle_decode_step.restype = None
    lib.wkv_oracle_decode_step.argtypes = [_I64, _I64, _D, _D, _D, _D, _D, _D, _D, _D]
    bwd = [_I64, _I64, _I64, _D, _D, _D, _D, _D, _D, _D, _D, _D]
    lib.wkv_oracle_backward_direct.restype = None
    lib.wkv_oracle_backward_direct.argtypes = bwd
    lib.wkv_oracle_backward_recurrent.restype = ctypes.c_int
    lib.wkv_oracle_backward_recurrent.argtypes = bwd
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = _configure(ctypes.CDLL(build()))
    return _lib


def use_library(path: str | None):
    """Route every routine through another build of wkv_oracle.c (None: the default).

    Used by the mutation tests, which compile deliberately broken copies of the source
    to show that the pins catch them.
    """
    global _lib
    _lib = None if path is None else _configure(ctypes.CDLL(path))


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x), dtype=np.float64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(_D)


def _shapes(w, u, k, v):
    k = _f64(k)
    v = _f64(v)
    if k.ndim != 3 or k.shape != v.shape:
        raise ValueError("k and v must both be [B, T, C]")
    B, T, C = k.shape
    w = _f64(w).reshape(-1)
    u = _f64(u).reshape(-1)
    if w.shape != (C,) or u.shape != (C,):
        raise ValueError("w and u must be [C]")
    return B, T, C, w, u, k, v


def num_threads() -> int:
    """OpenMP threads the oracle routines use."""
    return int(_load().wkv_oracle_num_threads())


def forward_direct(w, u, k, v) -> np.ndarray:
    """y [B,T,C] from the O(T^2) definition (max-shifted softmax per output position)."""
    B, T, C, w, u, k, v = _shapes(w, u, k, v)
    y = np.empty((B, T, C), np.float64)
    _load().wkv_oracle_forward_direct(B, T, C, _p(w), _p(u), _p(k), _p(v), _p(y))
    return y


def forward_recurrent(w, u, k, v) -> np.ndarray:
    """y [B,T,C] from the plain (unscaled) recursion; needs max|k| + max|u| < 600."""
    B, T, C, w, u, k, v = _shapes(w, u, k, v)
    y = np.empty((B, T, C), np.float64)
    rc = _load().wkv_oracle_forward_recurrent(B, T, C, _p(w), _p(u), _p(k), _p(v), _p(y))
    if rc:
        raise OverflowError("plain recursion needs max|k| + max|u| < 600")
    return y


def forward_rescaled(w, u, k, v, state=None):
    """Recursion on the rescaled state (a, b, p), A = a e^p, B = b e^p.

    ``state`` is None (empty state) or a tuple of three [B, C] arrays, which are not
    modified. Returns (y, (a, b, p)) with the final state.
    """
    B, T, C, w, u, k, v = _shapes(w, u, k, v)
    if state is None:
        a = np.zeros((B, C))
        b = np.zeros((B, C))
        p = np.full((B, C), -1e38)
    else:
        a, b, p = (_f64(s).reshape(B, C).copy() for s in state)
    y = np.empty((B, T, C), np.float64)
    _load().wkv_oracle_forward_rescaled(B, T, C, _p(w), _p(u), _p(k), _p(v), _p(y),
                                        _p(a), _p(b), _p(p))
    return y, (a, b, p)


def decode_step(w, u, k, v, state):
    """One token for B sequences: k, v [B, C]; returns (y [B, C], new state)."""
    k = _f64(k)
    if k.ndim != 2:
        raise ValueError("decode k, v must be [B, C]")
    y, st = forward_rescaled(w, u, k[:, None, :], _f64(v)[:, None, :], state)
    return y[:, 0, :], st


def backward_direct(w, u, k, v, dy):
    """(dk, dv, dw, du) of L = sum(dy * y) from the O(T^2) softmax form."""
    B, T, C, w, u, k, v = _shapes(w, u, k, v)
    dy = _f64(dy)
    if dy.shape != k.shape:
        raise ValueError("dy must be [B, T, C]")
    dk = np.empty_like(k)
    dv = np.empty_like(k)
    dw = np.empty(C)
    du = np.empty(C)
    _load().wkv_oracle_backward_direct(B, T, C, _p(w), _p(u), _p(k), _p(v), _p(dy),
                                       _p(dk), _p(dv), _p(dw), _p(du))
    return dk, dv, dw, du


def backward_recurrent(w, u, k, v, dy):
    """(dk, dv, dw, du) from linear-time plain carries; needs max|k| + max|u| < 600."""
    B, T, C, w, u, k, v = _shapes(w, u, k, v)
    dy = _f64(dy)
    if dy.shape != k.shape:
        raise ValueError("dy must be [B, T, C]")
    dk = np.empty_like(k)
    dv = np.empty_like(k)
    dw = np.empty(C)
    du = np.empty(C)
    rc = _load().wkv_oracle_backward_recurrent(B, T, C, _p(w), _p(u), _p(k), _p(v), _p(dy),
                                               _p(dk), _p(dv), _p(dw), _p(du))
    if rc:
        raise OverflowError("plain recursion needs max|k| + max|u| < 600")
    return dk, dv, dw, du


from .token_shift import token_shift, token_shift_backward  # noqa: E402,F401
