"""ctypes wrapper of the plain-C OpenMP recurrence (ssd_oracle.c) -- test infrastructure.

``build()`` compiles ssd_oracle.c with gcc into oracle/_lib/libssd_oracle.so; ``forward`` runs it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIBDIR = os.path.join(_HERE, "_lib")
LIB_PATH = os.path.join(_LIBDIR, "libssd_oracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle (always recompiles). Returns the library path."""
    os.makedirs(_LIBDIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    global _lib
    _lib = None
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.ssd_oracle_forward.argtypes = [i64] * 6 + [p] * 7 + [p, p] + [p, i64, ctypes.c_int]
        lib.ssd_oracle_forward.restype = ctypes.c_int
        lib.ssd_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().ssd_oracle_max_threads())


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def forward(x, dt, A, B, C, D, initial_state=None, units=None, nthreads: int = 0):
    """Float64 recurrence over float32 inputs (exact values) and a float64 initial state.

    Same layouts as the numpy oracle.

    units: optional list of (batch * H + head) indices; only those heads are computed and the
    other entries of y / final_state are left as NaN.  Returns (y, final_state) as float64.
    """
    x, dt, A, B, C, D = (_f32(v) for v in (x, dt, A, B, C, D))
    h0 = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if dt.shape != (Bt, L, H) or A.shape != (H,) or D.shape != (H,):
        raise ValueError("shape mismatch")
    if B.shape != (Bt, L, G, N) or C.shape != (Bt, L, G, N):
        raise ValueError("shape mismatch")
    if h0 is not None and h0.shape != (Bt, H, P, N):
        raise ValueError("shape mismatch")
    y = np.full((Bt, L, H, P), np.nan)
    fin = np.full((Bt, H, P, N), np.nan)
    u = None
    if units is not None:
        u = np.ascontiguousarray(units, dtype=np.int64)
        if u.size and (u.min() < 0 or u.max() >= Bt * H):
            raise ValueError("unit index out of range")
    rc = _load().ssd_oracle_forward(Bt, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                    _ptr(C), _ptr(D), _ptr(h0), _ptr(y), _ptr(fin), _ptr(u),
                                    0 if u is None else u.size, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_forward failed ({rc})")
    return y, fin
