"""Sequential fp64 selective scan -- oracle, TEST INFRASTRUCTURE ONLY.

Python wrapper around ``mssm_oracle.c`` (compiled with gcc into
``oracle/libmssm_oracle.so``).  The C core is the plain definition: for every
(batch, channel) chain, h starts at h0 (zero by default, "Understanding Mamba"
section 3.1 starts from h_{-1} = 0), and for t = 0..L-1, n = 0..N-1:

    Abar = exp(delta[b,t,d] * A[d,n])                    eq. (2)
    Bbar = delta[b,t,d] * B[b,t,n]          ("euler", first-order, the form
                                             "Selective State Space Models"
                                             says Mamba uses)
         = (Abar - 1) / A[d,n] * B[b,t,n]   ("zoh", exact zero-order hold,
                                             eq. (2) for diagonal A)
    h[n] = Abar * h[n] + Bbar * x[b,t,d]                 eq. (3)
    y[b,t,d] = sum_n C[b,t,n] * h[n]  (+ Dskip[d] * x)   eq. (3)
    y[b,t,d] *= SiLU(z[b,t,d])        when a gate is given, eq. (9)

All inputs are converted exactly to float64 before the call (float32 and
bfloat16 values are representable in float64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mssm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmssm_oracle.so")
# A test can point the wrapper at another build of the same source (the mutation
# tests build deliberately broken copies to check that the pins catch them).
_LIB_OVERRIDE = os.environ.get("MSSM_ORACLE_LIBRARY")
_lib = None

_BBAR_MODES = {"euler": 0, "zoh": 1}


def build_library() -> str:
    """Compile the C core with gcc (fp64, no fast-math) and return the .so path."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-pthread", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_library():
    """Load the compiled oracle, building it first only if nothing is built."""
    global _lib
    if _lib is not None:
        return _lib
    path = _LIB_OVERRIDE or _LIB_PATH
    if not _LIB_OVERRIDE and not os.path.exists(_LIB_PATH):
        build_library()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_selective_scan.argtypes = [dp] * 10 + [ctypes.c_int64] * 4 + [ctypes.c_int] * 2
    lib.oracle_selective_scan.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(a, shape, name):
    if a is None:
        return None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if arr.shape != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {arr.shape}")
    return arr


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def selective_scan(x, delta, A, B, C, *, bbar: str = "euler", Dskip=None, z=None,
                   h0=None, return_last_state: bool = False, nthreads: int | None = None):
    """Sequential selective scan in fp64.

    Shapes: x, delta, z: [batch, L, D]; A: [D, N]; B, C: [batch, L, N];
    Dskip: [D]; h0: [batch, D, N].  Returns y [batch, L, D] (float64), and the
    final state [batch, D, N] too when ``return_last_state``.

    Pinned by tests/test_oracle_pins.py against the printed examples of
    "Understanding Mamba" (sections 2.3, 3.1, 5.3, 7.2 and the appendix),
    "State Space Models and Mamba" (traced example, Q3, Q4), "Mathematical
    Prerequisites for Mamba" (sections 5-7) and "Mamba and Selective State
    Spaces" (worked example 1), plus closed forms and brute-force forms.
    """
    if bbar not in _BBAR_MODES:
        raise ValueError(f"bbar must be one of {sorted(_BBAR_MODES)}")
    x = np.asarray(x)
    if x.ndim != 3:
        raise ValueError("x must be [batch, L, D]")
    batch, L, D = x.shape
    A = np.asarray(A)
    if A.ndim != 2 or A.shape[0] != D:
        raise ValueError("A must be [D, N]")
    N = A.shape[1]
    xs = _f64(x, (batch, L, D), "x")
    ds = _f64(delta, (batch, L, D), "delta")
    As = _f64(A, (D, N), "A")
    Bs = _f64(B, (batch, L, N), "B")
    Cs = _f64(C, (batch, L, N), "C")
    Dk = _f64(Dskip, (D,), "Dskip")
    zs = _f64(z, (batch, L, D), "z")
    h0s = _f64(h0, (batch, D, N), "h0")
    y = np.zeros((batch, L, D), dtype=np.float64)
    hl = np.zeros((batch, D, N), dtype=np.float64) if return_last_state else None
    if nthreads is None:
        nthreads = min(os.cpu_count() or 1, 16)
    rc = load_library().oracle_selective_scan(
        _ptr(xs), _ptr(ds), _ptr(As), _ptr(Bs), _ptr(Cs), _ptr(Dk), _ptr(zs), _ptr(h0s),
        _ptr(y), _ptr(hl), batch, L, D, N, _BBAR_MODES[bbar], int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_selective_scan failed with code {rc}")
    return (y, hl) if return_last_state else y


def selective_scan_step(h_prev, x_t, delta_t, A, B_t, C_t, *, bbar: str = "euler",
                        Dskip=None, z_t=None):
    """One recurrent step (the O(1)-per-token decode of "Understanding Mamba"
    section 9.1): the scan above with L = 1 and h0 = h_prev.

    Shapes: h_prev [batch, D, N]; x_t, delta_t, z_t [batch, D]; B_t, C_t
    [batch, N].  Returns (y_t [batch, D], h_t [batch, D, N]).
    """
    x_t = np.asarray(x_t, dtype=np.float64)
    batch, D = x_t.shape
    y, h = selective_scan(
        x_t[:, None, :], np.asarray(delta_t, dtype=np.float64)[:, None, :], A,
        np.asarray(B_t, dtype=np.float64)[:, None, :],
        np.asarray(C_t, dtype=np.float64)[:, None, :], bbar=bbar, Dskip=Dskip,
        z=None if z_t is None else np.asarray(z_t, dtype=np.float64)[:, None, :],
        h0=h_prev, return_last_state=True)
    return y[:, 0, :], h
