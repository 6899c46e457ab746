"""CPU oracle for the Mamba-2 SSD selective-scan forward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  It shares
no code with the HIP library and imports nothing from it.

Two independent formulations of the same forward are held here:

* ``ssd_fwd`` / ``chunk_intermediates`` -- the plain per-timestep recurrence
  in fp64, written in C (``ssd_oracle.c``) and called through ctypes;
  ``ssd_bwd`` -- its adjoint (the gradients), step by step, in the same file;
* ``quadratic.ssd_fwd_quadratic`` -- the dual "masked attention" form in
  NumPy fp64 (q = C, k = B, v = dt * x, log-gate dt*A, no 1/sqrt(d) scale),
  written from the flash-linear-attention PR #49 page's mapping between
  simple_gla and the mamba2_ssd kernel.  It is used to pin the recurrence.

Every input is a float32 NumPy array holding the exact fp32 (or bf16) input
values; results are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ssd_oracle.c")
LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")


def compile_library(src: str = SOURCE, dst: str = LIB_PATH) -> str:
    """Compile a C oracle source with gcc (host code only, OpenMP over (b, h))."""
    tmp = dst + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, dst)
    return dst


def build(force: bool = True) -> str:
    """Build ``libssd_oracle.so`` next to its source."""
    if force or not os.path.exists(LIB_PATH):
        compile_library()
    return LIB_PATH


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class OracleLib:
    """ctypes front of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        p, i64, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
        lib.oracle_ssd_fwd.argtypes = ([p] * 8 + [d, d, p, p, p, p] + [i64] * 6 +
                                       [p, ctypes.c_int])
        lib.oracle_ssd_fwd.restype = ctypes.c_int
        lib.oracle_ssd_chunk_intermediates.argtypes = (
            [p] * 5 + [d, d] + [p] * 6 + [i64] * 7 + [ctypes.c_int])
        lib.oracle_ssd_chunk_intermediates.restype = ctypes.c_int
        lib.oracle_ssd_bwd.argtypes = ([p] * 8 + [d, d] + [p] * 13 + [i64] * 6 + [ctypes.c_int])
        lib.oracle_ssd_bwd.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = [ctypes.c_int]
        lib.oracle_max_threads.restype = ctypes.c_int
        self.lib = lib

    def max_threads(self, nthreads: int = 0) -> int:
        return int(self.lib.oracle_max_threads(int(nthreads)))

    def ssd_fwd(self, x, dt, A, B, C, D=None, z=None, dt_bias=None,
                dt_limit=(0.0, float("inf")), initial_states=None, return_final_states=False,
                head_mask=None, nthreads=0, seq_idx=None):
        x, dt, A, B, C = _f32(x), _f32(dt), _f32(A), _f32(B), _f32(C)
        D, z, dt_bias = _f32(D), _f32(z), _f32(dt_bias)
        init = _f64(initial_states)
        seq = _i32(seq_idx)
        b, L, H, P = x.shape
        assert seq is None or seq.shape == (b, L)
        G, N = B.shape[2], B.shape[3]
        assert dt.shape == (b, L, H) and B.shape == (b, L, G, N) and C.shape == B.shape
        assert A.shape == (H,)
        assert z is None or z.shape == x.shape
        assert init is None or init.shape == (b, H, P, N)
        out = np.full((b, L, H, P), np.nan, dtype=np.float64)
        final = np.full((b, H, P, N), np.nan) if return_final_states else None
        mask = None
        if head_mask is not None:
            mask = np.ascontiguousarray(np.asarray(head_mask, dtype=np.uint8).reshape(b, H))
        rc = self.lib.oracle_ssd_fwd(
            _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
            float(dt_limit[0]), float(dt_limit[1]), _ptr(init), _ptr(out), _ptr(final),
            _ptr(seq), b, L, H, P, N, G, _ptr(mask), int(nthreads))
        if rc != 0:
            raise ValueError("oracle_ssd_fwd rejected the shapes")
        return (out, final) if return_final_states else out

    def ssd_bwd(self, x, dt, A, B, C, dout, D=None, z=None, dt_bias=None,
                dt_limit=(0.0, float("inf")), initial_states=None, dfinal=None, seq_idx=None,
                nthreads=0):
        x, dt, A, B, C = _f32(x), _f32(dt), _f32(A), _f32(B), _f32(C)
        D, z, dt_bias = _f32(D), _f32(z), _f32(dt_bias)
        init, dout, dfinal = _f64(initial_states), _f64(dout), _f64(dfinal)
        seq = _i32(seq_idx)
        b, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        assert dout.shape == x.shape and (dfinal is None or dfinal.shape == (b, H, P, N))
        g = {"dx": np.zeros((b, L, H, P)), "dz": np.zeros((b, L, H, P)),
             "ddt": np.zeros((b, L, H)), "dA": np.zeros(H), "dB": np.zeros((b, L, G, N)),
             "dC": np.zeros((b, L, G, N)), "dD": np.zeros(H), "ddt_bias": np.zeros(H),
             "dinitial_states": np.zeros((b, H, P, N))}
        rc = self.lib.oracle_ssd_bwd(
            _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
            float(dt_limit[0]), float(dt_limit[1]), _ptr(init), _ptr(seq), _ptr(dout),
            _ptr(dfinal), _ptr(g["dx"]), _ptr(g["dz"]), _ptr(g["ddt"]), _ptr(g["dA"]),
            _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["ddt_bias"]),
            _ptr(g["dinitial_states"]), b, L, H, P, N, G, int(nthreads))
        if rc != 0:
            raise ValueError("oracle_ssd_bwd rejected the shapes")
        if z is None:
            g["dz"] = None
        return g

    def chunk_intermediates(self, x, dt, A, B, chunk_size, dt_bias=None,
                            dt_limit=(0.0, float("inf")), initial_states=None, nthreads=0,
                            seq_idx=None):
        x, dt, A, B, dt_bias = _f32(x), _f32(dt), _f32(A), _f32(B), _f32(dt_bias)
        init = _f64(initial_states)
        seq = _i32(seq_idx)
        b, L, H, P = x.shape
        assert seq is None or seq.shape == (b, L)
        G, N = B.shape[2], B.shape[3]
        Q = int(chunk_size)
        nc = (L + Q - 1) // Q
        res = {
            "dt": np.zeros((b, H, nc, Q)),
            "cum": np.zeros((b, H, nc, Q)),
            "chunk_states": np.zeros((b, nc, H, P, N)),
            "states_in": np.zeros((b, nc, H, P, N)),
        }
        rc = self.lib.oracle_ssd_chunk_intermediates(
            _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(dt_bias), float(dt_limit[0]),
            float(dt_limit[1]), _ptr(init), _ptr(res["dt"]), _ptr(res["cum"]),
            _ptr(res["chunk_states"]), _ptr(res["states_in"]), _ptr(seq), b, L, H, P, N, G, Q,
            int(nthreads))
        if rc != 0:
            raise ValueError("oracle_ssd_chunk_intermediates rejected the shapes")
        return res


_default = None


def _lib() -> OracleLib:
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        _default = OracleLib(LIB_PATH)
    return _default


def max_threads(nthreads: int = 0) -> int:
    """Threads the oracle's OpenMP loop uses (after setting ``nthreads`` if > 0)."""
    return _lib().max_threads(nthreads)


def ssd_fwd(*args, **kwargs):
    """Plain recurrence.  x [b,L,H,P], dt [b,L,H], A/D/dt_bias [H], B/C [b,L,G,N],
    z like x, initial_states [b,H,P,N], seq_idx [b,L] int32 (the state resets
    where it changes).  Returns out [b,L,H,P] fp64 (and, with
    ``return_final_states``, the final state [b,H,P,N] fp64).  ``head_mask``
    [b,H] restricts the work to some (b, h) pairs; other outputs are NaN."""
    return _lib().ssd_fwd(*args, **kwargs)


def ssd_bwd(*args, **kwargs):
    """Gradients of sum(dout * out) + sum(dfinal * final) with respect to every
    input of ``ssd_fwd``: a dict with dx, dz (None without z), ddt (for dt_raw),
    dA, dB, dC, dD, ddt_bias and dinitial_states, fp64."""
    return _lib().ssd_bwd(*args, **kwargs)


def chunk_intermediates(*args, **kwargs):
    """Per-chunk intermediates (definitions in ssd_oracle.c): a dict with ``dt``
    and ``cum`` [b,H,nc,Q] and ``chunk_states``, ``states_in`` [b,nc,H,P,N]."""
    return _lib().chunk_intermediates(*args, **kwargs)
