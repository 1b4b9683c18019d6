"""fp64 CPU oracle for the Orthogonal State Recurrence (OSR).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library.

The arithmetic lives in ``osr_oracle.c`` (plain C, IEEE double), which follows
the token-by-token recurrence of "Lattice: Learning to Efficiently Compress the
Memory" (arXiv 2504.05646): eq. OSR with the forget gate of eq.
dacay_recurrence, the unit-sphere projection of eq. normalized_recurrence, and
the chunk linearisation of eq. recurrence_linear2 (exact when C = 1).  This
module only builds/loads the shared object and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "osr_oracle.c")
_LIB = os.path.join(_HERE, "libosr_oracle.so")

MODE_DEC = 0
MODE_SIM = 1
MODE_ENC = 2

LIN2 = 0  # eq. recurrence_linear2 (default)
LIN1 = 1  # eq. recurrence_linear1

STATUS = {
    0: "ok",
    -1: "null pointer",
    -2: "bad shape",
    -6: "slot of zero norm",
    -7: "out of memory",
}


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("T", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("m", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("gamma_per_slot", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("linearisation", ctypes.c_int32),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math) into oracle/libosr_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
             "-ffp-contract=off", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_osr_forward.argtypes = [ctypes.POINTER(_Problem), dp, dp, dp, dp, dp, dp, dp, dp,
                                           ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
        lib.oracle_osr_forward.restype = ctypes.c_int
        lib.oracle_osr_hardware_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def hardware_threads() -> int:
    return int(_load().oracle_osr_hardware_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def osr_forward(q, k, v, gamma, mu, state, chunk_size: int = 1, mode: int = MODE_DEC,
                nthreads: int = 0, return_threads: bool = False, linearisation: int = LIN2):
    """Run OSR-C over a whole batch in float64.

    q, k: [B,T,H,m]; v: [B,T,H,d]; gamma: [B,T,H,m] or [B,T,H]; mu: [B,T,H];
    state: [B,H,m,d] (row = slot).  Returns (y [B,T,H,d], state_out [B,H,m,d]).
    """
    q, k, v, gamma, mu, state = (_f64(x) for x in (q, k, v, gamma, mu, state))
    B, T, H, m = q.shape
    d = v.shape[-1]
    if k.shape != (B, T, H, m) or v.shape != (B, T, H, d) or mu.shape != (B, T, H) \
            or state.shape != (B, H, m, d):
        raise ValueError("oracle: inconsistent shapes")
    if gamma.shape == (B, T, H, m):
        per_slot = 1
    elif gamma.shape == (B, T, H):
        per_slot = 0
    else:
        raise ValueError("oracle: gamma must be [B,T,H,m] or [B,T,H]")
    prob = _Problem(B, T, H, m, d, per_slot, int(mode), int(chunk_size), int(linearisation))
    y = np.zeros((B, T, H, d), dtype=np.float64)
    out = np.zeros((B, H, m, d), dtype=np.float64)
    used = ctypes.c_int(0)
    rc = _load().oracle_osr_forward(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                    _ptr(mu), _ptr(state), _ptr(out), _ptr(y), int(nthreads),
                                    ctypes.byref(used))
    if rc != 0:
        raise ValueError(f"oracle_osr_forward failed: {rc} ({STATUS.get(rc, '?')})")
    if return_threads:
        return y, out, used.value
    return y, out
