"""fp64 CPU oracle for the Orthogonal State Recurrence (OSR).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library.

The arithmetic lives in ``osr_oracle.c`` (plain C, IEEE double), which follows
the token-by-token recurrence of "Lattice: Learning to Efficiently Compress the
Memory" (arXiv 2504.05646): eq. OSR with the forget gate of eq.
dacay_recurrence, the unit-sphere projection of eq. normalized_recurrence, and
the chunk linearisation of eq. recurrence_linear2 (exact when C = 1).
``osr_glue.c`` holds the layer glue the pages put around the recurrence
(section "Experiments", the Lattice block): the short causal convolution of q
and k, the sigmoid writing intensity and the GeLU post-gate.  This module only
builds/loads the shared object and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "osr_oracle.c")
_SRCS = (_SRC, os.path.join(_HERE, "osr_glue.c"))
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


def _stale() -> bool:
    return not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(s) for s in _SRCS)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math) into oracle/libosr_oracle.so."""
    if force or _stale():
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
             "-ffp-contract=off", "-Wall", "-Wextra", *_SRCS, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _stale():
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_osr_forward.argtypes = [ctypes.POINTER(_Problem), dp, dp, dp, dp, dp, dp, dp, dp,
                                           ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
        lib.oracle_osr_forward.restype = ctypes.c_int
        lib.oracle_osr_hardware_threads.restype = ctypes.c_int
        lib.oracle_glue_conv.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, dp, dp, dp, dp, dp, dp]
        lib.oracle_glue_conv.restype = ctypes.c_int
        lib.oracle_glue_sigmoid.argtypes = [ctypes.c_int64, dp, dp]
        lib.oracle_glue_sigmoid.restype = ctypes.c_int
        lib.oracle_glue_gelu_gate.argtypes = [ctypes.c_int64, dp, dp, dp]
        lib.oracle_glue_gelu_gate.restype = ctypes.c_int
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


# --- layer glue (osr_glue.c): short causal convolution, sigmoid gate, GeLU post-gate ---

CONV_WIDTH = 4


def _optr(a):
    return None if a is None else _ptr(a)


def glue_conv(x, w, b=None, hist=None, return_hist: bool = False):
    """Depthwise causal width-4 convolution along T of x [B,T,N] (any trailing shape
    flattened into N channels), weights w [N,4] (w[:,3] weighs the current token),
    bias b [N] or None, history hist [B,3,N] (oldest first) or None (zeros).
    Returns out [B,T,*] (and the history for the next call, [B,3,*])."""
    x = _f64(x)
    B, T = x.shape[:2]
    tail = x.shape[2:]
    N = int(np.prod(tail)) if tail else 1
    w = _f64(w).reshape(N, CONV_WIDTH)
    b = None if b is None else _f64(b).reshape(N)
    hist = None if hist is None else _f64(hist).reshape(B, CONV_WIDTH - 1, N)
    out = np.zeros((B, T, N), dtype=np.float64)
    hout = np.zeros((B, CONV_WIDTH - 1, N), dtype=np.float64)
    rc = _load().oracle_glue_conv(B, T, N, _ptr(x.reshape(B, T, N)), _ptr(w), _optr(b), _optr(hist),
                                  _ptr(out), _ptr(hout))
    if rc != 0:
        raise ValueError(f"oracle_glue_conv failed: {rc}")
    out = out.reshape((B, T) + tail)
    if return_hist:
        return out, hout.reshape((B, CONV_WIDTH - 1) + tail)
    return out


def glue_sigmoid(logit):
    """gamma = sigmoid(logit), elementwise."""
    x = _f64(logit)
    out = np.zeros_like(x)
    rc = _load().oracle_glue_sigmoid(x.size, _ptr(x), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_glue_sigmoid failed: {rc}")
    return out


def glue_gelu_gate(y, g):
    """out = y * GeLU(g) with the exact GeLU x Phi(x), elementwise."""
    y, g = _f64(y), _f64(g)
    if y.shape != g.shape:
        raise ValueError("oracle: y and g must have one shape")
    out = np.zeros_like(y)
    rc = _load().oracle_glue_gelu_gate(y.size, _ptr(y), _ptr(g), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_glue_gelu_gate failed: {rc}")
    return out


def glue_pre(xq, xk, gamma_logit, wq, wk, bq=None, bk=None, hist_q=None, hist_k=None):
    """The glue before the recurrence: q = conv(xq), k = conv(xk), gamma = sigmoid(logit).
    xq, xk [B,T,H,m]; gamma_logit [B,T,H,m] or [B,T,H]; wq, wk [H,m,4]; bq, bk [H,m];
    hist_q, hist_k [B,3,H,m].  Returns q, k, gamma, hist_q_out, hist_k_out."""
    q, hq = glue_conv(xq, wq, bq, hist_q, return_hist=True)
    k, hk = glue_conv(xk, wk, bk, hist_k, return_hist=True)
    return q, k, glue_sigmoid(gamma_logit), hq, hk
