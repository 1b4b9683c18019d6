"""Python binding of liblattice_osr.so (include/lattice_osr.h).

Argument marshalling only: every step of the recurrence runs in the library's
HIP kernels.  Tensors are PyTorch device tensors (PyTorch provides device
memory and the stream); the functions keep the C entry points' names.

If the library has not been built (``python -m compressed_memory_linear_amd.build``)
the first call raises; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblattice_osr.so")

F32, BF16 = 0, 1
MODE_DEC, MODE_SIM, MODE_ENC = 0, 1, 2
LIN2, LIN1 = 0, 1

OK = 0
ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH, ERR_ALIAS, ERR_ALIGN = -1, -2, -3, -4, -5, -6, -7

EXPORTED = ("lattice_osr_fwd_chunked", "lattice_osr_fwd_recurrent", "lattice_osr_decode_step",
            "lattice_osr_workspace_bytes", "lattice_osr_status_string", "lattice_osr_abi_version",
            "lattice_osr_bwd_chunked", "lattice_osr_bwd_workspace_bytes", "lattice_osr_glue_pre",
            "lattice_osr_glue_post")


class lattice_osr_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "H", "m", "d", "gamma_per_slot", "in_dtype", "y_dtype", "mode", "linearisation")]


class OSRError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


_lib = None


def load_library():
    """Load liblattice_osr.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m compressed_memory_linear_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, dp = ctypes.c_void_p, ctypes.POINTER(lattice_osr_desc)
        fwd = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.lattice_osr_fwd_chunked.argtypes = [dp, ctypes.c_int32] + fwd[1:]
        lib.lattice_osr_fwd_recurrent.argtypes = fwd
        lib.lattice_osr_decode_step.argtypes = fwd
        for f in ("lattice_osr_fwd_chunked", "lattice_osr_fwd_recurrent", "lattice_osr_decode_step"):
            getattr(lib, f).restype = ctypes.c_int
        lib.lattice_osr_bwd_chunked.argtypes = [dp, ctypes.c_int32] + [vp] * 15 + [ctypes.c_size_t, vp]
        lib.lattice_osr_bwd_chunked.restype = ctypes.c_int
        lib.lattice_osr_bwd_workspace_bytes.argtypes = [dp, ctypes.c_int32]
        lib.lattice_osr_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.lattice_osr_workspace_bytes.argtypes = [dp, ctypes.c_int32]
        lib.lattice_osr_workspace_bytes.restype = ctypes.c_size_t
        lib.lattice_osr_glue_pre.argtypes = [dp] + [vp] * 15
        lib.lattice_osr_glue_pre.restype = ctypes.c_int
        lib.lattice_osr_glue_post.argtypes = [dp, vp, vp, vp, vp]
        lib.lattice_osr_glue_post.restype = ctypes.c_int
        lib.lattice_osr_status_string.argtypes = [ctypes.c_int]
        lib.lattice_osr_status_string.restype = ctypes.c_char_p
        lib.lattice_osr_abi_version.argtypes = []
        lib.lattice_osr_abi_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def lattice_osr_abi_version() -> int:
    return int(load_library().lattice_osr_abi_version())


def status_string(status: int) -> str:
    return load_library().lattice_osr_status_string(int(status)).decode()


lattice_osr_status_string = status_string


def make_desc(B, T, H, m, d, gamma_per_slot=1, in_dtype=BF16, y_dtype=F32, mode=MODE_DEC, linearisation=LIN2):
    return lattice_osr_desc(B, T, H, m, d, gamma_per_slot, in_dtype, y_dtype, mode, linearisation)


def lattice_osr_workspace_bytes(desc: lattice_osr_desc, chunk_size: int) -> int:
    n = int(load_library().lattice_osr_workspace_bytes(ctypes.byref(desc), int(chunk_size)))
    if n == ctypes.c_size_t(-1).value:
        raise OSRError(ERR_SHAPE, "lattice_osr_workspace_bytes")
    return n


# ------------------------------------------------------------ marshalling --
_DT = {torch.float32: F32, torch.bfloat16: BF16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _desc_from(q, k, v, gamma, mu, state_in, y_dtype, mode, linearisation=0) -> lattice_osr_desc:
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q/k/gamma are [B,T,H,m], v is [B,T,H,d]")
    B, T, H, m = q.shape
    d = v.shape[-1]
    if q.dtype not in _DT:
        raise ValueError("inputs must be float32 or bfloat16")
    for t in (q, k, v, gamma, mu):
        if t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError("q, k, v, gamma, mu must share dtype/device and be contiguous")
    if state_in.dtype != torch.float32 or not state_in.is_contiguous():
        raise ValueError("state must be contiguous float32 [B,H,m,d]")
    per_slot = 1 if gamma.dim() == 4 else 0
    return make_desc(B, T, H, m, d, per_slot, _DT[q.dtype], _DT[y_dtype], mode, linearisation)


def _outputs(desc, q, state_in, state_out, y, y_dtype):
    if y is None:
        y = torch.empty((desc.B, desc.T, desc.H, desc.d), dtype=y_dtype, device=q.device)
    if state_out is None:
        state_out = torch.empty_like(state_in)
    return state_out, y


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def lattice_osr_fwd_chunked(q, k, v, gamma, mu, state_in, chunk_size: int, *, mode: int = MODE_DEC,
                            y_dtype=torch.float32, state_out=None, y=None, workspace=None,
                            stream=None, linearisation: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunk-wise OSR forward.  Returns (y [B,T,H,d], state_out [B,H,m,d]).
    linearisation: LIN2 (default, eq. recurrence_linear2) or LIN1."""
    lib = load_library()
    desc = _desc_from(q, k, v, gamma, mu, state_in, y_dtype, mode, linearisation)
    state_out, y = _outputs(desc, q, state_in, state_out, y, y_dtype)
    need = lattice_osr_workspace_bytes(desc, chunk_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.lattice_osr_fwd_chunked(ctypes.byref(desc), int(chunk_size), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(gamma), _ptr(mu), _ptr(state_in), _ptr(state_out), _ptr(y),
                                     _ptr(workspace), wbytes, _stream(stream))
    if rc != OK:
        raise OSRError(rc, "lattice_osr_fwd_chunked")
    return y, state_out


def lattice_osr_fwd_recurrent(q, k, v, gamma, mu, state_in, *, mode: int = MODE_DEC,
                              y_dtype=torch.float32, state_out=None, y=None,
                              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Exact token-by-token OSR forward.  Returns (y, state_out)."""
    lib = load_library()
    desc = _desc_from(q, k, v, gamma, mu, state_in, y_dtype, mode)
    state_out, y = _outputs(desc, q, state_in, state_out, y, y_dtype)
    rc = lib.lattice_osr_fwd_recurrent(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                       _ptr(mu), _ptr(state_in), _ptr(state_out), _ptr(y), None, 0,
                                       _stream(stream))
    if rc != OK:
        raise OSRError(rc, "lattice_osr_fwd_recurrent")
    return y, state_out


def lattice_osr_decode_step(q, k, v, gamma, mu, state_in, *, mode: int = MODE_DEC,
                            y_dtype=torch.float32, state_out=None, y=None,
                            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One exact decode step (T = 1); state_out may be state_in (in place)."""
    lib = load_library()
    desc = _desc_from(q, k, v, gamma, mu, state_in, y_dtype, mode)
    state_out, y = _outputs(desc, q, state_in, state_out, y, y_dtype)
    rc = lib.lattice_osr_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                     _ptr(mu), _ptr(state_in), _ptr(state_out), _ptr(y), None, 0,
                                     _stream(stream))
    if rc != OK:
        raise OSRError(rc, "lattice_osr_decode_step")
    return y, state_out


def lattice_osr_bwd_workspace_bytes(desc: lattice_osr_desc, chunk_size: int) -> int:
    n = int(load_library().lattice_osr_bwd_workspace_bytes(ctypes.byref(desc), int(chunk_size)))
    if n == ctypes.c_size_t(-1).value:
        raise OSRError(ERR_UNSUPPORTED, "lattice_osr_bwd_workspace_bytes")
    return n


def lattice_osr_bwd_chunked(q, k, v, gamma, mu, state_in, dy, dstate_out, chunk_size: int, *,
                            mode: int = MODE_DEC, grads: Optional[dict] = None, workspace=None,
                            stream=None, linearisation: int = LIN2) -> dict:
    """Backward of the chunk-wise forward: gradients of sum(dy*y) +
    sum(dstate_out*state_out) with respect to q, k, v, gamma, mu and
    state_in.  dy has y's shape (float32 or bfloat16), dstate_out the state's.
    Returns a dict of float32 tensors dq, dk, dv, dgamma, dmu, dstate_in
    (allocated unless passed in `grads`)."""
    lib = load_library()
    desc = _desc_from(q, k, v, gamma, mu, state_in, dy.dtype, mode, linearisation)
    if not dy.is_contiguous() or dy.shape != v.shape or dy.device != q.device:
        raise ValueError("dy must be contiguous with v's shape")
    if dstate_out.dtype != torch.float32 or not dstate_out.is_contiguous() or dstate_out.shape != state_in.shape:
        raise ValueError("dstate_out must be contiguous float32 with the state's shape")
    if grads is None:
        grads = {"d" + n: torch.empty(t.shape, dtype=torch.float32, device=q.device)
                 for n, t in (("q", q), ("k", k), ("v", v), ("gamma", gamma), ("mu", mu),
                              ("state_in", state_in))}
    need = lattice_osr_bwd_workspace_bytes(desc, chunk_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    g = grads
    rc = lib.lattice_osr_bwd_chunked(ctypes.byref(desc), int(chunk_size), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(gamma), _ptr(mu), _ptr(state_in), _ptr(dy), _ptr(dstate_out),
                                     _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dgamma"]),
                                     _ptr(g["dmu"]), _ptr(g["dstate_in"]), _ptr(workspace), wbytes,
                                     _stream(stream))
    if rc != OK:
        raise OSRError(rc, "lattice_osr_bwd_chunked")
    return grads


# ------------------------------------------------------------ host inputs --
def lattice_osr_glue_pre(xq, xk, gamma_logit, conv_wq, conv_wk, conv_bq=None, conv_bk=None, hist_q=None,
                         hist_k=None, *, q=None, k=None, gamma=None, hist_q_out=None, hist_k_out=None,
                         return_history: bool = False, stream=None):
    """q = conv4(xq), k = conv4(xk), gamma = sigmoid(gamma_logit) in one pass.

    xq, xk [B,T,H,m] and gamma_logit [B,T,H,m] or [B,T,H] share a dtype (float32 or
    bfloat16); conv_w* [H,m,4] and conv_b* [H,m] are float32; hist_* [B,3,H,m] carry
    the three raw rows before this call.  Returns (q, k, gamma) and, with
    return_history, also the history for the next call."""
    lib = load_library()
    if xq.dim() != 4 or xq.dtype not in _DT:
        raise ValueError("xq/xk are [B,T,H,m] float32 or bfloat16")
    B, T, H, m = xq.shape
    for t in (xk, gamma_logit):
        if t.dtype != xq.dtype or not t.is_contiguous() or t.device != xq.device:
            raise ValueError("xq, xk, gamma_logit must share dtype/device and be contiguous")
    for t in (conv_wq, conv_wk, conv_bq, conv_bk):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("convolution weights and biases are contiguous float32")
    per_slot = 1 if gamma_logit.dim() == 4 else 0
    desc = make_desc(B, T, H, m, m, per_slot, _DT[xq.dtype], F32)
    q = torch.empty_like(xq) if q is None else q
    k = torch.empty_like(xk) if k is None else k
    gamma = torch.empty_like(gamma_logit) if gamma is None else gamma
    if return_history:
        hist_q_out = xq.new_empty((B, 3, H, m)) if hist_q_out is None else hist_q_out
        hist_k_out = xk.new_empty((B, 3, H, m)) if hist_k_out is None else hist_k_out
    rc = lib.lattice_osr_glue_pre(ctypes.byref(desc), _ptr(xq), _ptr(xk), _ptr(gamma_logit), _ptr(conv_wq),
                                  _ptr(conv_wk), _ptr(conv_bq), _ptr(conv_bk), _ptr(hist_q), _ptr(hist_k),
                                  _ptr(q), _ptr(k), _ptr(gamma), _ptr(hist_q_out), _ptr(hist_k_out),
                                  _stream(stream))
    if rc != OK:
        raise OSRError(rc, "lattice_osr_glue_pre")
    if return_history:
        return q, k, gamma, hist_q_out, hist_k_out
    return q, k, gamma


def lattice_osr_glue_post(y, gate, *, out=None, stream=None):
    """out = y * GeLU(gate) (exact GeLU); y [B,T,H,d] float32 or bfloat16, gate of y's shape in
    float32 or bfloat16.  out may be y (in place)."""
    lib = load_library()
    if y.dim() != 4 or y.dtype not in _DT or gate.dtype not in _DT or gate.shape != y.shape:
        raise ValueError("y and gate are [B,T,H,d] float32 or bfloat16 tensors of one shape")
    if not (y.is_contiguous() and gate.is_contiguous()):
        raise ValueError("y and gate must be contiguous")
    B, T, H, d = y.shape
    desc = make_desc(B, T, H, 16, d, 1, _DT[gate.dtype], _DT[y.dtype])
    out = torch.empty_like(y) if out is None else out
    rc = lib.lattice_osr_glue_post(ctypes.byref(desc), _ptr(y), _ptr(gate), _ptr(out), _stream(stream))
    if rc != OK:
        raise OSRError(rc, "lattice_osr_glue_post")
    return out


def to_device(inp, device="cuda") -> dict:
    """Move an OSRInputs batch (numpy, storage form) to device tensors.

    bf16 bit patterns become torch.bfloat16 tensors with the same bits.
    """
    out = {}
    for name in ("q", "k", "v", "gamma", "mu"):
        a = getattr(inp, name)
        t = torch.from_numpy(a.copy())
        if a.dtype.itemsize == 2:
            t = t.view(torch.bfloat16)
        out[name] = t.to(device)
    out["state"] = torch.from_numpy(inp.state.copy()).to(device)
    return out
