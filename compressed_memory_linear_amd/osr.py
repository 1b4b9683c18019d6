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
SCHED_AUTO, SCHED_SPLIT, SCHED_FUSED = 0, 1, 2
PAIRS_AUTO, PAIRS_OFF = 0, 1
WGS_AUTO, WGS_ONE = 0, 1
OVERLAP_AUTO, OVERLAP_OFF = 0, 1
BWD_AUTO, BWD_WALK, BWD_CHUNK = 0, 1, 2

OK = 0
ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH, ERR_ALIAS, ERR_ALIGN = -1, -2, -3, -4, -5, -6, -7

EXPORTED = ("lattice_osr_fwd_chunked", "lattice_osr_fwd_recurrent", "lattice_osr_decode_step",
            "lattice_osr_workspace_bytes", "lattice_osr_status_string", "lattice_osr_abi_version",
            "lattice_osr_bwd_chunked", "lattice_osr_bwd_workspace_bytes", "lattice_osr_glue_pre",
            "lattice_osr_glue_post", "lattice_osr_fwd_chunked_gated", "lattice_osr_fwd_chunked_noalloc",
            "lattice_osr_fwd_chunked_save", "lattice_osr_bwd_chunked_saved")
NOALLOC_SCRATCH_BYTES = 64 << 20


class lattice_osr_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "H", "m", "d", "gamma_per_slot", "in_dtype", "y_dtype", "mode", "linearisation",
                 "schedule", "chain_pairs", "chain_wgs", "readout_overlap", "bwd_form")]


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
        lib.lattice_osr_fwd_chunked_gated.argtypes = [dp, ctypes.c_int32] + [vp] * 6 + fwd[6:]
        lib.lattice_osr_fwd_chunked_gated.restype = ctypes.c_int
        lib.lattice_osr_fwd_chunked_noalloc.argtypes = [dp, ctypes.c_int32] + [vp] * 9
        lib.lattice_osr_fwd_chunked_noalloc.restype = ctypes.c_int
        lib.lattice_osr_fwd_recurrent.argtypes = fwd
        lib.lattice_osr_decode_step.argtypes = fwd
        for f in ("lattice_osr_fwd_chunked", "lattice_osr_fwd_recurrent", "lattice_osr_decode_step"):
            getattr(lib, f).restype = ctypes.c_int
        lib.lattice_osr_bwd_chunked.argtypes = [dp, ctypes.c_int32] + [vp] * 15 + [ctypes.c_size_t, vp]
        lib.lattice_osr_bwd_chunked.restype = ctypes.c_int
        lib.lattice_osr_bwd_chunked_saved.argtypes = [dp, ctypes.c_int32] + [vp] * 15 + [ctypes.c_size_t, vp]
        lib.lattice_osr_bwd_chunked_saved.restype = ctypes.c_int
        lib.lattice_osr_fwd_chunked_save.argtypes = [dp, ctypes.c_int32] + fwd[1:]
        lib.lattice_osr_fwd_chunked_save.restype = ctypes.c_int
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


def make_desc(B, T, H, m, d, gamma_per_slot=1, in_dtype=BF16, y_dtype=F32, mode=MODE_DEC, linearisation=LIN2,
              schedule=SCHED_AUTO, chain_pairs=PAIRS_AUTO, chain_wgs=WGS_AUTO, readout_overlap=OVERLAP_AUTO,
              bwd_form=BWD_AUTO):
    return lattice_osr_desc(B, T, H, m, d, gamma_per_slot, in_dtype, y_dtype, mode, linearisation, schedule,
                            chain_pairs, chain_wgs, readout_overlap, bwd_form)


def lattice_osr_workspace_bytes(desc: lattice_osr_desc, chunk_size: int) -> int:
    n = int(load_library().lattice_osr_workspace_bytes(ctypes.byref(desc), int(chunk_size)))
    if n == ctypes.c_size_t(-1).value:
        raise OSRError(ERR_SHAPE, "lattice_osr_workspace_bytes")
    return n


# ------------------------------------------------------------ marshalling --
_DT = {torch.float32: F32, torch.bfloat16: BF16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _shape_error(name, t, want):
    raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(want)}")


def _check_tensor(name, t, shape, dtype, device=None):
    """Shape, dtype and layout of one argument, then its device: the kernels
    index every buffer by the descriptor's sizes, so a mismatch would read or
    write past it on the GPU."""
    if tuple(t.shape) != tuple(shape):
        _shape_error(name, t, shape)
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} is {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_cuda(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("every tensor argument must be a GPU (cuda) tensor")


def _desc_from(q, k, v, gamma, mu, state_in, y_dtype, mode, linearisation=0, schedule=SCHED_AUTO,
               chain_pairs=PAIRS_AUTO, chain_wgs=WGS_AUTO, readout_overlap=OVERLAP_AUTO,
               bwd_form=BWD_AUTO) -> lattice_osr_desc:
    """Descriptor of a forward call, after checking every input against it:
    q, k [B,T,H,m]; v [B,T,H,d]; gamma [B,T,H,m] or [B,T,H]; mu [B,T,H]
    (all one dtype, float32 or bfloat16); state_in [B,H,m,d] float32; all
    contiguous, on one GPU."""
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q/k/gamma are [B,T,H,m], v is [B,T,H,d]")
    B, T, H, m = q.shape
    d = v.shape[-1]
    if q.dtype not in _DT:
        raise ValueError("inputs must be float32 or bfloat16")
    if y_dtype not in _DT:
        raise ValueError("y_dtype must be torch.float32 or torch.bfloat16")
    per_slot = 1 if gamma.dim() == 4 else 0
    _check_tensor("q", q, (B, T, H, m), q.dtype)
    _check_tensor("k", k, (B, T, H, m), q.dtype, q.device)
    _check_tensor("v", v, (B, T, H, d), q.dtype, q.device)
    _check_tensor("gamma", gamma, (B, T, H, m) if per_slot else (B, T, H), q.dtype, q.device)
    _check_tensor("mu", mu, (B, T, H), q.dtype, q.device)
    _check_tensor("state_in", state_in, (B, H, m, d), torch.float32, q.device)
    return make_desc(B, T, H, m, d, per_slot, _DT[q.dtype], _DT[y_dtype], mode, linearisation, schedule,
                     chain_pairs, chain_wgs, readout_overlap, bwd_form)


def _check_outputs(desc, q, state_in, state_out, y, y_dtype):
    """Caller-supplied outputs against the descriptor, then the device of
    every tensor."""
    if y is not None:
        _check_tensor("y", y, (desc.B, desc.T, desc.H, desc.d), y_dtype, q.device)
    if state_out is not None:
        _check_tensor("state_out", state_out, tuple(state_in.shape), torch.float32, q.device)
    _check_cuda(q)


def _outputs(desc, q, state_in, state_out, y, y_dtype):
    """Missing outputs are allocated (on the current stream, which the caller
    has set to the launch stream)."""
    if y is None:
        y = torch.empty((desc.B, desc.T, desc.H, desc.d), dtype=y_dtype, device=q.device)
    if state_out is None:
        state_out = torch.empty_like(state_in)
    return state_out, y


def _workspace(workspace, need, device):
    """The caller's workspace (a uint8 tensor on the inputs' device) or a new
    one of `need` bytes; returns (tensor or None, its size in bytes)."""
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    elif not workspace.is_contiguous() or workspace.device != device:
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return workspace, workspace.numel() * workspace.element_size()


def _launch_stream(stream):
    """The stream to launch on.  Temporaries (outputs, workspace) are
    allocated under it: the caching allocator then reuses their memory only
    in that stream's order, after the kernels that use it."""
    return torch.cuda.current_stream() if stream is None else stream


def lattice_osr_fwd_chunked(q, k, v, gamma, mu, state_in, chunk_size: int, *, mode: int = MODE_DEC,
                            y_dtype=torch.float32, state_out=None, y=None, workspace=None,
                            stream=None, linearisation: int = 0, schedule: int = SCHED_AUTO,
                            chain_pairs: int = PAIRS_AUTO, chain_wgs: int = WGS_AUTO,
                            readout_overlap: int = OVERLAP_AUTO) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunk-wise OSR forward.  Returns (y [B,T,H,d], state_out [B,H,m,d]).
    linearisation: LIN2 (default, eq. recurrence_linear2) or LIN1.
    schedule / chain_pairs / chain_wgs / readout_overlap: the matrix-core
    schedule (speed only)."""
    lib = load_library()
    desc = _desc_from(q, k, v, gamma, mu, state_in, y_dtype, mode, linearisation, schedule, chain_pairs, chain_wgs,
                      readout_overlap)
    _check_outputs(desc, q, state_in, state_out, y, y_dtype)
    st = _launch_stream(stream)
    with torch.cuda.stream(st):
        state_out, y = _outputs(desc, q, state_in, state_out, y, y_dtype)
        need = lattice_osr_workspace_bytes(desc, chunk_size)
        workspace, wbytes = _workspace(workspace, need, q.device)
        rc = lib.lattice_osr_fwd_chunked(ctypes.byref(desc), int(chunk_size), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(gamma), _ptr(mu), _ptr(state_in), _ptr(state_out), _ptr(y),
                                         _ptr(workspace), wbytes, st.cuda_stream)
    if rc != OK:
        raise OSRError(rc, "lattice_osr_fwd_chunked")
    return y, state_out


def lattice_osr_fwd_chunked_gated(q, k, v, gamma, mu, gate, state_in, chunk_size: int, *, mode: int = MODE_DEC,
                                  y_dtype=torch.float32, state_out=None, y=None, workspace=None, stream=None,
                                  linearisation: int = 0, schedule: int = SCHED_AUTO, chain_pairs: int = PAIRS_AUTO,
                                  chain_wgs: int = WGS_AUTO,
                                  readout_overlap: int = OVERLAP_AUTO) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunk-wise OSR forward with the GeLU post-gate fused into the output:
    y = OSR(...) * GeLU(gate), gate [B,T,H,d] in the inputs' dtype.
    Returns (y, state_out)."""
    lib = load_library()
    desc = _desc_from(q, k, v, gamma, mu, state_in, y_dtype, mode, linearisation, schedule, chain_pairs, chain_wgs,
                      readout_overlap)
    _check_tensor("gate", gate, tuple(v.shape), q.dtype, q.device)
    _check_outputs(desc, q, state_in, state_out, y, y_dtype)
    st = _launch_stream(stream)
    with torch.cuda.stream(st):
        state_out, y = _outputs(desc, q, state_in, state_out, y, y_dtype)
        need = lattice_osr_workspace_bytes(desc, chunk_size)
        workspace, wbytes = _workspace(workspace, need, q.device)
        rc = lib.lattice_osr_fwd_chunked_gated(ctypes.byref(desc), int(chunk_size), _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(gamma), _ptr(mu), _ptr(gate), _ptr(state_in), _ptr(state_out),
                                               _ptr(y), _ptr(workspace), wbytes, st.cuda_stream)
    if rc != OK:
        raise OSRError(rc, "lattice_osr_fwd_chunked_gated")
    return y, state_out


def lattice_osr_fwd_chunked_noalloc(q, k, v, gamma, mu, state_in, chunk_size: int, *, state_out, y,
                                    mode: int = MODE_DEC, stream=None, linearisation: int = 0,
                                    schedule: int = SCHED_AUTO, chain_pairs: int = PAIRS_AUTO,
                                    chain_wgs: int = WGS_AUTO) -> Tuple[torch.Tensor, torch.Tensor]:
    """lattice_osr_fwd_chunked without a workspace: the library's per-GPU
    scratch holds it (at most NOALLOC_SCRATCH_BYTES).  The caller passes the
    outputs (y with y's dtype, state_out); nothing is allocated.  Calls that
    overlap on one GPU race on the scratch.  The read-out never overlaps
    here (all work on the one stream)."""
    lib = load_library()
    desc = _desc_from(q, k, v, gamma, mu, state_in, y.dtype, mode, linearisation, schedule, chain_pairs, chain_wgs)
    _check_outputs(desc, q, state_in, state_out, y, y.dtype)
    st = _launch_stream(stream)
    rc = lib.lattice_osr_fwd_chunked_noalloc(ctypes.byref(desc), int(chunk_size), _ptr(q), _ptr(k), _ptr(v),
                                             _ptr(gamma), _ptr(mu), _ptr(state_in), _ptr(state_out), _ptr(y),
                                             st.cuda_stream)
    if rc != OK:
        raise OSRError(rc, "lattice_osr_fwd_chunked_noalloc")
    return y, state_out


def lattice_osr_fwd_recurrent(q, k, v, gamma, mu, state_in, *, mode: int = MODE_DEC,
                              y_dtype=torch.float32, state_out=None, y=None,
                              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Exact token-by-token OSR forward.  Returns (y, state_out)."""
    lib = load_library()
    desc = _desc_from(q, k, v, gamma, mu, state_in, y_dtype, mode)
    _check_outputs(desc, q, state_in, state_out, y, y_dtype)
    st = _launch_stream(stream)
    with torch.cuda.stream(st):
        state_out, y = _outputs(desc, q, state_in, state_out, y, y_dtype)
        rc = lib.lattice_osr_fwd_recurrent(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                           _ptr(mu), _ptr(state_in), _ptr(state_out), _ptr(y), None, 0,
                                           st.cuda_stream)
    if rc != OK:
        raise OSRError(rc, "lattice_osr_fwd_recurrent")
    return y, state_out


def lattice_osr_decode_step(q, k, v, gamma, mu, state_in, *, mode: int = MODE_DEC,
                            y_dtype=torch.float32, state_out=None, y=None,
                            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One exact decode step (T = 1); state_out may be state_in (in place)."""
    lib = load_library()
    desc = _desc_from(q, k, v, gamma, mu, state_in, y_dtype, mode)
    _check_outputs(desc, q, state_in, state_out, y, y_dtype)
    st = _launch_stream(stream)
    with torch.cuda.stream(st):
        state_out, y = _outputs(desc, q, state_in, state_out, y, y_dtype)
        rc = lib.lattice_osr_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                         _ptr(mu), _ptr(state_in), _ptr(state_out), _ptr(y), None, 0,
                                         st.cuda_stream)
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
                            stream=None, linearisation: int = LIN2, chain_wgs: int = WGS_AUTO,
                            bwd_form: int = BWD_AUTO) -> dict:
    """Backward of the chunk-wise forward: gradients of sum(dy*y) +
    sum(dstate_out*state_out) with respect to q, k, v, gamma, mu and
    state_in.  dy has y's shape (float32 or bfloat16), dstate_out the state's.
    Returns a dict of float32 tensors dq, dk, dv, dgamma, dmu, dstate_in
    (allocated unless passed in `grads`).  chain_wgs: WGS_ONE keeps each
    sequence of the token walk on one workgroup (speed only); bwd_form:
    BWD_WALK / BWD_CHUNK pick the backward's form (BWD_AUTO: the chunk form
    where it is built)."""
    return _bwd("lattice_osr_bwd_chunked", q, k, v, gamma, mu, state_in, dy, dstate_out, chunk_size, mode, grads,
                workspace, stream, linearisation, chain_wgs, bwd_form)


def lattice_osr_fwd_chunked_save(q, k, v, gamma, mu, state_in, chunk_size: int, *, mode: int = MODE_DEC,
                                 y_dtype=torch.float32, state_out=None, y=None, saved=None, stream=None,
                                 chain_wgs: int = WGS_AUTO, linearisation: int = LIN2):
    """The chunk-wise forward (small-chunk backward form only: C in 1, 2, 4, 8)
    that also stores what lattice_osr_bwd_chunked_saved needs.  Returns (y,
    state_out, saved); saved is a uint8 tensor of
    lattice_osr_bwd_workspace_bytes bytes (allocated unless passed), to be
    passed as that call's `saved`."""
    lib = load_library()
    desc = _desc_from(q, k, v, gamma, mu, state_in, y_dtype, mode, linearisation, chain_wgs=chain_wgs)
    _check_outputs(desc, q, state_in, state_out, y, y_dtype)
    st = _launch_stream(stream)
    with torch.cuda.stream(st):
        state_out, y = _outputs(desc, q, state_in, state_out, y, y_dtype)
        need = lattice_osr_bwd_workspace_bytes(desc, chunk_size)
        saved, sbytes = _workspace(saved, need, q.device)
        rc = lib.lattice_osr_fwd_chunked_save(ctypes.byref(desc), int(chunk_size), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(gamma), _ptr(mu), _ptr(state_in), _ptr(state_out), _ptr(y),
                                              _ptr(saved), sbytes, st.cuda_stream)
    if rc != OK:
        raise OSRError(rc, "lattice_osr_fwd_chunked_save")
    return y, state_out, saved


def lattice_osr_bwd_chunked_saved(q, k, v, gamma, mu, state_in, dy, dstate_out, chunk_size: int, *, saved,
                                  mode: int = MODE_DEC, grads: Optional[dict] = None, stream=None,
                                  chain_wgs: int = WGS_AUTO, linearisation: int = LIN2) -> dict:
    """lattice_osr_bwd_chunked's gradients, bit for bit, from the values a
    lattice_osr_fwd_chunked_save call with the same inputs stored in `saved`
    (its forward pass skipped)."""
    if saved is None:
        raise ValueError("saved: the tensor lattice_osr_fwd_chunked_save returned")
    return _bwd("lattice_osr_bwd_chunked_saved", q, k, v, gamma, mu, state_in, dy, dstate_out, chunk_size, mode,
                grads, saved, stream, linearisation, chain_wgs, BWD_AUTO)


def _bwd(entry, q, k, v, gamma, mu, state_in, dy, dstate_out, chunk_size, mode, grads, workspace, stream,
         linearisation, chain_wgs, bwd_form) -> dict:
    lib = load_library()
    desc = _desc_from(q, k, v, gamma, mu, state_in, dy.dtype, mode, linearisation, chain_wgs=chain_wgs,
                      bwd_form=bwd_form)
    _check_tensor("dy", dy, tuple(v.shape), None, q.device)
    _check_tensor("dstate_out", dstate_out, tuple(state_in.shape), torch.float32, q.device)
    named = (("q", q), ("k", k), ("v", v), ("gamma", gamma), ("mu", mu), ("state_in", state_in))
    if grads is not None:
        for n, t in named:
            if "d" + n not in grads:
                raise ValueError(f"grads lacks d{n}")
            _check_tensor("d" + n, grads["d" + n], tuple(t.shape), torch.float32, q.device)
    _check_cuda(q)
    st = _launch_stream(stream)
    with torch.cuda.stream(st):
        if grads is None:
            grads = {"d" + n: torch.empty(t.shape, dtype=torch.float32, device=q.device) for n, t in named}
        need = lattice_osr_bwd_workspace_bytes(desc, chunk_size)
        workspace, wbytes = _workspace(workspace, need, q.device)
        g = grads
        rc = getattr(lib, entry)(ctypes.byref(desc), int(chunk_size), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(gamma), _ptr(mu), _ptr(state_in), _ptr(dy), _ptr(dstate_out),
                                 _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dgamma"]),
                                 _ptr(g["dmu"]), _ptr(g["dstate_in"]), _ptr(workspace), wbytes,
                                 st.cuda_stream)
    if rc != OK:
        raise OSRError(rc, entry)
    return grads


# ------------------------------------------------------------ layer glue --
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
    dev = xq.device
    per_slot = 1 if gamma_logit.dim() == 4 else 0
    gshape = (B, T, H, m) if per_slot else (B, T, H)
    _check_tensor("xq", xq, (B, T, H, m), xq.dtype)
    _check_tensor("xk", xk, (B, T, H, m), xq.dtype, dev)
    _check_tensor("gamma_logit", gamma_logit, gshape, xq.dtype, dev)
    _check_tensor("conv_wq", conv_wq, (H, m, 4), torch.float32, dev)
    _check_tensor("conv_wk", conv_wk, (H, m, 4), torch.float32, dev)
    for name, t in (("conv_bq", conv_bq), ("conv_bk", conv_bk)):
        if t is not None:
            _check_tensor(name, t, (H, m), torch.float32, dev)
    if (hist_q is None) != (hist_k is None):
        raise ValueError("pass both histories or neither")
    for name, t in (("hist_q", hist_q), ("hist_k", hist_k)):
        if t is not None:
            _check_tensor(name, t, (B, 3, H, m), xq.dtype, dev)
    _check_cuda(xq)
    desc = make_desc(B, T, H, m, m, per_slot, _DT[xq.dtype], F32)
    st = _launch_stream(stream)
    with torch.cuda.stream(st):
        outs = {}
        for name, t, like, shape in (("q", q, xq, (B, T, H, m)), ("k", k, xk, (B, T, H, m)),
                                     ("gamma", gamma, gamma_logit, gshape)):
            if t is None:
                t = torch.empty_like(like)
            else:
                _check_tensor(name, t, shape, xq.dtype, dev)
            outs[name] = t
        q, k, gamma = outs["q"], outs["k"], outs["gamma"]
        if return_history:
            hist_q_out = xq.new_empty((B, 3, H, m)) if hist_q_out is None else hist_q_out
            hist_k_out = xk.new_empty((B, 3, H, m)) if hist_k_out is None else hist_k_out
        for name, t in (("hist_q_out", hist_q_out), ("hist_k_out", hist_k_out)):
            if t is not None:
                _check_tensor(name, t, (B, 3, H, m), xq.dtype, dev)
        rc = lib.lattice_osr_glue_pre(ctypes.byref(desc), _ptr(xq), _ptr(xk), _ptr(gamma_logit), _ptr(conv_wq),
                                      _ptr(conv_wk), _ptr(conv_bq), _ptr(conv_bk), _ptr(hist_q), _ptr(hist_k),
                                      _ptr(q), _ptr(k), _ptr(gamma), _ptr(hist_q_out), _ptr(hist_k_out),
                                      st.cuda_stream)
    if rc != OK:
        raise OSRError(rc, "lattice_osr_glue_pre")
    if return_history:
        return q, k, gamma, hist_q_out, hist_k_out
    return q, k, gamma


def lattice_osr_glue_post(y, gate, *, out=None, stream=None):
    """out = y * GeLU(gate) (exact GeLU); y [B,T,H,d] float32 or bfloat16, gate of y's shape in
    float32 or bfloat16.  out may be y (in place)."""
    lib = load_library()
    if y.dim() != 4 or y.dtype not in _DT or gate.dtype not in _DT:
        raise ValueError("y and gate are [B,T,H,d] float32 or bfloat16 tensors of one shape")
    _check_tensor("y", y, tuple(y.shape), y.dtype)
    _check_tensor("gate", gate, tuple(y.shape), gate.dtype, y.device)
    _check_cuda(y)
    B, T, H, d = y.shape
    desc = make_desc(B, T, H, 16, d, 1, _DT[gate.dtype], _DT[y.dtype])
    st = _launch_stream(stream)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty_like(y)
        else:
            _check_tensor("out", out, tuple(y.shape), y.dtype, y.device)
        rc = lib.lattice_osr_glue_post(ctypes.byref(desc), _ptr(y), _ptr(gate), _ptr(out), st.cuda_stream)
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
