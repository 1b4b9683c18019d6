"""fp64 CPU oracle for the gradient of the OSR forward (training backward).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It
shares no code with the HIP library.

What it computes.  The backward of a layer is the vector-Jacobian product of
its forward: given upstream gradients dy (of the read-outs y) and dS_T (of
the returned state), the gradients of sum(dy * y) + sum(dS_T * S_T) with
respect to every input q, k, v, gamma, mu and the initial state S_0.  The
pages train the layer by differentiating the chunk-wise form ("Lattice:
Learning to Efficiently Compress the Memory", arXiv 2504.05646, section
"Parallel and Hardware Efficient Form"; the experiments' default chunk size
is 4), so the function differentiated here is the chunk-linearised forward
at the same chunk size C (exact at C = 1).

The forward is written out below in the pages' notation, batched over
(batch, head) with plain torch float64 CPU operations, and differentiated by
torch autograd (the library primitive that evaluates a vector-Jacobian
product).  Per chunk, with S the state at the chunk start:

  Z        = rows of S projected onto the unit sphere      (eq. normalized_recurrence)
  h_t      = phi(Z) k_t - v_t | -v_t | v_t                  (decoding / similarity /
                                                             encoding layer, eq. OSR)
  h~_{t,i} = z_i . h_t
  c_{t,i}  = k_{t,i}, or h~_{t,i} - k_{t,i} for the encoding layer
  |ds_i|^2 = (gamma_i c_i)^2 (|h_t|^2 - h~_{t,i}^2), kept only where positive
                                                            (appendix "Computing beta")
  beta_i   = (mu_t^2 + |ds_i|^2)^(-1/2)
  k^_i     = gamma_i beta_i c_i
  s_i      <- (mu_t beta_i + h~_i k^_i) s_i - k^_i h_t       (eq. recurrence_linear2)
           or mu_t beta_i s_i + h~_i k^_i z_i - k^_i h_t      (eq. recurrence_linear1)
  y_t      = sum_i q_{t,i} s_i
and the returned state is the final S with its rows projected once more.
The same readings as the C oracle (osr_oracle.c) apply: mu^2 in beta, the
minus sign under the clamp, no epsilon, no factor 2.

The gradient is chained backwards over segments of whole chunks: the forward
stores each segment's starting state (no graph), then each segment is run
again with its starting state as a leaf and differentiated given the
gradient arriving at its end.  Chunks only interact through the state, so
this is the chain rule and nothing else; it bounds autograd's memory to one
segment.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

MODE_DEC, MODE_SIM, MODE_ENC = 0, 1, 2
LIN2, LIN1 = 0, 1

_DT = torch.float64


def _project(S: torch.Tensor) -> torch.Tensor:
    """Rows (slots) of S onto the unit sphere."""
    return S / torch.sqrt((S * S).sum(dim=-1, keepdim=True))


def _chunk_forward(S, q, k, v, gamma, mu, mode, lin):
    """One chunk.  S [B,H,m,d] (state at the chunk start, before projection);
    q, k [B,C,H,m]; v [B,C,H,d]; gamma [B,C,H,m] or [B,C,H]; mu [B,C,H].
    Returns (state at the chunk end [B,H,m,d], y [B,C,H,d])."""
    Z = _project(S)
    R = Z
    ys = []
    C = q.shape[1]
    per_slot = gamma.dim() == 4
    for t in range(C):
        kt = k[:, t]                                  # [B,H,m]
        vt = v[:, t]                                  # [B,H,d]
        mut = mu[:, t][..., None]                     # [B,H,1]
        gt = gamma[:, t] if per_slot else gamma[:, t][..., None]
        if mode == MODE_DEC:
            h = (kt[..., None] * Z).sum(dim=-2) - vt  # sum_i k_i z_i - v
        elif mode == MODE_SIM:
            h = -vt
        else:
            h = vt
        htil = (Z * h[..., None, :]).sum(dim=-1)      # [B,H,m]
        hsq = (h * h).sum(dim=-1, keepdim=True)       # [B,H,1]
        coeff = htil - kt if mode == MODE_ENC else kt
        wint = gt * coeff
        dsq = wint * wint * (hsq - htil * htil)
        dsq = torch.where(dsq > 0, dsq, torch.zeros_like(dsq))
        beta = 1.0 / torch.sqrt(mut * mut + dsq)
        khat = gt * beta * coeff
        if lin == LIN1:
            R = (mut * beta)[..., None] * R + (htil * khat)[..., None] * Z - khat[..., None] * h[..., None, :]
        else:
            R = (mut * beta + htil * khat)[..., None] * R - khat[..., None] * h[..., None, :]
        ys.append((q[:, t][..., None] * R).sum(dim=-2))
    return R, torch.stack(ys, dim=1)


def _segment_forward(S, q, k, v, gamma, mu, C, mode, lin):
    ys = []
    for t0 in range(0, q.shape[1], C):
        sl = slice(t0, t0 + C)
        S, y = _chunk_forward(S, q[:, sl], k[:, sl], v[:, sl], gamma[:, sl], mu[:, sl], mode, lin)
        ys.append(y)
    return S, torch.cat(ys, dim=1)


def _t(a) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(np.asarray(a, dtype=np.float64)))


def osr_forward_torch(q, k, v, gamma, mu, state, chunk_size: int = 1, mode: int = MODE_DEC,
                      linearisation: int = LIN2):
    """The forward above, without gradients: (y [B,T,H,d], state_out [B,H,m,d])."""
    q, k, v, gamma, mu, S = (_t(a) for a in (q, k, v, gamma, mu, state))
    if q.shape[1] % chunk_size:
        raise ValueError("T % chunk_size != 0")
    with torch.no_grad():
        S, y = _segment_forward(S, q, k, v, gamma, mu, chunk_size, mode, linearisation)
        return y.numpy(), _project(S).numpy()


def osr_backward(q, k, v, gamma, mu, state, dy, dstate_out, chunk_size: int = 1,
                 mode: int = MODE_DEC, linearisation: int = LIN2,
                 segment: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Gradients of sum(dy*y) + sum(dstate_out*state_out) of the chunk-wise
    forward.  Shapes as in the forward; dy [B,T,H,d], dstate_out [B,H,m,d].
    Returns float64 arrays dq, dk, dv, dgamma, dmu, dstate_in in the inputs'
    shapes.  segment: tokens per differentiated segment (a multiple of the
    chunk size; default the smallest multiple >= 64)."""
    q, k, v, gamma, mu, S0, dy, dSo = (_t(a) for a in (q, k, v, gamma, mu, state, dy, dstate_out))
    T, C = q.shape[1], int(chunk_size)
    if T % C:
        raise ValueError("T % chunk_size != 0")
    L = segment if segment is not None else C * max(1, -(-64 // C))
    if L % C:
        raise ValueError("segment must be a multiple of chunk_size")
    starts = list(range(0, T, L))

    # Forward: the state entering every segment (no graph kept).
    seg_states = []
    with torch.no_grad():
        S = S0
        for t0 in starts:
            seg_states.append(S)
            sl = slice(t0, min(t0 + L, T))
            S, _ = _segment_forward(S, q[:, sl], k[:, sl], v[:, sl], gamma[:, sl], mu[:, sl], C, mode,
                                    linearisation)
        S_end = S

    # The returned state is the projected end state.
    Se = S_end.clone().requires_grad_(True)
    (dS,) = torch.autograd.grad(_project(Se), Se, grad_outputs=dSo)

    grads = {n: torch.zeros_like(a) for n, a in (("q", q), ("k", k), ("v", v), ("gamma", gamma),
                                                  ("mu", mu))}
    for t0, S_start in zip(reversed(starts), reversed(seg_states)):
        sl = slice(t0, min(t0 + L, T))
        leaves = [S_start.clone().requires_grad_(True)] + \
                 [a[:, sl].clone().requires_grad_(True) for a in (q, k, v, gamma, mu)]
        with torch.enable_grad():
            S_out, y = _segment_forward(*leaves, C, mode, linearisation)
            g = torch.autograd.grad((S_out, y), leaves, grad_outputs=(dS, dy[:, sl]), allow_unused=True)
        dS = g[0]
        for name, gi, leaf in zip(("q", "k", "v", "gamma", "mu"), g[1:], leaves[1:]):
            grads[name][:, sl] = gi if gi is not None else torch.zeros_like(leaf)
    out = {"d" + n: a.numpy() for n, a in grads.items()}
    out["dstate_in"] = dS.numpy()
    return out
