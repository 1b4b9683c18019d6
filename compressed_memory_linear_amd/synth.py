"""Seeded synthetic inputs for the OSR forward and decode.

This module holds input generation only (no step of the recurrence): it is the
one piece of code that the GPU path, the tests and the CPU oracle all read
from.  Distributions follow the workloads used to exercise the method:

* initial slots: N(0, I_d) rows scaled to unit norm (random unit vectors);
* q, v ~ N(0, 1); k ~ N(0, 1) then scaled to unit L2 norm over the m slots;
* writing intensity gamma = sigmoid(N(0, 1)) per token and slot (or per token);
* forget gate mu = sigmoid(N(mu_mean, 1)) per token (mu_mean 2, or 3 for the
  long-retention workload).

Draw order is fixed (state, q, k, v, gamma, mu) from numpy's PCG64 with the
given seed, in float32.  bf16 inputs are produced from those float32 draws by
round-to-nearest-even and stored as raw uint16 bit patterns, so the GPU and
the oracle consume exactly the same values.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


@dataclass
class OSRInputs:
    """One batch of inputs in storage form.

    q, k, gamma: [B,T,H,m] (gamma [B,T,H] if not per slot); v: [B,T,H,d];
    mu: [B,T,H]; state: [B,H,m,d] float32 (row = slot).  For bf16 inputs the
    arrays hold uint16 bit patterns; for f32 they hold float32.
    """
    B: int
    T: int
    H: int
    m: int
    d: int
    in_dtype: str
    gamma_per_slot: bool
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    gamma: np.ndarray
    mu: np.ndarray
    state: np.ndarray

    def value(self, name: str) -> np.ndarray:
        """The float32 values an input stands for (exact for bf16)."""
        a = getattr(self, name)
        if name == "state" or self.in_dtype == F32:
            return a.astype(np.float32)
        return bf16_bits_to_f32(a)

    def values_f64(self):
        """(q, k, v, gamma, mu, state) as float64, for the oracle."""
        return tuple(self.value(n).astype(np.float64)
                     for n in ("q", "k", "v", "gamma", "mu", "state"))

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.T


def make_inputs(B: int, T: int, H: int, m: int, d: int, seed: int, in_dtype: str = BF16,
                gamma_per_slot: bool = True, mu_mean: float = 2.0,
                state: Optional[np.ndarray] = None) -> OSRInputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    s0 = rng.standard_normal((B, H, m, d), dtype=np.float32)
    s0 = (s0 / np.linalg.norm(s0.astype(np.float64), axis=-1, keepdims=True)).astype(np.float32)
    if state is not None:
        s0 = np.ascontiguousarray(state, dtype=np.float32)
    q = rng.standard_normal((B, T, H, m), dtype=np.float32)
    k = rng.standard_normal((B, T, H, m), dtype=np.float32)
    k = (k / np.linalg.norm(k.astype(np.float64), axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((B, T, H, d), dtype=np.float32)
    gshape = (B, T, H, m) if gamma_per_slot else (B, T, H)
    gamma = _sigmoid(rng.standard_normal(gshape, dtype=np.float32))
    mu = _sigmoid(rng.standard_normal((B, T, H), dtype=np.float32) + np.float32(mu_mean))
    if in_dtype == BF16:
        q, k, v, gamma, mu = (bf16_round_bits(a) for a in (q, k, v, gamma, mu))
    elif in_dtype != F32:
        raise ValueError(in_dtype)
    return OSRInputs(B, T, H, m, d, in_dtype, gamma_per_slot, q, k, v, gamma, mu, s0)


@dataclass
class GlueInputs:
    """Inputs of the layer glue in storage form (uint16 bf16 bit patterns or float32).

    xq, xk: [B,T,H,m] raw projections before the short convolution; logit:
    [B,T,H,m] or [B,T,H] (the writing intensity's pre-activation); wq, wk:
    [H,m,4] float32 filters (tap 3 = current token); bq, bk: [H,m] float32;
    hist_q, hist_k: [B,3,H,m] raw rows before the sequence; y: [B,T,H,d] the
    recurrence's output (float32, or bf16 when y_dtype is bf16); gate:
    [B,T,H,d] the post-gate branch's projection.
    """
    in_dtype: str
    y_dtype: str
    xq: np.ndarray
    xk: np.ndarray
    logit: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    bq: np.ndarray
    bk: np.ndarray
    hist_q: np.ndarray
    hist_k: np.ndarray
    y: np.ndarray
    gate: np.ndarray

    def value(self, name: str) -> np.ndarray:
        """The float64 values an input stands for (exact for bf16)."""
        a = getattr(self, name)
        bf = (self.y_dtype if name == "y" else self.in_dtype) == BF16
        if name in ("wq", "wk", "bq", "bk") or not bf:
            return a.astype(np.float64)
        return bf16_bits_to_f32(a).astype(np.float64)


def make_glue_inputs(B: int, T: int, H: int, m: int, d: int, seed: int, in_dtype: str = BF16,
                     y_dtype: str = F32, gamma_per_slot: bool = True) -> GlueInputs:
    """Draw order: xq, xk, logit, wq, wk, bq, bk, hist_q, hist_k, y, gate (PCG64, float32).
    Projections and y ~ N(0,1); logits ~ N(0,2^2); filters ~ N(0,1/4) per tap (a
    short filter of unit-scale output); biases ~ N(0, 0.1^2); gate ~ N(0,2^2)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f = np.float32
    xq = rng.standard_normal((B, T, H, m), dtype=f)
    xk = rng.standard_normal((B, T, H, m), dtype=f)
    logit = rng.standard_normal((B, T, H, m) if gamma_per_slot else (B, T, H), dtype=f) * f(2)
    wq = rng.standard_normal((H, m, 4), dtype=f) * f(0.5)
    wk = rng.standard_normal((H, m, 4), dtype=f) * f(0.5)
    bq = rng.standard_normal((H, m), dtype=f) * f(0.1)
    bk = rng.standard_normal((H, m), dtype=f) * f(0.1)
    hist_q = rng.standard_normal((B, 3, H, m), dtype=f)
    hist_k = rng.standard_normal((B, 3, H, m), dtype=f)
    y = rng.standard_normal((B, T, H, d), dtype=f)
    gate = rng.standard_normal((B, T, H, d), dtype=f) * f(2)
    if in_dtype == BF16:
        xq, xk, logit, hist_q, hist_k, gate = (bf16_round_bits(a) for a in (xq, xk, logit, hist_q, hist_k, gate))
    elif in_dtype != F32:
        raise ValueError(in_dtype)
    if y_dtype == BF16:
        y = bf16_round_bits(y)
    elif y_dtype != F32:
        raise ValueError(y_dtype)
    return GlueInputs(in_dtype, y_dtype, xq, xk, logit, wq, wk, bq, bk, hist_q, hist_k, y, gate)


# The workloads, named by what they are.  chunk=None means "several chunk sizes".
WORKLOADS = {
    "tiny_f32_m16d32_t64": dict(B=1, H=1, T=64, m=16, d=32, in_dtype=F32, chunk=None,
                                mu_mean=2.0, seed=1000),
    "chunked_b4h8_t2048_m64d64_c64": dict(B=4, H=8, T=2048, m=64, d=64, in_dtype=BF16, chunk=64,
                                          mu_mean=2.0, seed=1001),
    "chunked_b8h16_t4096_m64d128_c64": dict(B=8, H=16, T=4096, m=64, d=128, in_dtype=BF16,
                                            chunk=64, mu_mean=2.0, seed=1002),
    "decode_s256h32_m128d128": dict(B=256, H=32, T=1, m=128, d=128, in_dtype=BF16, chunk=1,
                                    mu_mean=2.0, seed=1003),
    "chunked_b1h16_t65536_m128d128_c128": dict(B=1, H=16, T=65536, m=128, d=128, in_dtype=BF16,
                                               chunk=128, mu_mean=3.0, seed=1004),
}


def workload_inputs(name: str, T: Optional[int] = None, B: Optional[int] = None,
                    H: Optional[int] = None) -> OSRInputs:
    w = WORKLOADS[name]
    return make_inputs(B or w["B"], T or w["T"], H or w["H"], w["m"], w["d"], seed=w["seed"],
                       in_dtype=w["in_dtype"], gamma_per_slot=True, mu_mean=w["mu_mean"])
