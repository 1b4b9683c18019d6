"""GPU parity on the method's degenerate cases and on bf16 outputs.

Every case goes through the C ABI and is compared with the fp64 oracle at the
stated bars (max-abs error over the oracle's RMS: 1e-4 for fp32 inputs, 2e-2
for bf16 inputs), on each kernel family: the split matrix-core schedule
(state passing + read-out), the fused matrix-core kernel, the fp32 token loop,
the exact recurrent forward and the decode step.  The inputs are the synthetic
draws of compressed_memory_linear_amd.synth with one property forced:

* gamma = 0, or k = 0: nothing is written (the writing intensity gamma k is
  zero; Lattice paper, section 3.1, k as the writing intensity), so the state
  stays at its projected start and y_t = sum_i q_{t,i} z_i;
* h parallel to a slot: the orthogonal part of h is zero for that slot, so
  |h|^2 - c^2 is zero up to rounding and the clamp at 0 of the appendix
  "Computing beta" is what keeps beta finite;
* mu near 0, mu = 1 (no decay) and mu near 1 (eq. dacay_recurrence);
* initial slots whose norms span six decades (every slot is projected onto
  the unit sphere first: eq. normalized_recurrence).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from compressed_memory_linear_amd import osr, synth

pytestmark = pytest.mark.gpu

TOL = {synth.F32: 1e-4, synth.BF16: 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    osr.load_library()
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _rel(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref)) / np.sqrt(np.mean(ref ** 2)))


# (name, in_dtype, entry, chunk size, schedule, T)
PATHS = [("split", synth.BF16, "chunked", 64, osr.SCHED_SPLIT, 256),
         ("fused", synth.BF16, "chunked", 32, osr.SCHED_FUSED, 256),
         ("tokenloop", synth.F32, "chunked", 4, osr.SCHED_AUTO, 128),
         ("recurrent", synth.F32, "recurrent", 1, osr.SCHED_AUTO, 64),
         ("decode", synth.BF16, "decode", 1, osr.SCHED_AUTO, 1)]


def _set(inp, name, f32):
    """Replace one input by the float32 array f32 (rounded to bf16 for bf16 inputs)."""
    f32 = np.ascontiguousarray(f32, dtype=np.float32)
    setattr(inp, name, synth.bf16_round_bits(f32) if inp.in_dtype == synth.BF16 else f32)


def _make(path, seed, m=64, d=64, per_slot=True):
    _, dt, entry, C, sched, T = path
    B, H = (8, 8) if entry == "decode" else (2, 2)
    return synth.make_inputs(B, T, H, m, d, seed=seed, in_dtype=dt, gamma_per_slot=per_slot)


def _run(path, inp, mode=osr.MODE_DEC, y_dtype=torch.float32):
    _, dt, entry, C, sched, T = path
    t = osr.to_device(inp)
    args = (t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"])
    if entry == "chunked":
        y, S = osr.lattice_osr_fwd_chunked(*args, C, mode=mode, y_dtype=y_dtype, schedule=sched)
    elif entry == "recurrent":
        y, S = osr.lattice_osr_fwd_recurrent(*args, mode=mode, y_dtype=y_dtype)
    else:
        y, S = osr.lattice_osr_decode_step(*args, mode=mode, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), S.cpu().numpy()


def _compare(path, inp, mode=osr.MODE_DEC, y_dtype=torch.float32):
    C = path[3]
    y, S = _run(path, inp, mode, y_dtype)
    yr, Sr = oracle.osr_forward(*inp.values_f64(), chunk_size=C, mode=mode)
    ey, es = _rel(y, yr), _rel(S, Sr)
    tol = TOL[inp.in_dtype]
    _say(f"  y err/rms = {ey:.3e}, state err/rms = {es:.3e} (tol {tol:g})")
    assert np.isfinite(y).all() and np.isfinite(S).all()
    assert ey <= tol and es <= tol, (ey, es)
    return y, S, yr, Sr


def _projected_start(inp):
    s = inp.state.astype(np.float64)
    return s / np.linalg.norm(s, axis=-1, keepdims=True)


@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM, osr.MODE_ENC])
def test_zero_writing_intensity(path, mode):
    """gamma = 0: no write for any objective; the state stays at the
    projected start and y_t = sum_i q_{t,i} z_i."""
    _say(f"gamma = 0, path {path[0]}, mode {mode}")
    inp = _make(path, 2001 + mode)
    inp.state = (inp.state * np.random.default_rng(1).uniform(0.5, 2.0, inp.state.shape[:-1] + (1,))
                 ).astype(np.float32)
    _set(inp, "gamma", np.zeros(inp.gamma.shape, np.float32))
    y, S, yr, Sr = _compare(path, inp, mode)
    Z = _projected_start(inp)
    q = inp.values_f64()[0]
    np.testing.assert_allclose(Sr, Z, atol=1e-12)  # the oracle's closed form, as a check of the case
    np.testing.assert_allclose(yr, np.einsum("bthi,bhid->bthd", q, Z), atol=1e-10)
    assert np.max(np.abs(S - Z)) <= 1e-5


@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM])
def test_zero_key(path, mode):
    """k = 0: the writing intensity gamma k is zero (decoding and similarity
    objectives), so nothing is written."""
    _say(f"k = 0, path {path[0]}, mode {mode}")
    inp = _make(path, 2011 + mode)
    _set(inp, "k", np.zeros(inp.k.shape, np.float32))
    y, S, yr, Sr = _compare(path, inp, mode)
    assert np.max(np.abs(S - _projected_start(inp))) <= 1e-5


@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM])
def test_h_parallel_to_a_slot(path, mode):
    """h parallel to slot 0 at every token: slot 0 starts at e_0 and every v_t
    is a multiple of e_0.  Similarity objective: h = -v.  Decoding objective:
    k_t = 0.25 e_0, so h = 0.25 z_0 - v_t and only slot 0 is written.  For
    slot 0, |h|^2 - c^2 = 0 up to rounding: the clamp at 0 is active and slot
    0 must stay e_0.  (There g = 1 + a c / mu and kappa = -a / mu: the write
    cancels the gain exactly.  The chunk-parallel form sums such terms in
    closed form, which loses accuracy once the gates' running product spans
    many decades over a sub-block; v_0 in [0, 2] keeps |g - 1| below ~0.3.)"""
    _say(f"h parallel to slot 0, path {path[0]}, mode {mode}")
    inp = _make(path, 2021 + mode)
    S0 = inp.state.copy()
    S0[:, :, 0, :] = 0.0
    S0[:, :, 0, 0] = 1.0
    inp.state = S0
    rng = np.random.default_rng(7)
    v = np.zeros(inp.v.shape, np.float32)
    v[..., 0] = rng.uniform(0.0, 2.0, v.shape[:-1])
    _set(inp, "v", v)
    if mode == osr.MODE_DEC:
        k = np.zeros(inp.k.shape, np.float32)
        k[..., 0] = 0.25
        _set(inp, "k", k)
    y, S, yr, Sr = _compare(path, inp, mode)
    e0 = np.zeros(inp.d)
    e0[0] = 1.0
    np.testing.assert_allclose(Sr[:, :, 0], np.broadcast_to(e0, Sr[:, :, 0].shape), atol=1e-12)
    assert np.max(np.abs(S[:, :, 0] - e0)) <= 1e-5


@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
@pytest.mark.parametrize("which", ["near0", "one", "near1"])
def test_forget_gate_extremes(path, which):
    """mu in [1e-3, 1e-2] (the old state is nearly forgotten each token), mu =
    1 (no decay) and mu in [0.99, 1) (exact in fp32; bf16 rounds it to 0.9961
    or 1)."""
    _say(f"mu {which}, path {path[0]}")
    inp = _make(path, 2031)
    rng = np.random.default_rng(11)
    shape = inp.mu.shape
    mu = {"near0": rng.uniform(1e-3, 1e-2, shape), "one": np.ones(shape),
          "near1": rng.uniform(0.99, 1.0, shape)}[which]
    _set(inp, "mu", mu.astype(np.float32))
    for mode in (osr.MODE_DEC, osr.MODE_SIM):
        _compare(path, inp, mode)


@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
def test_unequal_initial_slot_norms(path):
    """Initial slots with norms 10^U(-3, 3): the chunk-start projection makes
    them unit before any product."""
    _say(f"initial slot norms over six decades, path {path[0]}")
    inp = _make(path, 2041)
    scale = 10.0 ** np.random.default_rng(3).uniform(-3, 3, inp.state.shape[:-1] + (1,))
    inp.state = (inp.state * scale).astype(np.float32)
    # the encoding layer amplifies rounding-size perturbations (its parity
    # over long sequences is covered elsewhere at short lengths); here the
    # projection of the start state is what is exercised
    modes = (osr.MODE_DEC, osr.MODE_SIM) + ((osr.MODE_ENC,) if inp.in_dtype == synth.BF16 else ())
    for mode in modes:
        _compare(path, inp, mode)


# The encoding layer only with bf16 inputs: its fp32 parity at this length is
# beyond fp32 (it amplifies rounding; covered at short lengths elsewhere).
BF16_OUT_CASES = [(p, mode) for p in PATHS for mode in (osr.MODE_DEC, osr.MODE_SIM, osr.MODE_ENC)
                  if mode != osr.MODE_ENC or p[1] == synth.BF16]


@pytest.mark.parametrize("path,mode", BF16_OUT_CASES, ids=[f"{p[0]}-{m}" for p, m in BF16_OUT_CASES])
def test_bf16_output(path, mode):
    """y stored as bf16 by every kernel family: bit for bit the round-to-
    nearest-even of the same kernel's fp32 y (the store is the only
    difference), the fp32 y within the stated bar of the oracle, and the
    state unchanged."""
    _say(f"bf16 y, path {path[0]}, mode {mode}")
    inp = _make(path, 2051 + mode)
    C = path[3]
    y16, S16 = _run(path, inp, mode, torch.bfloat16)
    y32, S32 = _run(path, inp, mode, torch.float32)
    yr, Sr = oracle.osr_forward(*inp.values_f64(), chunk_size=C, mode=mode)
    rounded = synth.bf16_bits_to_f32(synth.bf16_round_bits(y32))
    mism = int(np.sum(rounded.view(np.uint32) != y16.astype(np.float32).view(np.uint32)))
    ey = _rel(y32, yr)
    _say(f"  bf16 y vs RNE(fp32 y): {mism} mismatches; fp32 y err/rms = {ey:.3e}")
    assert mism == 0
    assert np.array_equal(S16, S32)
    assert ey <= TOL[inp.in_dtype]


def test_bf16_output_first_linearisation():
    """bf16 y from the split schedule's first-linearisation read-out: the
    rounding of its fp32 y, which meets the bar."""
    _say("bf16 y, first linearisation, split schedule m64 d64 C64")
    inp = synth.make_inputs(2, 256, 2, 64, 64, seed=2061, in_dtype=synth.BF16)
    t = osr.to_device(inp)
    ys = {}
    for dt in (torch.bfloat16, torch.float32):
        y, S = osr.lattice_osr_fwd_chunked(t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"], 64,
                                           y_dtype=dt, linearisation=osr.LIN1)
        torch.cuda.synchronize()
        ys[dt] = y.float().cpu().numpy()
    yr, Sr = oracle.osr_forward(*inp.values_f64(), chunk_size=64, mode=osr.MODE_DEC, linearisation=oracle.LIN1)
    rounded = synth.bf16_bits_to_f32(synth.bf16_round_bits(ys[torch.float32]))
    assert np.array_equal(rounded, ys[torch.bfloat16])
    ey, es = _rel(ys[torch.float32], yr), _rel(S.cpu().numpy(), Sr)
    _say(f"  fp32 y err/rms = {ey:.3e}, state err/rms = {es:.3e}")
    assert ey <= 2e-2 and es <= 2e-2
