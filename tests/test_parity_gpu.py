"""GPU parity: every entry point of liblattice_osr.so against the fp64 oracle.

Inputs are seeded and synthetic (compressed_memory_linear_amd.synth); the
oracle consumes exactly the values the GPU reads (bf16 inputs are decoded
bit-exactly).  The bar is the one stated for this path: the maximum absolute
error, divided by the RMS of the oracle's output, is at most 1e-4 for fp32
inputs and 2e-2 for bf16 inputs (fp32 state); the returned state is held to
the same bar relative to its own RMS.

Small shapes are compared in full.  At the full workload sizes the oracle
recomputes a sample of whole (batch, head) sequences, each from its own state
(sequences are independent), and those are compared element by element.
"""
import concurrent.futures as cf
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
    got = np.asarray(got, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(got - ref)) / rms)


def _oracle(inp, C, mode, bh=None):
    """Oracle outputs for all (b,h), or only for the listed (b,h) pairs."""
    q, k, v, g, mu, S = inp.values_f64()
    if bh is None:
        return oracle.osr_forward(q, k, v, g, mu, S, chunk_size=C, mode=mode)

    def one(pair):
        b, h = pair
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        return oracle.osr_forward(q[sl], k[sl], v[sl], g[sl], mu[b:b + 1, :, h:h + 1],
                                  S[b:b + 1, h:h + 1], chunk_size=C, mode=mode, nthreads=1)

    with cf.ThreadPoolExecutor(min(len(bh), 16)) as ex:
        return list(ex.map(one, bh))


def _check(inp, y, S, C, mode, bh=None, y_tol=None):
    tol = y_tol or TOL[inp.in_dtype]
    y = y.float().cpu().numpy()
    S = S.cpu().numpy()
    if bh is None:
        yr, Sr = _oracle(inp, C, mode)
        ey, es = _rel(y, yr), _rel(S, Sr)
    else:
        outs = _oracle(inp, C, mode, bh)
        ey = max(_rel(y[b, :, h], o[0][0, :, 0]) for (b, h), o in zip(bh, outs))
        es = max(_rel(S[b, h], o[1][0, 0]) for (b, h), o in zip(bh, outs))
    _say(f"  y err/rms = {ey:.3e}, state err/rms = {es:.3e} (tol {tol:g})")
    assert np.isfinite(y).all() and np.isfinite(S).all()
    assert ey <= tol, ey
    assert es <= tol, es
    return ey, es


def _run(entry, inp, C=None, mode=osr.MODE_DEC, y_dtype=torch.float32, **kw):
    t = osr.to_device(inp)
    args = (t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"])
    if entry == "chunked":
        y, S = osr.lattice_osr_fwd_chunked(*args, C, mode=mode, y_dtype=y_dtype, **kw)
    elif entry == "recurrent":
        y, S = osr.lattice_osr_fwd_recurrent(*args, mode=mode, y_dtype=y_dtype, **kw)
    else:
        y, S = osr.lattice_osr_decode_step(*args, mode=mode, y_dtype=y_dtype, **kw)
    torch.cuda.synchronize()
    return y, S


# ---------------------------------------------------------------- tiny fp32 --
TINY = synth.WORKLOADS["tiny_f32_m16d32_t64"]


def _tiny(per_slot=True, seed=None):
    w = TINY
    return synth.make_inputs(w["B"], w["T"], w["H"], w["m"], w["d"], seed=seed or w["seed"],
                             in_dtype=synth.F32, gamma_per_slot=per_slot, mu_mean=w["mu_mean"])


@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM, osr.MODE_ENC])
@pytest.mark.parametrize("per_slot", [True, False])
def test_tiny_recurrent(mode, per_slot):
    _say(f"tiny recurrent mode={mode} per_slot={per_slot}")
    inp = _tiny(per_slot)
    y, S = _run("recurrent", inp, mode=mode)
    _check(inp, y, S, 1, mode)


@pytest.mark.parametrize("C", [1, 4, 16, 64])
@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM, osr.MODE_ENC])
def test_tiny_chunked(C, mode):
    _say(f"tiny chunked C={C} mode={mode}")
    inp = _tiny()
    y, S = _run("chunked", inp, C, mode=mode)
    _check(inp, y, S, C, mode)


def test_tiny_decode_repeated_equals_recurrent():
    _say("tiny decode x T (in place)")
    inp = _tiny()
    t = osr.to_device(inp)
    state = t["state"].clone()
    ys = []
    for i in range(inp.T):
        sl = slice(i, i + 1)
        y, state = osr.lattice_osr_decode_step(t["q"][:, sl].contiguous(), t["k"][:, sl].contiguous(),
                                               t["v"][:, sl].contiguous(), t["gamma"][:, sl].contiguous(),
                                               t["mu"][:, sl].contiguous(), state, state_out=state)
        ys.append(y)
    torch.cuda.synchronize()
    _check(inp, torch.cat(ys, dim=1), state, 1, osr.MODE_DEC)


def test_tiny_bf16_output():
    _say("tiny recurrent with bf16 y")
    inp = _tiny()
    y32, _ = _run("recurrent", inp)
    y16, _ = _run("recurrent", inp, y_dtype=torch.bfloat16)
    assert y16.dtype == torch.bfloat16
    # bf16 output is the fp32 output rounded to nearest: relative error <= 2^-9
    diff = (y16.float() - y32).abs()
    assert torch.all(diff <= y32.abs() * 2.0 ** -8 + 1e-30)


# --------------------------------------------------------- bf16 shape sweep --
SHAPES = [(16, 16), (16, 128), (32, 32), (64, 64), (64, 128), (128, 64), (128, 128)]


@pytest.mark.parametrize("m,d", SHAPES)
@pytest.mark.parametrize("C", [1, 16, 64])
def test_bf16_shape_sweep(m, d, C):
    _say(f"bf16 sweep m={m} d={d} C={C}")
    inp = synth.make_inputs(2, 256, 2, m, d, seed=7 + m + d + C, in_dtype=synth.BF16)
    y, S = _run("chunked", inp, C)
    _check(inp, y, S, C, osr.MODE_DEC)


@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM, osr.MODE_ENC])
@pytest.mark.parametrize("per_slot", [True, False])
def test_bf16_modes_and_gamma_layouts(mode, per_slot):
    _say(f"bf16 mode={mode} per_slot={per_slot} C=32")
    inp = synth.make_inputs(2, 256, 3, 64, 64, seed=31, in_dtype=synth.BF16, gamma_per_slot=per_slot)
    y, S = _run("chunked", inp, 32, mode=mode)
    _check(inp, y, S, 32, mode)


# ---------------------------------------------- first chunk linearisation --
# eq. recurrence_linear1 (desc linearisation = LIN1): the token loop for fp32 inputs
# or C < 16, the split matrix-core schedule for bf16 inputs with C >= 16.
def _oracle_lin1(inp, C, mode):
    q, k, v, g, mu, S = inp.values_f64()
    return oracle.osr_forward(q, k, v, g, mu, S, chunk_size=C, mode=mode, linearisation=oracle.LIN1)


def _check_lin1(inp, y, S, C, mode):
    tol = TOL[inp.in_dtype]
    yr, Sr = _oracle_lin1(inp, C, mode)
    ey, es = _rel(y.float().cpu().numpy(), yr), _rel(S.cpu().numpy(), Sr)
    _say(f"  y err/rms = {ey:.3e}, state err/rms = {es:.3e} (tol {tol:g})")
    assert ey <= tol and es <= tol, (ey, es)


# The encoding layer with the first linearisation amplifies perturbations
# fast: in the fp64 oracle a 2^-17 relative change of every input (the
# precision of the split-bf16 operands) moves y or the state by O(1) of their
# RMS within 128 - 256 tokens at m = 16 (C = 4) and m = d = 128 (C = 16), where
# the decoding and similarity objectives damp it.  Element-wise parity at the
# fixed bar is therefore checked over lengths where that change stays below
# 7e-3 (measured: m16 d32 C4 T32 <= 6.3e-3; m64 d64 C64 T128 <= 1.6e-3;
# m128 d128 C16 T32 <= 6.6e-3; m32 d128 C128 T256 <= 3.2e-3).
ENC_LIN1_T = {4: 32, 16: 32, 64: 128, 128: 256}


@pytest.mark.parametrize("C", [1, 4, 16, 64])
@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM, osr.MODE_ENC])
def test_tiny_chunked_lin1(C, mode):
    _say(f"tiny chunked, first linearisation, C={C} mode={mode}")
    inp = _tiny()
    t = osr.to_device(inp)
    y, S = osr.lattice_osr_fwd_chunked(t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"], C,
                                       mode=mode, linearisation=osr.LIN1)
    torch.cuda.synchronize()
    _check_lin1(inp, y, S, C, mode)


@pytest.mark.parametrize("m,d,C", [(16, 32, 4), (64, 64, 64), (128, 128, 16), (32, 128, 128)])
@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM, osr.MODE_ENC])
@pytest.mark.parametrize("per_slot", [True, False])
def test_bf16_chunked_lin1(m, d, C, mode, per_slot):
    T = ENC_LIN1_T[C] if mode == osr.MODE_ENC else 256
    _say(f"bf16 chunked, first linearisation, m={m} d={d} C={C} T={T} mode={mode} per_slot={per_slot}")
    inp = synth.make_inputs(2, T, 3, m, d, seed=800 + m + d + C, in_dtype=synth.BF16, gamma_per_slot=per_slot)
    t = osr.to_device(inp)
    y, S = osr.lattice_osr_fwd_chunked(t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"], C,
                                       mode=mode, linearisation=osr.LIN1)
    torch.cuda.synchronize()
    _check_lin1(inp, y, S, C, mode)


def test_workload_chunked_b4h8_t2048_m64d64_c64_lin1():
    _say("chunked workload B4 H8 T2048 m64 d64 C64, first linearisation (full compare)")
    inp = synth.workload_inputs("chunked_b4h8_t2048_m64d64_c64")
    t = osr.to_device(inp)
    y, S = osr.lattice_osr_fwd_chunked(t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"], 64,
                                       linearisation=osr.LIN1)
    torch.cuda.synchronize()
    _check_lin1(inp, y, S, 64, osr.MODE_DEC)


# ------------------------------------------------------------ decode sweep --
# 37 x 64 = 2368 states, one workgroup each: more workgroups than the device
# holds at once for every shape, and not a multiple of its compute units, so
# the grid runs in several rounds with a ragged last one.
DECODE_SHAPES = [(16, 16), (32, 64), (64, 128), (128, 128)]


@pytest.mark.parametrize("m,d", DECODE_SHAPES)
@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM, osr.MODE_ENC])
@pytest.mark.parametrize("per_slot", [True, False])
def test_decode_sweep_bf16(m, d, mode, per_slot):
    _say(f"decode sweep bf16 m={m} d={d} mode={mode} per_slot={per_slot} (2368 states)")
    inp = synth.make_inputs(37, 1, 64, m, d, seed=400 + m + d, in_dtype=synth.BF16, gamma_per_slot=per_slot)
    y, S = _run("decode", inp, mode=mode)
    _check(inp, y, S, 1, mode)


@pytest.mark.parametrize("m,d", [(16, 32), (128, 128)])
def test_decode_sweep_f32(m, d):
    _say(f"decode sweep fp32 m={m} d={d} (2368 states)")
    inp = synth.make_inputs(37, 1, 64, m, d, seed=500 + m + d, in_dtype=synth.F32)
    y, S = _run("decode", inp)
    _check(inp, y, S, 1, osr.MODE_DEC)


# ------------------------------------------------------- workload-size runs --
def test_workload_decode_s256h32_m128d128():
    _say("decode workload 256 seq x 32 heads, m=d=128")
    inp = synth.workload_inputs("decode_s256h32_m128d128")
    y, S = _run("decode", inp)
    _check(inp, y, S, 1, osr.MODE_DEC)


def test_workload_chunked_b4h8_t2048_m64d64_c64():
    _say("chunked workload B4 H8 T2048 m64 d64 C64 (full compare)")
    inp = synth.workload_inputs("chunked_b4h8_t2048_m64d64_c64")
    y, S = _run("chunked", inp, 64)
    _check(inp, y, S, 64, osr.MODE_DEC)


# The encoding layer feeds the state back into its own writing intensity
# (gamma (phi(S)^T v - k)), and on these inputs it amplifies perturbations:
# in the fp64 oracle a 1e-7 relative change of the initial state grows to
# ~1e-3 of the output RMS within ~800 tokens, where the decoding and
# similarity recurrences damp it to 1e-15 (pinned on the CPU in
# test_oracle_pins).  Rounding at fp32 (and 2^-16 for the split products)
# therefore cannot stay within 2e-2 element by element over 2048 tokens, so
# element-wise parity is checked over the workload's first 256 tokens (every
# (b,h), growth below ~30x there), and the full length through what holds at
# any length: finite outputs and unit slots in the returned state.
def test_workload_chunked_b4h8_m64d64_c64_encoding_first_256_tokens():
    _say("chunked workload shape B4 H8 m64 d64 C64, encoding layer, first 256 tokens")
    w = synth.WORKLOADS["chunked_b4h8_t2048_m64d64_c64"]
    inp = synth.make_inputs(w["B"], 256, w["H"], w["m"], w["d"], seed=w["seed"], in_dtype=synth.BF16)
    y, S = _run("chunked", inp, 64, mode=osr.MODE_ENC)
    _check(inp, y, S, 64, osr.MODE_ENC)


def test_workload_chunked_b4h8_t2048_m64d64_c64_encoding_invariants():
    _say("chunked workload B4 H8 T2048 m64 d64 C64, encoding layer: finite, unit slots")
    inp = synth.workload_inputs("chunked_b4h8_t2048_m64d64_c64")
    y, S = _run("chunked", inp, 64, mode=osr.MODE_ENC)
    assert torch.isfinite(y).all() and torch.isfinite(S).all()
    assert (S.norm(dim=-1) - 1.0).abs().max().item() <= 1e-5


def test_workload_chunked_b8h16_t4096_m64d128_c64():
    _say("chunked workload B8 H16 T4096 m64 d128 C64 (sampled sequences)")
    inp = synth.workload_inputs("chunked_b8h16_t4096_m64d128_c64")
    y, S = _run("chunked", inp, 64)
    _check(inp, y, S, 64, osr.MODE_DEC, bh=[(0, 0), (3, 7), (7, 15), (5, 2)])


def test_workload_chunked_b1h16_t65536_m128d128_c128():
    _say("chunked workload B1 H16 T65536 m=d=128 C128 (sampled sequences)")
    inp = synth.workload_inputs("chunked_b1h16_t65536_m128d128_c128")
    y, S = _run("chunked", inp, 128)
    _check(inp, y, S, 128, osr.MODE_DEC, bh=[(0, 0), (0, 11)])


# ------------------------------------------------------------ composition --
@pytest.mark.parametrize("C", [1, 16])
def test_resume_at_chunk_boundary(C):
    _say(f"resume at chunk boundary C={C}")
    inp = synth.make_inputs(2, 128, 2, 32, 64, seed=5, in_dtype=synth.BF16)
    t = osr.to_device(inp)
    names = ("q", "k", "v", "gamma", "mu")
    y, S = osr.lattice_osr_fwd_chunked(*(t[n] for n in names), t["state"], C)
    T1 = 64
    y1, S1 = osr.lattice_osr_fwd_chunked(*(t[n][:, :T1].contiguous() for n in names), t["state"], C)
    y2, S2 = osr.lattice_osr_fwd_chunked(*(t[n][:, T1:].contiguous() for n in names), S1, C)
    torch.cuda.synchronize()
    assert (torch.cat([y1, y2], dim=1) - y).abs().max().item() <= 1e-5 * y.abs().max().item()
    assert (S2 - S).abs().max().item() <= 1e-5


def test_prefill_then_decode_equals_recurrent():
    _say("prefill (C=1) then decode == recurrent")
    inp = synth.make_inputs(3, 40, 2, 64, 32, seed=9, in_dtype=synth.BF16)
    t = osr.to_device(inp)
    names = ("q", "k", "v", "gamma", "mu")
    y, S = osr.lattice_osr_fwd_recurrent(*(t[n] for n in names), t["state"])
    yp, Sp = osr.lattice_osr_fwd_chunked(*(t[n][:, :39].contiguous() for n in names), t["state"], 1)
    yd, Sd = osr.lattice_osr_decode_step(*(t[n][:, 39:].contiguous() for n in names), Sp)
    torch.cuda.synchronize()
    assert (yd[:, 0] - y[:, 39]).abs().max().item() <= 1e-5 * y.abs().max().item()
    assert (Sd - S).abs().max().item() <= 1e-5


@pytest.mark.parametrize("entry,C", [("chunked", 64), ("recurrent", None), ("decode", None)])
def test_deterministic(entry, C):
    _say(f"determinism {entry}")
    T = 1 if entry == "decode" else 256
    inp = synth.make_inputs(2, T, 4, 64, 64, seed=13, in_dtype=synth.BF16)
    y1, S1 = _run(entry, inp, C)
    y2, S2 = _run(entry, inp, C)
    assert torch.equal(y1, y2) and torch.equal(S1, S2)


# ----------------------------------------------------- MFMA chunk schedules --
SCHED = {"split": osr.SCHED_SPLIT, "fused": osr.SCHED_FUSED}
MFMA_CASES = [(16, 16, 16), (32, 32, 32), (64, 64, 64), (64, 128, 64), (128, 64, 32), (128, 128, 128),
              (32, 128, 16), (128, 32, 64)]


@pytest.mark.parametrize("schedule", ["split", "fused"])
@pytest.mark.parametrize("m,d,C", MFMA_CASES)
def test_mfma_schedules(schedule, m, d, C):
    _say(f"mfma schedule={schedule} m={m} d={d} C={C}")
    inp = synth.make_inputs(2, 4 * C, 3, m, d, seed=100 + m + 3 * d + C, in_dtype=synth.BF16)
    y, S = _run("chunked", inp, C, schedule=SCHED[schedule])
    _check(inp, y, S, C, osr.MODE_DEC)


# Encoding layer on both MFMA schedules over the shapes of the sweep above
# (the read-out is mode-independent; the state passing and the fused kernel
# start H at +V and write with gamma (c - k)).
@pytest.mark.parametrize("schedule", ["split", "fused"])
@pytest.mark.parametrize("m,d,C", [(16, 16, 16), (64, 64, 64), (64, 128, 64), (128, 128, 128), (32, 128, 16)])
def test_mfma_schedules_encoding(schedule, m, d, C):
    _say(f"mfma encoding layer schedule={schedule} m={m} d={d} C={C}")
    inp = synth.make_inputs(2, 4 * C, 3, m, d, seed=700 + m + 3 * d + C, in_dtype=synth.BF16)
    y, S = _run("chunked", inp, C, mode=osr.MODE_ENC, schedule=SCHED[schedule])
    _check(inp, y, S, C, osr.MODE_ENC)


# Odd chunk counts: the read-out kernel then takes one chunk per workgroup
# (its chunk groups must divide the count), and (b,h) counts that are not
# powers of two.
@pytest.mark.parametrize("schedule", ["split", "fused"])
@pytest.mark.parametrize("m,d,C,nc", [(64, 64, 64, 5), (64, 128, 64, 3), (128, 128, 128, 3), (32, 64, 32, 7),
                                      (16, 32, 16, 9)])
def test_mfma_odd_chunk_counts(schedule, m, d, C, nc):
    _say(f"mfma schedule={schedule} m={m} d={d} C={C} chunks={nc}")
    inp = synth.make_inputs(3, nc * C, 5, m, d, seed=600 + m + d + nc, in_dtype=synth.BF16)
    y, S = _run("chunked", inp, C, schedule=SCHED[schedule])
    _check(inp, y, S, C, osr.MODE_DEC)


@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM, osr.MODE_ENC])
def test_mfma_split_and_fused_agree(mode):
    _say(f"mfma split vs fused mode={mode}")
    inp = synth.make_inputs(2, 256, 2, 64, 64, seed=77, in_dtype=synth.BF16)
    ys, Ss = _run("chunked", inp, 64, mode=mode, schedule=osr.SCHED_SPLIT)
    yf, Sf = _run("chunked", inp, 64, mode=mode, schedule=osr.SCHED_FUSED)
    # The schedules evaluate the same chunk formula with different sub-block
    # lengths and MFMA shapes, so they agree to the rounding of the split-bf16
    # products (about 2^-16 relative each, summed over tens of products per
    # output), not bit for bit; each one separately meets the oracle tolerance.
    assert (ys - yf).abs().max().item() <= 2e-4 * ys.abs().max().item()
    assert (Ss - Sf).abs().max().item() <= 1e-4


# ------------------------------------ state passing with and without pairs --
# Pairs run for m <= 32 with C >= 32; the m = 64 case checks that the
# override leaves the one-wave kernel in place there.
PAIR_CASES = [(32, 32, 32), (32, 32, 64), (16, 64, 64), (16, 16, 32), (32, 64, 64), (32, 128, 32), (64, 64, 64)]
PAIRS = {"1": osr.PAIRS_AUTO, "0": osr.PAIRS_OFF}


@pytest.mark.parametrize("pairs", ["1", "0"])
@pytest.mark.parametrize("m,d,C", PAIR_CASES)
def test_chain_pairs(pairs, m, d, C):
    """Shapes where a chunk is one sub-block: the two-waves-per-slot-block
    state passing (default) and the one-wave form, both against the oracle,
    over several chunks and both objectives."""
    _say(f"state passing pairs={pairs} m={m} d={d} C={C}")
    for mode in (osr.MODE_DEC, osr.MODE_SIM):
        inp = synth.make_inputs(2, 6 * C, 2, m, d, seed=300 + m + d + C + mode, in_dtype=synth.BF16)
        y, S = _run("chunked", inp, C, mode=mode, schedule=osr.SCHED_SPLIT, chain_pairs=PAIRS[pairs])
        _check(inp, y, S, C, mode)


def test_chain_pairs_agree():
    """The pair split regroups the chunk's suffix products exactly; the two
    forms agree to the split-bf16 rounding of their products."""
    _say("state passing pairs vs one wave per slot block")
    inp = synth.make_inputs(2, 512, 2, 32, 64, seed=404, in_dtype=synth.BF16)
    y1, S1 = _run("chunked", inp, 64, schedule=osr.SCHED_SPLIT, chain_pairs=osr.PAIRS_AUTO)
    y0, S0 = _run("chunked", inp, 64, schedule=osr.SCHED_SPLIT, chain_pairs=osr.PAIRS_OFF)
    assert (y1 - y0).abs().max().item() <= 2e-4 * y0.abs().max().item()
    assert (S1 - S0).abs().max().item() <= 1e-4


@pytest.mark.parametrize("pairs", ["1", "0"])
@pytest.mark.parametrize("m,d,C", [(32, 32, 64), (16, 64, 64), (32, 128, 32), (64, 128, 64), (128, 64, 128)])
def test_chain_pairs_first_linearisation(pairs, m, d, C):
    """The first linearisation on the matrix cores, with the state passing in
    both its pair and one-wave forms (where a chunk is one sub-block) and in
    sub-blocks (m64 d128 C64, m128 d64 C128), several chunks, all objectives."""
    _say(f"first linearisation, state passing pairs={pairs} m={m} d={d} C={C}")
    for mode in (osr.MODE_DEC, osr.MODE_SIM, osr.MODE_ENC):
        inp = synth.make_inputs(2, 4 * C, 2, m, d, seed=900 + m + d + C + mode, in_dtype=synth.BF16)
        t = osr.to_device(inp)
        y, S = osr.lattice_osr_fwd_chunked(t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"], C,
                                           mode=mode, linearisation=osr.LIN1, chain_pairs=PAIRS[pairs])
        torch.cuda.synchronize()
        _check_lin1(inp, y, S, C, mode)


def test_first_linearisation_ignores_fused_override():
    """The first linearisation runs on the split schedule even where the
    default would take the fused kernel (many sequences) or it is asked for."""
    _say("first linearisation with the fused schedule asked for, B32 H8 m64 d64 C64")
    inp = synth.make_inputs(32, 128, 8, 64, 64, seed=950, in_dtype=synth.BF16)
    t = osr.to_device(inp)
    y, S = osr.lattice_osr_fwd_chunked(t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"], 64,
                                       linearisation=osr.LIN1, schedule=osr.SCHED_FUSED)
    torch.cuda.synchronize()
    _check_lin1(inp, y, S, 64, osr.MODE_DEC)


# ------------------------- state passing split over several workgroups --
# Where a chunk is 2 or 4 sub-blocks of the state-passing kernel and the
# sequences are few, each sub-block of every chunk runs on its own workgroup
# and the workgroups exchange their parts of the chunk-end state
# (chain_wgs AUTO); chain_wgs ONE keeps one workgroup per sequence.  Shapes
# (m, d, C) with 2 or 4 sub-blocks per chunk, several chunks, (b,h) counts
# that are not multiples of 8, every objective and both linearisations.
WGS_CASES = [(128, 128, 128), (128, 128, 64), (128, 64, 128), (64, 128, 64), (64, 128, 128), (32, 128, 64),
             (16, 128, 128), (64, 64, 128), (32, 32, 128)]


@pytest.mark.parametrize("m,d,C", WGS_CASES)
@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM, osr.MODE_ENC])
def test_chain_workgroup_split(m, d, C, mode):
    _say(f"state passing over several workgroups m={m} d={d} C={C} mode={mode}")
    inp = synth.make_inputs(3, 4 * C, 5, m, d, seed=1100 + m + d + C + mode, in_dtype=synth.BF16)
    ys, Ss = _run("chunked", inp, C, mode=mode, chain_wgs=osr.WGS_AUTO)
    y1, S1 = _run("chunked", inp, C, mode=mode, chain_wgs=osr.WGS_ONE)
    _check(inp, ys, Ss, C, mode)
    _check(inp, y1, S1, C, mode)
    # the same chunk formula with the chunk-end sum regrouped by sub-block:
    # the two agree to the rounding of the split products (the encoding
    # layer amplifies such differences; there each meets the bar on its own)
    if mode != osr.MODE_ENC:
        assert (ys - y1).abs().max().item() <= 2e-4 * y1.abs().max().item()
        assert (Ss - S1).abs().max().item() <= 1e-4


@pytest.mark.parametrize("m,d,C", [(128, 128, 128), (64, 128, 64)])
def test_chain_workgroup_split_first_linearisation(m, d, C):
    _say(f"state passing over several workgroups, first linearisation m={m} d={d} C={C}")
    inp = synth.make_inputs(2, 4 * C, 3, m, d, seed=1200 + m + d + C, in_dtype=synth.BF16)
    t = osr.to_device(inp)
    y, S = osr.lattice_osr_fwd_chunked(t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"], C,
                                       linearisation=osr.LIN1)
    torch.cuda.synchronize()
    _check_lin1(inp, y, S, C, osr.MODE_DEC)


def test_chain_workgroup_split_deterministic():
    _say("state passing over several workgroups: bit-identical reruns, B1 H16 T2048 m=d=128 C128")
    inp = synth.make_inputs(1, 2048, 16, 128, 128, seed=1300, in_dtype=synth.BF16, mu_mean=3.0)
    y1, S1 = _run("chunked", inp, 128)
    y2, S2 = _run("chunked", inp, 128)
    assert torch.equal(y1, y2) and torch.equal(S1, S2)


# The read-out overlapped with the state passing by chunk ranges (64 chunks or
# a multiple: 4 ranges, the state handed from range to range unprojected):
# the same kernels over the same chunks, so the results equal those of the
# serial launch bit for bit, and meet the bar against the oracle.
OVERLAP_CASES = [  # (B, H, m, d, C, chunks): workgroups per sequence 4, 2 and 1; 96 sequences (equal ranges)
    (1, 2, 128, 128, 128, 64), (1, 3, 128, 128, 64, 128), (2, 3, 64, 64, 32, 64), (1, 2, 32, 128, 64, 64),
    (4, 24, 32, 32, 16, 64),
]


@pytest.mark.parametrize("B,H,m,d,C,nc", OVERLAP_CASES)
@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM])
def test_overlapped_readout(B, H, m, d, C, nc, mode):
    _say(f"read-out overlapped by chunk ranges B{B} H{H} m={m} d={d} C={C} chunks={nc} mode={mode}")
    inp = synth.make_inputs(B, nc * C, H, m, d, seed=1400 + m + d + C + nc + mode, in_dtype=synth.BF16)
    yo, So = _run("chunked", inp, C, mode=mode)
    ys, Ss = _run("chunked", inp, C, mode=mode, readout_overlap=osr.OVERLAP_OFF)
    assert torch.equal(yo, ys) and torch.equal(So, Ss)
    _check(inp, yo, So, C, mode)


def test_overlapped_readout_first_linearisation_and_bf16_y():
    _say("read-out overlapped by chunk ranges, first linearisation and bf16 y, B1 H2 m=d=128 C128, 64 chunks")
    inp = synth.make_inputs(1, 64 * 128, 2, 128, 128, seed=1500, in_dtype=synth.BF16)
    for kw in ({"linearisation": osr.LIN1}, {"y_dtype": torch.bfloat16}):
        yo, So = _run("chunked", inp, 128, **kw)
        ys, Ss = _run("chunked", inp, 128, readout_overlap=osr.OVERLAP_OFF, **kw)
        assert torch.equal(yo, ys) and torch.equal(So, Ss), kw
    _check_lin1(inp, *_run("chunked", inp, 128, linearisation=osr.LIN1), 128, osr.MODE_DEC)


def test_overlapped_readout_on_a_side_stream_of_the_caller():
    """A call on a stream other than the current one: the outputs are final
    once that stream is synchronised (its last work waits for the library's
    side stream)."""
    _say("read-out overlapped, caller's own stream, B1 H2 m=d=64 C32, 64 chunks")
    inp = synth.make_inputs(1, 64 * 32, 2, 64, 64, seed=1600, in_dtype=synth.BF16)
    t = osr.to_device(inp)
    args = (t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"])
    ref_y, ref_S = osr.lattice_osr_fwd_chunked(*args, 32, readout_overlap=osr.OVERLAP_OFF)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    y, S = osr.lattice_osr_fwd_chunked(*args, 32, stream=s)
    s.synchronize()
    assert torch.equal(y, ref_y) and torch.equal(S, ref_S)
