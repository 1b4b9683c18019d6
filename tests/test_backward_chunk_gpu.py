"""GPU parity of the chunk-parallel backward (lattice_osr_bwd_chunked with
desc.bwd_form = LATTICE_OSR_BWD_CHUNK: the matrix form of the chunk's
vector-Jacobian product on the fp32 matrix cores) against the fp64 gradient
oracle (oracle/osr_backward.py), and against the token walk (BWD_WALK).

It is built for m = d = C = 64 with bf16 inputs, the default linearisation
and the decoding and similarity objectives.  Bars: the backward's (max-abs
error over the oracle gradient's RMS at most 2e-2 for bf16 inputs); the two
forms evaluate the same fp32 gradient of the same chunk-start states, so they
agree to 1e-4 of RMS (fp32 rounding of differently ordered sums).
"""
import sys

import numpy as np
import pytest
import torch

from compressed_memory_linear_amd import osr, synth
from oracle import osr_backward as ob

pytestmark = pytest.mark.gpu

TOL = 2e-2
AGREE = 1e-4
KEYS = ("dq", "dk", "dv", "dgamma", "dmu", "dstate_in")


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
    return float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2)))


def _upstream(inp, seed, dy_bf16=False):
    rng = np.random.Generator(np.random.PCG64(seed + 500))
    dy = rng.standard_normal((inp.B, inp.T, inp.H, inp.d), dtype=np.float32)
    dso = rng.standard_normal((inp.B, inp.H, inp.m, inp.d), dtype=np.float32)
    if dy_bf16:
        dy = synth.bf16_bits_to_f32(synth.bf16_round_bits(dy))
    return dy, dso


def _gpu_bwd(inp, dy, dso, mode, form, dy_bf16=False):
    t = osr.to_device(inp, "cuda")
    dyt = torch.from_numpy(dy).cuda()
    if dy_bf16:
        dyt = dyt.to(torch.bfloat16)   # exact: dy already holds bf16 values
    g = osr.lattice_osr_bwd_chunked(t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"], dyt,
                                    torch.from_numpy(dso).cuda(), 64, mode=mode, bwd_form=form)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def _compare(inp, dy, dso, mode, dy_bf16=False, agree_bar=AGREE):
    chunk = _gpu_bwd(inp, dy, dso, mode, osr.BWD_CHUNK, dy_bf16)
    walk = _gpu_bwd(inp, dy, dso, mode, osr.BWD_WALK, dy_bf16)
    ref = ob.osr_backward(*inp.values_f64(), dy, dso, chunk_size=64, mode=mode)
    errs = {k: _rel(chunk[k], ref[k]) for k in KEYS}
    agree = {k: _rel(chunk[k], walk[k]) for k in KEYS}
    _say("  vs oracle " + ", ".join(f"{k} {e:.2e}" for k, e in errs.items()))
    _say("  vs walk   " + ", ".join(f"{k} {e:.2e}" for k, e in agree.items()))
    for k in KEYS:
        assert np.isfinite(chunk[k]).all(), k
        assert errs[k] <= TOL, (k, errs[k])
        assert agree[k] <= agree_bar, (k, agree[k])


@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM])
@pytest.mark.parametrize("per_slot", [True, False])
@pytest.mark.parametrize("dy_bf16", [False, True])
def test_chunk_form_small(mode, per_slot, dy_bf16):
    """B2 H2 T256 (four chunks of four tiles), every objective it covers, both
    gamma layouts, fp32 and bf16 dy."""
    _say(f"bwd chunk form B2 H2 T256 m=d=C=64 mode{mode} per_slot{per_slot} dy_bf16{dy_bf16}")
    inp = synth.make_inputs(2, 256, 2, 64, 64, seed=3100 + mode + 2 * per_slot, in_dtype=synth.BF16,
                            gamma_per_slot=per_slot)
    dy, dso = _upstream(inp, 3100, dy_bf16)
    _compare(inp, dy, dso, mode, dy_bf16)


def test_chunk_form_one_chunk():
    """A single chunk (T = C): only the returned state's projection feeds lambda."""
    _say("bwd chunk form B1 H3 T64")
    inp = synth.make_inputs(1, 64, 3, 64, 64, seed=3200, in_dtype=synth.BF16)
    dy, dso = _upstream(inp, 3200)
    _compare(inp, dy, dso, osr.MODE_DEC)


@pytest.mark.parametrize("which", ["near0", "one"])
def test_chunk_form_decay_extremes(which):
    """mu in [1e-3, 1e-2] and mu = 1 (no decay).  With mu near 0 the gate
    products over half a tile reach ~1e-16, and the tile's causal products pair
    factors up to ~1e16 with ones down to ~1e-16: fp32 keeps their ratio but
    not every digit of the sums, so the two forms agree there to 5e-3 of RMS
    (measured 1.6e-3), each well within the 2e-2 bar of the oracle."""
    _say(f"bwd chunk form, mu {which}")
    inp = synth.make_inputs(1, 256, 2, 64, 64, seed=3300, in_dtype=synth.BF16)
    rng = np.random.default_rng(3301)
    mu = rng.uniform(1e-3, 1e-2, inp.mu.shape) if which == "near0" else np.ones(inp.mu.shape)
    inp.mu = synth.bf16_round_bits(mu.astype(np.float32))  # (bf16 inputs are stored as bit patterns)
    dy, dso = _upstream(inp, 3300)
    _compare(inp, dy, dso, osr.MODE_DEC, agree_bar=5e-3 if which == "near0" else AGREE)


def test_chunk_form_zero_write():
    """gamma = 0: nothing is written, y_t = sum_i q_{t,i} z_i.  Then dk, dv and
    dmu vanish in exact arithmetic (the gates no longer depend on h, and
    g = beta mu = 1): dk and dv come out exactly zero, and dmu, a sum over the
    64 slots of dg beta (1 - beta^2 mu^2) with beta = 1/mu up to an ulp, is
    zero to fp32 rounding (measured 2e-5 of dq's RMS; bar 1e-4); dq, dgamma
    and the state's gradient meet the bar."""
    _say("bwd chunk form, gamma = 0")
    inp = synth.make_inputs(1, 128, 2, 64, 64, seed=3400, in_dtype=synth.BF16)
    inp.gamma = synth.bf16_round_bits(np.zeros(inp.gamma.shape, np.float32))
    dy, dso = _upstream(inp, 3400)
    got = _gpu_bwd(inp, dy, dso, osr.MODE_SIM, osr.BWD_CHUNK)
    ref = ob.osr_backward(*inp.values_f64(), dy, dso, chunk_size=64, mode=osr.MODE_SIM)
    scale = float(np.sqrt(np.mean(ref["dq"] ** 2)))
    for k in ("dq", "dgamma", "dstate_in"):
        e = _rel(got[k], ref[k])
        _say(f"  {k} {e:.2e}")
        assert e <= TOL, (k, e)
    for k in ("dk", "dv", "dmu"):
        z = float(np.max(np.abs(got[k]))) / scale
        _say(f"  max |{k}| / rms(dq) = {z:.2e}")
        assert z <= 1e-4, (k, z)


def test_chunk_form_deterministic():
    _say("bwd chunk form, bit-identical reruns B2 H2 T256")
    inp = synth.make_inputs(2, 256, 2, 64, 64, seed=3500, in_dtype=synth.BF16)
    dy, dso = _upstream(inp, 3500)
    a = _gpu_bwd(inp, dy, dso, osr.MODE_DEC, osr.BWD_CHUNK)
    b = _gpu_bwd(inp, dy, dso, osr.MODE_DEC, osr.BWD_CHUNK)
    for key in KEYS:
        assert np.array_equal(a[key], b[key]), key
