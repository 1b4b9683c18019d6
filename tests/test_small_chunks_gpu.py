"""GPU parity of the chunked forward at small chunk sizes (C = 1, 2, 4, 8: the
batched token loop, osr_tokenloop_small_kernel; at C = 1 it is the exact
recurrence, which the recurrent entry runs too) against the fp64 oracle.

The paper trains with C = 4.  Bars as for every forward: max-abs error over
the oracle's RMS at most 1e-4 for fp32 inputs and 2e-2 for bf16 inputs.
Shapes cover every slot-row layout of the loop (rows per thread 1 to 8), the
objectives, the first linearisation, both gamma layouts, the fused GeLU
post-gate, and token counts that end inside a read-out batch.
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
    got = np.asarray(got, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2)))


def _run_check(inp, C, mode=osr.MODE_DEC, lin=osr.LIN2, gate=None):
    t = osr.to_device(inp)
    args = (t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"])
    olin = oracle.LIN1 if lin == osr.LIN1 else oracle.LIN2
    yr, Sr = oracle.osr_forward(*inp.values_f64(), chunk_size=C, mode=mode, linearisation=olin)
    if gate is None:
        y, S = osr.lattice_osr_fwd_chunked(*args, C, mode=mode, linearisation=lin)
    else:
        gt = torch.from_numpy(gate).cuda()  # (float32 values exact in the inputs' dtype)
        if inp.in_dtype == synth.BF16:
            gt = gt.to(torch.bfloat16)
        y, S = osr.lattice_osr_fwd_chunked_gated(t["q"], t["k"], t["v"], t["gamma"], t["mu"], gt, t["state"], C,
                                                 mode=mode, linearisation=lin)
        g64 = gt.float().cpu().numpy().astype(np.float64)
        yr = oracle.glue_gelu_gate(yr, g64)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    S = S.cpu().numpy()
    ey, es = _rel(y, yr), _rel(S, Sr)
    tol = TOL[inp.in_dtype]
    _say(f"  y err/rms = {ey:.3e}, state err/rms = {es:.3e} (tol {tol:g})")
    assert np.isfinite(y).all() and np.isfinite(S).all()
    assert ey <= tol and es <= tol, (ey, es)


SHAPES = [(16, 16), (32, 64), (64, 64), (64, 128), (128, 32), (128, 128)]


@pytest.mark.parametrize("m,d", SHAPES)
@pytest.mark.parametrize("C", [1, 2, 4, 8])
@pytest.mark.parametrize("dt", [synth.F32, synth.BF16])
def test_small_chunks_shapes(m, d, C, dt):
    _say(f"small chunks m={m} d={d} C={C} {dt}")
    inp = synth.make_inputs(2, 96, 2, m, d, seed=4100 + m + d + C, in_dtype=dt)
    _run_check(inp, C)


@pytest.mark.parametrize("mode", [osr.MODE_SIM, osr.MODE_ENC])
@pytest.mark.parametrize("C", [1, 2, 4, 8])
def test_small_chunks_objectives(mode, C):
    # the encoding layer over 32 tokens, where its conditioning keeps fp32 within the bar
    T = 32 if mode == osr.MODE_ENC else 128
    _say(f"small chunks mode={mode} C={C} T={T}")
    inp = synth.make_inputs(1, T, 3, 32, 32, seed=4200 + mode + C, in_dtype=synth.F32)
    _run_check(inp, C, mode=mode)


@pytest.mark.parametrize("C", [1, 2, 4, 8])
@pytest.mark.parametrize("per_slot", [True, False])
def test_small_chunks_first_linearisation(C, per_slot):
    _say(f"small chunks, first linearisation, C={C} per_slot={per_slot}")
    inp = synth.make_inputs(2, 128, 2, 64, 64, seed=4300 + C, in_dtype=synth.F32, gamma_per_slot=per_slot)
    _run_check(inp, C, lin=osr.LIN1)


@pytest.mark.parametrize("C,T", [(4, 4), (4, 12), (4, 20), (4, 36), (1, 1), (1, 13)])
def test_small_chunks_partial_read_out_batch(C, T):
    """Token counts whose last read-out batch is partial (batches of 8 tokens
    at m = d = 64)."""
    _say(f"small chunks C={C} T={T}")
    inp = synth.make_inputs(2, T, 2, 64, 64, seed=4400 + T, in_dtype=synth.F32)
    _run_check(inp, C)


@pytest.mark.parametrize("C", [1, 4])
def test_small_chunks_gated(C):
    _say(f"small chunks with the fused GeLU post-gate, C={C}, bf16")
    inp = synth.make_inputs(2, 64, 2, 64, 64, seed=4500, in_dtype=synth.BF16)
    gate = np.random.default_rng(4501).standard_normal((2, 64, 2, 64)).astype(np.float32)
    _run_check(inp, C, gate=synth.bf16_bits_to_f32(synth.bf16_round_bits(gate)))


@pytest.mark.parametrize("m,d,dt,mode", [(64, 64, synth.BF16, osr.MODE_DEC), (16, 32, synth.F32, osr.MODE_SIM),
                                         (128, 128, synth.BF16, osr.MODE_DEC), (32, 16, synth.F32, osr.MODE_ENC)])
def test_recurrent_equals_chunked_at_one(m, d, dt, mode):
    """The recurrent entry and the chunked forward at C = 1 run the same
    kernel on the same values: equal bit for bit (and within the bar of the
    oracle's exact recurrence)."""
    _say(f"recurrent vs chunked C=1 m={m} d={d} {dt} mode={mode}")
    T = 16 if mode == osr.MODE_ENC else 40
    inp = synth.make_inputs(2, T, 2, m, d, seed=4600 + m + d + mode, in_dtype=dt)
    t = osr.to_device(inp)
    args = (t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"])
    y1, S1 = osr.lattice_osr_fwd_chunked(*args, 1, mode=mode)
    y2, S2 = osr.lattice_osr_fwd_recurrent(*args, mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(S1, S2)
    _run_check(inp, 1, mode=mode)
