"""GPU parity of the backward at small chunks (C = 1, 2, 4, 8, and 16 with bf16
inputs), where the automatic form is the small-chunk reverse walk (the chunk's
per-token states in registers; its phase 1 the forward's small-chunk token
loop, or at C = 16 the matrix-core state passing), against the
fp64 gradient oracle (oracle/osr_backward.py) and against the general walk
(desc.bwd_form = LATTICE_OSR_BWD_WALK).

Bars: the backward's (max-abs error over the oracle gradient's RMS at most
1e-4 for fp32 inputs, 2e-2 for bf16 inputs).  Both walks evaluate the same
fp32 gradient from chunk-start states that their forwards form in different
orders, so they agree to 1e-4 of RMS on short sequences and to 1e-3 over the
2048 tokens (512 chunks) of the full workload.  Shapes span every (m, d)
class the form is built for: one and two slot rows per thread, d from 16 to
128, one chunk and many, per-slot and per-token gamma, fp32 and bf16 dy, and
all three objectives (the encoding layer on short sequences, where its
gradient's sensitivity to rounding stays below the bar).
"""
import concurrent.futures as cf
import sys

import numpy as np
import pytest
import torch

from compressed_memory_linear_amd import osr, synth
from oracle import osr_backward as ob

pytestmark = pytest.mark.gpu

TOL = {synth.F32: 1e-4, synth.BF16: 2e-2}
AGREE = 1e-4
AGREE_LONG = 1e-3
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


def _gpu_bwd(inp, dy, dso, C, mode, form, dy_bf16=False, wgs=osr.WGS_AUTO, lin=osr.LIN2):
    t = osr.to_device(inp, "cuda")
    dyt = torch.from_numpy(dy).cuda()
    if dy_bf16:
        dyt = dyt.to(torch.bfloat16)  # exact: dy already holds bf16 values
    g = osr.lattice_osr_bwd_chunked(t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"], dyt,
                                    torch.from_numpy(dso).cuda(), C, mode=mode, bwd_form=form, chain_wgs=wgs,
                                    linearisation=lin)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def _oracle_seq(inp, dy, dso, C, mode, b, h):
    q, k, v, g, mu, S = inp.values_f64()
    sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
    return ob.osr_backward(q[sl], k[sl], v[sl], g[sl], mu[b:b + 1, :, h:h + 1], S[b:b + 1, h:h + 1],
                           dy[sl], dso[b:b + 1, h:h + 1], chunk_size=C, mode=mode)


def _pick(key, arr, b, h):
    return arr[b, h] if key == "dstate_in" else arr[b, :, h]


def _errs(got, ref):
    return {key: _rel(got[key], ref[key]) for key in KEYS}


def _report_and_check(label, errs, bar):
    _say(f"  {label}: " + ", ".join(f"{k} {e:.2e}" for k, e in errs.items()) + f" (bar {bar:g})")
    for key, e in errs.items():
        assert e <= bar, (label, key, e)


# (B, T, H, m, d, C, in dtype, per-slot gamma, objective, bf16 dy)
CASES = [
    (1, 64, 2, 16, 16, 2, synth.F32, True, osr.MODE_DEC, False),
    (1, 64, 2, 16, 32, 4, synth.F32, False, osr.MODE_DEC, False),
    (2, 96, 2, 32, 32, 8, synth.F32, True, osr.MODE_DEC, False),
    (1, 64, 2, 64, 64, 4, synth.F32, True, osr.MODE_DEC, False),
    (1, 64, 3, 64, 64, 2, synth.F32, False, osr.MODE_SIM, False),
    (1, 64, 2, 64, 64, 8, synth.BF16, True, osr.MODE_DEC, False),
    (2, 64, 2, 32, 128, 4, synth.BF16, True, osr.MODE_DEC, True),
    (1, 32, 2, 16, 128, 4, synth.F32, True, osr.MODE_SIM, False),
    (1, 32, 2, 128, 32, 2, synth.BF16, False, osr.MODE_SIM, True),
    (1, 64, 2, 128, 16, 8, synth.BF16, True, osr.MODE_DEC, False),
    (1, 4, 2, 64, 64, 4, synth.F32, True, osr.MODE_DEC, False),    # one chunk
    (1, 8, 2, 16, 32, 4, synth.F32, True, osr.MODE_ENC, False),    # encoding layer, short
    (1, 8, 2, 32, 32, 2, synth.F32, False, osr.MODE_ENC, False),
    # m d = 8192 and m = d = 128: the rows over at least 2 or 4 workgroups
    (2, 64, 2, 64, 128, 4, synth.BF16, True, osr.MODE_DEC, False),
    (1, 64, 2, 128, 64, 2, synth.F32, False, osr.MODE_SIM, True),
    (1, 32, 2, 128, 128, 2, synth.BF16, True, osr.MODE_DEC, False),
    # C = 1: the exact recurrence (a projection after every token)
    (1, 64, 2, 64, 64, 1, synth.BF16, True, osr.MODE_DEC, False),
    (1, 32, 2, 16, 32, 1, synth.F32, False, osr.MODE_SIM, True),
    # per-token gamma with the rows split (its gradient travels in the exchanged sums)
    (2, 64, 2, 64, 64, 4, synth.BF16, False, osr.MODE_DEC, False),
    (1, 64, 2, 64, 64, 8, synth.F32, False, osr.MODE_SIM, False),
    # C = 16 (bf16 inputs): after the matrix-core state passing, h from its fragments
    (2, 64, 2, 64, 64, 16, synth.BF16, True, osr.MODE_DEC, False),
    (1, 64, 3, 32, 32, 16, synth.BF16, False, osr.MODE_SIM, True),
    (1, 64, 2, 64, 32, 16, synth.BF16, True, osr.MODE_DEC, True),
]


@pytest.mark.parametrize("B,T,H,m,d,C,dt,per_slot,mode,dyb", CASES)
def test_small_chunk_backward(B, T, H, m, d, C, dt, per_slot, mode, dyb):
    _say(f"bwd small-chunk B{B} T{T} H{H} m{m} d{d} C{C} {'bf16' if dt == synth.BF16 else 'fp32'} "
         f"per_slot{per_slot} mode{mode} dy_bf16{dyb}")
    inp = synth.make_inputs(B, T, H, m, d, seed=31 + C, in_dtype=dt, gamma_per_slot=per_slot)
    dy, dso = _upstream(inp, 31 + C, dy_bf16=dyb)
    got = _gpu_bwd(inp, dy, dso, C, mode, osr.BWD_AUTO, dy_bf16=dyb)
    for key in KEYS:
        assert np.isfinite(got[key]).all(), key
    ref = ob.osr_backward(*inp.values_f64(), dy, dso, chunk_size=C, mode=mode)
    _report_and_check("vs oracle", _errs(got, ref), TOL[dt])
    walk = _gpu_bwd(inp, dy, dso, C, mode, osr.BWD_WALK, dy_bf16=dyb)
    _report_and_check("vs general walk", _errs(got, walk), AGREE)


# (B, T, H, m, d, C, objective): from m = 32 and C = 4 the automatic choice splits
# the slot rows of each sequence over two workgroups (four at C = 8 where a
# quarter of the rows can stage a chunk: m64 d64 and m128 d32 here) that exchange
# each chunk's sums
@pytest.mark.parametrize("B,T,H,m,d,C,mode", [(2, 128, 3, 64, 64, 4, osr.MODE_DEC), (1, 64, 2, 32, 128, 4, osr.MODE_DEC),
                                              (2, 64, 2, 128, 16, 8, osr.MODE_SIM), (1, 96, 4, 32, 32, 8, osr.MODE_DEC),
                                              (1, 64, 4, 64, 64, 8, osr.MODE_DEC), (2, 16, 2, 128, 32, 8, osr.MODE_ENC)])
def test_small_chunk_backward_split_vs_one(B, T, H, m, d, C, mode):
    """The split over workgroups against one workgroup per sequence
    (LATTICE_OSR_WGS_ONE): the same gradient up to the order of the fp32
    sums over slots (1e-4 of RMS), bit-identical on a rerun."""
    _say(f"bwd small-chunk split vs one B{B} T{T} H{H} m{m} d{d} C{C} mode{mode}")
    inp = synth.make_inputs(B, T, H, m, d, seed=41, in_dtype=synth.BF16)
    dy, dso = _upstream(inp, 41)
    split = _gpu_bwd(inp, dy, dso, C, mode, osr.BWD_AUTO)
    one = _gpu_bwd(inp, dy, dso, C, mode, osr.BWD_AUTO, wgs=osr.WGS_ONE)
    _report_and_check("split vs one workgroup", _errs(split, one), AGREE)
    again = _gpu_bwd(inp, dy, dso, C, mode, osr.BWD_AUTO)
    for key in KEYS:
        assert np.array_equal(split[key], again[key]), key


# The policy's other branches: B*H = 160 (B*H*2 > 256: one workgroup per sequence)
# at C = 4, B*H = 100 at C = 8 (B*H*4 > 256: two workgroups, not four), and at
# m64 d128 B*H = 128 (two workgroups, the fewest that shape allows, filling 256)
@pytest.mark.parametrize("B,H,m,d,C", [(4, 40, 64, 64, 4), (4, 25, 64, 64, 8), (8, 16, 64, 128, 4)])
def test_small_chunk_backward_many_sequences(B, H, m, d, C):
    _say(f"bwd small-chunk many sequences B{B} T32 H{H} m{m} d{d} C{C} bf16")
    inp = synth.make_inputs(B, 32, H, m, d, seed=43, in_dtype=synth.BF16)
    dy, dso = _upstream(inp, 43)
    got = _gpu_bwd(inp, dy, dso, C, osr.MODE_DEC, osr.BWD_AUTO)
    walk = _gpu_bwd(inp, dy, dso, C, osr.MODE_DEC, osr.BWD_WALK)
    _report_and_check("vs general walk", _errs(got, walk), AGREE)
    bh = [(0, 0), (B - 1, H - 1)]
    refs = [_oracle_seq(inp, dy, dso, C, osr.MODE_DEC, b, h) for b, h in bh]
    errs = {key: max(_rel(_pick(key, got[key], b, h), _pick(key, r[key], 0, 0)) for (b, h), r in zip(bh, refs))
            for key in KEYS}
    _report_and_check("vs oracle (2 sequences)", errs, TOL[synth.BF16])


# The first chunk linearisation (eq. recurrence_linear1) in the same form:
# (B, T, H, m, d, C, in dtype, per-slot gamma, objective) over one, two and four
# workgroups (its encoding layer: the stated short case of test_backward_gpu.py,
# C4 T8 seed 23, which takes this form too)
LIN1_CASES = [(1, 64, 2, 16, 32, 4, synth.F32, True, osr.MODE_DEC), (2, 64, 2, 64, 64, 4, synth.BF16, True, osr.MODE_DEC),
              (1, 64, 2, 64, 64, 8, synth.BF16, False, osr.MODE_SIM), (1, 64, 3, 32, 32, 2, synth.F32, False, osr.MODE_DEC)]


@pytest.mark.parametrize("B,T,H,m,d,C,dt,per_slot,mode", LIN1_CASES)
def test_small_chunk_backward_first_linearisation(B, T, H, m, d, C, dt, per_slot, mode):
    _say(f"bwd small-chunk LIN1 B{B} T{T} H{H} m{m} d{d} C{C} mode{mode} per_slot{per_slot}")
    inp = synth.make_inputs(B, T, H, m, d, seed=59, in_dtype=dt, gamma_per_slot=per_slot)
    dy, dso = _upstream(inp, 59)
    got = _gpu_bwd(inp, dy, dso, C, mode, osr.BWD_AUTO, lin=osr.LIN1)
    ref = ob.osr_backward(*inp.values_f64(), dy, dso, chunk_size=C, mode=mode, linearisation=ob.LIN1)
    _report_and_check("vs oracle", _errs(got, ref), TOL[dt])
    walk = _gpu_bwd(inp, dy, dso, C, mode, osr.BWD_WALK, lin=osr.LIN1)
    _report_and_check("vs general walk", _errs(got, walk), AGREE)


def test_small_chunk_backward_deterministic():
    _say("bwd small-chunk determinism B2 T128 H2 m64 d64 C4 bf16")
    inp = synth.make_inputs(2, 128, 2, 64, 64, seed=37, in_dtype=synth.BF16)
    dy, dso = _upstream(inp, 37)
    a = _gpu_bwd(inp, dy, dso, 4, osr.MODE_DEC, osr.BWD_AUTO)
    b = _gpu_bwd(inp, dy, dso, 4, osr.MODE_DEC, osr.BWD_AUTO)
    for key in KEYS:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("C", [4, 8, 16])
def test_small_chunk_backward_workload_sampled(C):
    """B4 H8 T2048 m64 d64 (the training workload's shape) at C = 4, 8, 16:
    against the general walk in full, and two whole sequences against the
    oracle."""
    _say(f"bwd small-chunk workload B4 H8 T2048 m64 d64 C{C} bf16, sampled (b,h)")
    inp = synth.workload_inputs("chunked_b4h8_t2048_m64d64_c64")
    dy, dso = _upstream(inp, 23)
    got = _gpu_bwd(inp, dy, dso, C, osr.MODE_DEC, osr.BWD_AUTO)
    walk = _gpu_bwd(inp, dy, dso, C, osr.MODE_DEC, osr.BWD_WALK)
    _report_and_check("vs general walk", _errs(got, walk), AGREE_LONG)
    bh = [(0, 0), (3, 7)]
    with cf.ThreadPoolExecutor(2) as ex:
        refs = list(ex.map(lambda p: _oracle_seq(inp, dy, dso, C, osr.MODE_DEC, *p), bh))
    errs = {key: max(_rel(_pick(key, got[key], b, h), _pick(key, r[key], 0, 0)) for (b, h), r in zip(bh, refs))
            for key in KEYS}
    _report_and_check("vs oracle (2 sequences)", errs, TOL[synth.BF16])


# (B, T, H, m, d, C, in dtype, objective, bf16 y and dy)
SAVED_CASES = [(2, 64, 3, 64, 64, 4, synth.BF16, osr.MODE_DEC, False), (1, 64, 2, 16, 32, 2, synth.F32, osr.MODE_DEC, False),
               (1, 64, 4, 64, 64, 8, synth.BF16, osr.MODE_SIM, True), (2, 32, 2, 32, 128, 4, synth.BF16, osr.MODE_DEC, True),
               (1, 16, 2, 32, 32, 4, synth.F32, osr.MODE_ENC, False), (1, 32, 2, 128, 128, 2, synth.BF16, osr.MODE_DEC, False),
               (2, 24, 3, 64, 32, 1, synth.BF16, osr.MODE_DEC, True), (1, 16, 2, 16, 16, 1, synth.F32, osr.MODE_SIM, False)]


@pytest.mark.parametrize("lin", [osr.LIN2, osr.LIN1])
@pytest.mark.parametrize("B,T,H,m,d,C,dt,mode,bf16_out", SAVED_CASES)
def test_saved_training_pair(B, T, H, m, d, C, dt, mode, bf16_out, lin):
    """lattice_osr_fwd_chunked_save returns lattice_osr_fwd_chunked's y and
    state_out bit for bit, and lattice_osr_bwd_chunked_saved, from what it
    stored, lattice_osr_bwd_chunked's gradients bit for bit (the same kernels
    on the same values; the second backward from the same saved values too)."""
    _say(f"saved training pair B{B} T{T} H{H} m{m} d{d} C{C} mode{mode} bf16 y/dy {bf16_out}")
    inp = synth.make_inputs(B, T, H, m, d, seed=47, in_dtype=dt)
    dy, dso = _upstream(inp, 47, dy_bf16=bf16_out)
    t = osr.to_device(inp, "cuda")
    ydt = torch.bfloat16 if bf16_out else torch.float32
    y0, s0 = osr.lattice_osr_fwd_chunked(t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"], C, mode=mode,
                                         y_dtype=ydt, linearisation=lin)
    y1, s1, saved = osr.lattice_osr_fwd_chunked_save(t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"], C,
                                                     mode=mode, y_dtype=ydt, linearisation=lin)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(s0, s1)
    ref = _gpu_bwd(inp, dy, dso, C, mode, osr.BWD_AUTO, dy_bf16=bf16_out, lin=lin)
    dyt = torch.from_numpy(dy).cuda()
    if bf16_out:
        dyt = dyt.to(torch.bfloat16)
    dsot = torch.from_numpy(dso).cuda()
    for rep in range(2):
        g = osr.lattice_osr_bwd_chunked_saved(t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"], dyt, dsot, C,
                                              saved=saved, mode=mode, linearisation=lin)
        torch.cuda.synchronize()
        for key in KEYS:
            assert np.array_equal(g[key].cpu().numpy(), ref[key]), (rep, key)


def test_small_chunk_backward_long_sequence():
    """B1 H16 T65536 m64 d64 C4 (16384 chunks: the longest workload's length,
    its hand-off tags and buffer parities over a long run): against the
    general walk in full at the long-sequence bar."""
    _say("bwd small-chunk long sequence B1 T65536 H16 m64 d64 C4 bf16")
    inp = synth.make_inputs(1, 65536, 16, 64, 64, seed=53, in_dtype=synth.BF16)
    dy, dso = _upstream(inp, 53)
    got = _gpu_bwd(inp, dy, dso, 4, osr.MODE_DEC, osr.BWD_AUTO)
    for key in KEYS:
        assert np.isfinite(got[key]).all(), key
    walk = _gpu_bwd(inp, dy, dso, 4, osr.MODE_DEC, osr.BWD_WALK)
    _report_and_check("vs general walk", _errs(got, walk), AGREE_LONG)
