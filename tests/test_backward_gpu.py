"""GPU parity of the backward (lattice_osr_bwd_chunked) against the fp64
gradient oracle (oracle/osr_backward.py, itself pinned to finite differences
of the C oracle).

Inputs are seeded and synthetic (compressed_memory_linear_amd.synth); the
upstream gradients dy and dstate_out are N(0, 1) draws from their own seed.
The bar for every gradient tensor is the forward's: max-abs error over the
RMS of the oracle's gradient at most 1e-4 for fp32 inputs and 2e-2 for bf16
inputs.  Small shapes are compared in full; at the workload sizes the oracle
recomputes a sample of whole (batch, head) sequences (sequences are
independent, so their gradients are too).  The encoding layer's gradient
amplifies rounding-size perturbations: it is compared element by element at
the same fixed bars over short sequences where the oracle's own change under
such perturbations stays well below the bar, and at 1024 tokens through a
property that holds at any length.
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


def _gpu_bwd(inp, dy, dso, C, mode, dy_bf16=False, lin=osr.LIN2, chain_wgs=osr.WGS_AUTO, bwd_form=osr.BWD_AUTO):
    t = osr.to_device(inp, "cuda")
    dyt = torch.from_numpy(dy).cuda()
    if dy_bf16:
        dyt = dyt.to(torch.bfloat16)   # exact: dy already holds bf16 values
    g = osr.lattice_osr_bwd_chunked(t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"], dyt,
                                    torch.from_numpy(dso).cuda(), C, mode=mode, linearisation=lin,
                                    chain_wgs=chain_wgs, bwd_form=bwd_form)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def _oracle(inp, dy, dso, C, mode, bh=None, lin=ob.LIN2):
    a = inp.values_f64()
    if bh is None:
        return ob.osr_backward(*a, dy, dso, chunk_size=C, mode=mode, linearisation=lin)
    q, k, v, g, mu, S = a

    def one(pair):
        b, h = pair
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        return ob.osr_backward(q[sl], k[sl], v[sl], g[sl], mu[b:b + 1, :, h:h + 1], S[b:b + 1, h:h + 1],
                               dy[sl], dso[b:b + 1, h:h + 1], chunk_size=C, mode=mode, linearisation=lin)

    with cf.ThreadPoolExecutor(min(len(bh), 8)) as ex:
        return list(ex.map(one, bh))


def _pick(key, arr, b, h):
    if key == "dstate_in":
        return arr[b, h]
    return arr[b, :, h]


def _check(inp, got, ref, tol=None, bh=None):
    tol = tol or TOL[inp.in_dtype]
    errs = {}
    for key in KEYS:
        assert np.isfinite(got[key]).all(), key
        if bh is None:
            errs[key] = _rel(got[key], ref[key])
        else:
            errs[key] = max(_rel(_pick(key, got[key], b, h), _pick(key, r[key], 0, 0))
                            for (b, h), r in zip(bh, ref))
    _say("  " + ", ".join(f"{k} {e:.2e}" for k, e in errs.items()) + f" (tol {tol:g})")
    for key, e in errs.items():
        assert e <= tol, (key, e)


@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM])
@pytest.mark.parametrize("C", [1, 4, 16, 64])
@pytest.mark.parametrize("per_slot", [True, False])
def test_bwd_tiny_fp32(mode, C, per_slot):
    _say(f"bwd tiny fp32 B1 H2 T64 m16 d32 C{C} mode{mode} per_slot{per_slot}")
    inp = synth.make_inputs(1, 64, 2, 16, 32, seed=11, in_dtype=synth.F32, gamma_per_slot=per_slot)
    dy, dso = _upstream(inp, 11)
    _check(inp, _gpu_bwd(inp, dy, dso, C, mode), _oracle(inp, dy, dso, C, mode))


# The encoding layer's gradient is badly conditioned: in the fp64 gradient
# oracle a 1e-7 relative change of every input (fp32 rounding size) moves it by
# up to 2.5e-3 of its RMS at 16 tokens (C = 1) and by 5e-6 - 1e-4 at 4 - 16
# tokens, depending on the draw.  fp32 evaluation can meet the fixed 1e-4 bar
# only where that change is a few 1e-5 or less, so each case is a stated
# (chunk size, length, seed) where the oracle's change at 1e-7 is measured at
# <= 3e-5: C1 T4 seed 23 (per token) 5.9e-6 and seed 11 (per slot) 1.4e-5;
# C4 T8 seed 41 (per slot) 1.5e-5 and seed 31 (per token) 7.9e-6; C16 T16
# seed 11 5.1e-6 (per slot) and 6.3e-6 (per token).
ENC_FP32_CASES = [(1, 4, 23, False), (1, 4, 11, True), (4, 8, 41, True), (4, 8, 31, False), (16, 16, 11, True),
                  (16, 16, 11, False)]


@pytest.mark.parametrize("C,T,seed,per_slot", ENC_FP32_CASES)
def test_bwd_encoding_layer_short_fp32(C, T, seed, per_slot):
    _say(f"bwd encoding layer fp32 B1 H2 T{T} m16 d32 C{C} per_slot{per_slot} seed{seed}")
    inp = synth.make_inputs(1, T, 2, 16, 32, seed=seed, in_dtype=synth.F32, gamma_per_slot=per_slot)
    dy, dso = _upstream(inp, seed)
    _check(inp, _gpu_bwd(inp, dy, dso, C, osr.MODE_ENC), _oracle(inp, dy, dso, C, osr.MODE_ENC))


@pytest.mark.parametrize("m,d", [(16, 16), (32, 64), (64, 64), (64, 128), (128, 32), (128, 128)])
@pytest.mark.parametrize("C", [16, 64])
def test_bwd_shapes_bf16(m, d, C):
    _say(f"bwd bf16 B2 H2 T128 m{m} d{d} C{C}")
    inp = synth.make_inputs(2, 128, 2, m, d, seed=12, in_dtype=synth.BF16)
    dy, dso = _upstream(inp, 12)
    _check(inp, _gpu_bwd(inp, dy, dso, C, osr.MODE_DEC), _oracle(inp, dy, dso, C, osr.MODE_DEC))


# encoding layer: 16 tokens, where a 2^-17 relative change of the inputs moves
# the oracle's gradient by 1.3e-3 of its RMS (2.1e-2 at 32 tokens)
@pytest.mark.parametrize("mode,T", [(osr.MODE_SIM, 128), (osr.MODE_ENC, 16)])
def test_bwd_other_objectives_bf16(mode, T):
    _say(f"bwd bf16 B2 H3 T{T} m64 d64 C16 mode{mode}")
    inp = synth.make_inputs(2, T, 3, 64, 64, seed=13, in_dtype=synth.BF16)
    dy, dso = _upstream(inp, 13)
    _check(inp, _gpu_bwd(inp, dy, dso, 16, mode), _oracle(inp, dy, dso, 16, mode))


@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM, osr.MODE_ENC])
def test_bwd_state_gradient_orthogonal_to_slots(mode):
    """A property at any length: rescaling a slot of the initial state changes
    nothing, so dstate_in . s_i = 0 for every slot (here 1024 tokens, all
    objectives, initial slots of random norms)."""
    _say(f"bwd slot-orthogonality B2 H4 T1024 m64 d64 C64 mode{mode}")
    inp = synth.make_inputs(2, 1024, 4, 64, 64, seed=19, in_dtype=synth.BF16)
    inp.state = (inp.state * np.random.default_rng(4).uniform(0.5, 2.0, size=inp.state.shape[:-1] + (1,))
                 ).astype(np.float32)
    dy, dso = _upstream(inp, 19)
    g = _gpu_bwd(inp, dy, dso, 64, mode)
    ds = g["dstate_in"].astype(np.float64)
    s = inp.state.astype(np.float64)
    cos = np.abs(np.sum(ds * s, -1)) / (np.linalg.norm(ds, axis=-1) * np.linalg.norm(s, axis=-1))
    _say(f"  max |cos(dS_i, s_i)| = {cos.max():.2e}")
    for key in KEYS:
        assert np.isfinite(g[key]).all(), key
    assert cos.max() <= 1e-4


def test_bwd_dy_bf16_and_per_token_gamma():
    _say("bwd bf16 dy, per-token gamma B1 H4 T256 m32 d32 C16")
    inp = synth.make_inputs(1, 256, 4, 32, 32, seed=14, in_dtype=synth.BF16, gamma_per_slot=False)
    dy, dso = _upstream(inp, 14, dy_bf16=True)
    _check(inp, _gpu_bwd(inp, dy, dso, 16, osr.MODE_DEC, dy_bf16=True),
           _oracle(inp, dy, dso, 16, osr.MODE_DEC))


def test_bwd_deterministic():
    _say("bwd determinism B2 H2 T128 m64 d64 C64")
    inp = synth.make_inputs(2, 128, 2, 64, 64, seed=15, in_dtype=synth.BF16)
    dy, dso = _upstream(inp, 15)
    a = _gpu_bwd(inp, dy, dso, 64, osr.MODE_DEC)
    b = _gpu_bwd(inp, dy, dso, 64, osr.MODE_DEC)
    for key in KEYS:
        assert np.array_equal(a[key], b[key]), key


def test_bwd_headline_workload_sampled():
    """B4 H8 T2048 m64 d64 C64 (the chunk-wise training workload), whole
    batch on the GPU, four (b,h) sequences recomputed by the oracle."""
    _say("bwd headline chunked_b4h8_t2048_m64d64_c64, sampled (b,h)")
    inp = synth.workload_inputs("chunked_b4h8_t2048_m64d64_c64")
    dy, dso = _upstream(inp, 16)
    bh = [(0, 0), (1, 5), (2, 3), (3, 7)]
    ref = _oracle(inp, dy, dso, 64, osr.MODE_DEC, bh)
    for form in (osr.BWD_CHUNK, osr.BWD_WALK):
        _say(f"  form {form}")
        _check(inp, _gpu_bwd(inp, dy, dso, 64, osr.MODE_DEC, bwd_form=form), ref, bh=bh)


def test_bwd_d128_workload_sampled():
    """B8 H16 T4096 m64 d128 C64, whole batch on the GPU, two sequences
    recomputed by the oracle."""
    _say("bwd chunked_b8h16_t4096_m64d128_c64, sampled (b,h)")
    inp = synth.workload_inputs("chunked_b8h16_t4096_m64d128_c64")
    dy, dso = _upstream(inp, 17)
    got = _gpu_bwd(inp, dy, dso, 64, osr.MODE_DEC)
    bh = [(0, 0), (7, 15)]
    _check(inp, got, _oracle(inp, dy, dso, 64, osr.MODE_DEC, bh), bh=bh)


def test_bwd_long_context_shape_prefix():
    """The long-context shape (H16, m = d = 128, C128, mu = sigmoid(N(3,1)))
    over its first 2048 tokens, two sequences recomputed by the oracle."""
    _say("bwd chunked_b1h16_t65536_m128d128_c128 first 2048 tokens, sampled (b,h)")
    inp = synth.workload_inputs("chunked_b1h16_t65536_m128d128_c128", T=2048)
    dy, dso = _upstream(inp, 18)
    got = _gpu_bwd(inp, dy, dso, 128, osr.MODE_DEC)
    bh = [(0, 0), (0, 9)]
    _check(inp, got, _oracle(inp, dy, dso, 128, osr.MODE_DEC, bh), bh=bh)


# ---------------------------------------------------------------------------
# The first chunk linearisation (eq. recurrence_linear1)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM])
@pytest.mark.parametrize("C", [4, 16, 64])
@pytest.mark.parametrize("per_slot", [True, False])
def test_bwd_first_linearisation_tiny_fp32(mode, C, per_slot):
    _say(f"bwd LIN1 tiny fp32 B1 H2 T64 m16 d32 C{C} mode{mode} per_slot{per_slot}")
    inp = synth.make_inputs(1, 64, 2, 16, 32, seed=21, in_dtype=synth.F32, gamma_per_slot=per_slot)
    dy, dso = _upstream(inp, 21)
    _check(inp, _gpu_bwd(inp, dy, dso, C, mode, lin=osr.LIN1),
           _oracle(inp, dy, dso, C, mode, lin=ob.LIN1))


@pytest.mark.parametrize("m,d", [(64, 64), (64, 128), (128, 32)])
def test_bwd_first_linearisation_bf16(m, d):
    _say(f"bwd LIN1 bf16 B2 H2 T256 m{m} d{d} C64")
    inp = synth.make_inputs(2, 256, 2, m, d, seed=22, in_dtype=synth.BF16)
    dy, dso = _upstream(inp, 22)
    _check(inp, _gpu_bwd(inp, dy, dso, 64, osr.MODE_DEC, lin=osr.LIN1),
           _oracle(inp, dy, dso, 64, osr.MODE_DEC, lin=ob.LIN1))


# (chunk size, length, seed) where the oracle's gradient moves by <= 1e-5 of
# its RMS under a 1e-7 relative change of the inputs (C4 T8 seed 23: 1.0e-5;
# C16 T16 seed 11: 5.1e-6)
@pytest.mark.parametrize("C,T,seed", [(4, 8, 23), (16, 16, 11)])
def test_bwd_first_linearisation_encoding_layer_fp32(C, T, seed):
    _say(f"bwd LIN1 encoding layer fp32 B1 H2 T{T} m16 d32 C{C} seed{seed}")
    inp = synth.make_inputs(1, T, 2, 16, 32, seed=seed, in_dtype=synth.F32)
    dy, dso = _upstream(inp, seed)
    _check(inp, _gpu_bwd(inp, dy, dso, C, osr.MODE_ENC, lin=osr.LIN1),
           _oracle(inp, dy, dso, C, osr.MODE_ENC, lin=ob.LIN1))


def test_bwd_first_linearisation_headline_sampled():
    """B4 H8 T2048 m64 d64 C64 with the first linearisation, two sequences
    recomputed by the oracle."""
    _say("bwd LIN1 headline chunked_b4h8_t2048_m64d64_c64, sampled (b,h)")
    inp = synth.workload_inputs("chunked_b4h8_t2048_m64d64_c64")
    dy, dso = _upstream(inp, 24)
    got = _gpu_bwd(inp, dy, dso, 64, osr.MODE_DEC, lin=osr.LIN1)
    bh = [(0, 2), (3, 6)]
    _check(inp, got, _oracle(inp, dy, dso, 64, osr.MODE_DEC, bh, lin=ob.LIN1), bh=bh)


# The slot rows of a sequence split over P workgroups (bf16 inputs, C >= 16,
# decoding and similarity objectives; P = 8, 4, 2 below): each batch's sums
# over slots are exchanged between them and added in workgroup order, so the
# result is one workgroup's up to the order of those sums (fp32 rounding).
SPLIT_CASES = [(1, 2, 128, 128, 64, 256), (4, 8, 64, 64, 64, 256), (2, 3, 32, 64, 16, 128), (1, 3, 64, 128, 32, 128)]


@pytest.mark.parametrize("B,H,m,d,C,T", SPLIT_CASES)
@pytest.mark.parametrize("mode,lin", [(osr.MODE_DEC, osr.LIN2), (osr.MODE_SIM, osr.LIN2), (osr.MODE_DEC, osr.LIN1)])
def test_bwd_split_over_workgroups(B, H, m, d, C, T, mode, lin):
    _say(f"bwd slot rows split over workgroups B{B} H{H} m{m} d{d} C{C} T{T} mode{mode} lin{lin}")
    inp = synth.make_inputs(B, T, H, m, d, seed=2100 + m + d + C + mode, in_dtype=synth.BF16)
    dy, dso = _upstream(inp, 2200 + m + d)
    split = _gpu_bwd(inp, dy, dso, C, mode, lin=lin, bwd_form=osr.BWD_WALK)
    one = _gpu_bwd(inp, dy, dso, C, mode, lin=lin, chain_wgs=osr.WGS_ONE, bwd_form=osr.BWD_WALK)
    for key in split:
        assert _rel(split[key], one[key]) <= 1e-5, key
    _check(inp, split, _oracle(inp, dy, dso, C, mode, lin=ob.LIN1 if lin == osr.LIN1 else ob.LIN2))


def test_bwd_split_deterministic():
    _say("bwd split over workgroups: bit-identical reruns, B1 H4 T512 m=d=128 C64")
    inp = synth.make_inputs(1, 512, 4, 128, 128, seed=2300, in_dtype=synth.BF16)
    dy, dso = _upstream(inp, 2301)
    a = _gpu_bwd(inp, dy, dso, 64, osr.MODE_DEC, bwd_form=osr.BWD_WALK)
    b = _gpu_bwd(inp, dy, dso, 64, osr.MODE_DEC, bwd_form=osr.BWD_WALK)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
