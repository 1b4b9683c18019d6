"""GPU parity of the layer glue (lattice_osr_glue_pre / lattice_osr_glue_post)
against the fp64 oracle (oracle/osr_glue.c), element by element.

The glue is the Lattice block's short causal convolution of q and k (width 4),
the sigmoid writing intensity and the GeLU post-gate ("Lattice: Learning to
Efficiently Compress the Memory", section "Experiments", paragraph on the
Lattice block).  Bars, from the kernels' fp32 arithmetic on exactly
representable inputs:
  * convolution: four fused multiply-adds onto the bias, each rounding once,
    so |err| <= 8 u S with u = 2^-24 and S = |b| + sum_j |w_j x_j|;
  * sigmoid and the GeLU gate: the device's expf / erfcf (a few ulp) and a
    division or two products: relative 2^-19; the gate's erfc also takes the
    rounded argument -g/sqrt 2, and in the negative tail Phi(g) moves by a
    relative g^2 delta when its argument moves by a relative delta (the Mills
    ratio), so the gate adds 2 g^2 u;
  * a bf16 output adds its rounding: half an ulp, at most 2^-8 of the value.
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_memory_linear_amd import osr, synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _dev(a: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).copy())
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to("cuda")


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def _out_rel(dtype: str) -> float:
    return 2.0 ** -8 if dtype == synth.BF16 else 0.0


def _conv_scale(x, w, b, hist):
    """S = |b| + sum_j |w_j x_{t-3+j}| per output, with the history in front."""
    B, T = x.shape[:2]
    xe = np.concatenate([hist if hist is not None else np.zeros((B, 3) + x.shape[2:]), x], axis=1)
    S = np.abs(b)[None, None] if b is not None else np.zeros(x.shape[2:])[None, None]
    S = S + sum(np.abs(w[..., j])[None, None] * np.abs(xe[:, j:j + T]) for j in range(4))
    return S


def _check(got, ref, bound, what):
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {err.size} beyond the bar; worst at {i}: "
                             f"got {got[i]!r}, oracle {ref[i]!r}, bar {bound[i]!r}")


def _run_pre(inp, with_bias=True, with_hist=True, return_history=True):
    args = [_dev(inp.xq), _dev(inp.xk), _dev(inp.logit), _dev(inp.wq), _dev(inp.wk)]
    args += [_dev(inp.bq), _dev(inp.bk)] if with_bias else [None, None]
    args += [_dev(inp.hist_q), _dev(inp.hist_k)] if with_hist else [None, None]
    out = osr.lattice_osr_glue_pre(*args, return_history=return_history)
    torch.cuda.synchronize()
    return out


def _check_pre(inp, out, with_bias=True, with_hist=True):
    v = inp.value
    bq, bk = (v("bq"), v("bk")) if with_bias else (None, None)
    hq, hk = (v("hist_q"), v("hist_k")) if with_hist else (None, None)
    ref = oracle.glue_pre(v("xq"), v("xk"), v("logit"), v("wq"), v("wk"), bq, bk, hq, hk)
    rel = _out_rel(inp.in_dtype)
    for name, got, want, x, w, b, h in (("q", out[0], ref[0], v("xq"), v("wq"), bq, hq),
                                        ("k", out[1], ref[1], v("xk"), v("wk"), bk, hk)):
        bound = rel * np.abs(want) + (16 if rel else 8) * U * _conv_scale(x, w, b, h) + 1e-30
        _check(_f64(got), want, bound, name)
    _check(_f64(out[2]), ref[2], (rel + 2.0 ** -19) * np.abs(ref[2]) + 1e-30, "gamma")
    if len(out) == 5:
        # the history is raw input rows: bit-exact
        np.testing.assert_array_equal(_f64(out[3]), ref[3])
        np.testing.assert_array_equal(_f64(out[4]), ref[4])


@pytest.mark.parametrize("B,T,H,m,in_dtype,per_slot", [
    (2, 77, 3, 16, synth.BF16, True),    # a 64-token tile and a ragged tail of 13
    (1, 203, 2, 16, synth.BF16, True),   # three 64-token tiles and a ragged tail of 11
    (1, 64, 2, 32, synth.F32, True),
    (2, 45, 3, 16, synth.BF16, False),   # per-token gamma, H not a multiple of 8
    (1, 33, 16, 64, synth.F32, False),   # per-token gamma, rows of 16
    (1, 128, 1, 128, synth.BF16, True),
])
def test_glue_pre_matches_oracle(B, T, H, m, in_dtype, per_slot):
    inp = synth.make_glue_inputs(B, T, H, m, 16, seed=500 + T, in_dtype=in_dtype, gamma_per_slot=per_slot)
    print(f"glue_pre B{B} T{T} H{H} m{m} {in_dtype} per_slot={per_slot}", flush=True)
    _check_pre(inp, _run_pre(inp))


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_glue_pre_short_sequences_and_history(T):
    """Fewer tokens than the filter: the output and the next history both draw on the
    carried rows."""
    inp = synth.make_glue_inputs(2, T, 2, 16, 16, seed=600 + T)
    _check_pre(inp, _run_pre(inp))


def test_glue_pre_without_bias_or_history():
    inp = synth.make_glue_inputs(1, 40, 2, 32, 16, seed=700)
    out = _run_pre(inp, with_bias=False, with_hist=False, return_history=False)
    assert len(out) == 3
    _check_pre(inp, out, with_bias=False, with_hist=False)


def test_glue_pre_split_sequence_equals_one_call():
    """Two calls chained through the history give the single call's outputs bit for bit
    (the same fp32 operations on the same values)."""
    inp = synth.make_glue_inputs(2, 70, 2, 16, 16, seed=800)
    whole = _run_pre(inp)
    xq, xk, lg = _dev(inp.xq), _dev(inp.xk), _dev(inp.logit)
    w = [_dev(inp.wq), _dev(inp.wk), _dev(inp.bq), _dev(inp.bk)]
    cut = 37
    a = osr.lattice_osr_glue_pre(xq[:, :cut].contiguous(), xk[:, :cut].contiguous(), lg[:, :cut].contiguous(), *w,
                                 _dev(inp.hist_q), _dev(inp.hist_k), return_history=True)
    b = osr.lattice_osr_glue_pre(xq[:, cut:].contiguous(), xk[:, cut:].contiguous(), lg[:, cut:].contiguous(), *w,
                                 a[3], a[4], return_history=True)
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(torch.cat([a[i], b[i]], dim=1), whole[i]), i
    assert torch.equal(b[3], whole[3]) and torch.equal(b[4], whole[4])


def test_glue_pre_headline_size():
    """The layer of the chunked workload B4 H8 T2048 m64 (bf16), every element."""
    inp = synth.make_glue_inputs(4, 2048, 8, 64, 64, seed=900)
    _check_pre(inp, _run_pre(inp))


def _gate_rel(g):
    return 2.0 ** -19 + 2 * g * g * U


def _check_post(inp, got):
    g = inp.value("gate")
    ref = oracle.glue_gelu_gate(inp.value("y"), g)
    rel = _out_rel(inp.y_dtype)
    _check(_f64(got), ref, (rel + _gate_rel(g)) * np.abs(ref) + 1e-30, "out")


@pytest.mark.parametrize("in_dtype,y_dtype", [(synth.BF16, synth.F32), (synth.BF16, synth.BF16),
                                              (synth.F32, synth.F32), (synth.F32, synth.BF16)])
def test_glue_post_matches_oracle(in_dtype, y_dtype):
    inp = synth.make_glue_inputs(2, 53, 3, 16, 32, seed=1000, in_dtype=in_dtype, y_dtype=y_dtype)
    print(f"glue_post {in_dtype} gate, {y_dtype} y", flush=True)
    out = osr.lattice_osr_glue_post(_dev(inp.y), _dev(inp.gate))
    torch.cuda.synchronize()
    _check_post(inp, out)


def test_glue_post_in_place_and_headline_size():
    inp = synth.make_glue_inputs(4, 2048, 8, 16, 64, seed=1100)
    y = _dev(inp.y)
    out = osr.lattice_osr_glue_post(y, _dev(inp.gate), out=y)
    torch.cuda.synchronize()
    assert out.data_ptr() == y.data_ptr()
    _check_post(inp, out)


def test_glue_post_tails_of_the_gate():
    """Far out the gate passes y (GeLU(x) ~ x) or shuts it; the erfc form keeps the
    negative tail's relative accuracy."""
    g = torch.tensor([0.0, 1e-3, -1e-3, 5.0, -5.0, 9.0, -9.0, 12.0, -12.0, 30.0, -30.0, 2.0, -2.0, 0.5, -0.5, 40.0],
                     dtype=torch.float32)
    y = torch.linspace(-1.5, 2.0, g.numel(), dtype=torch.float32)
    out = osr.lattice_osr_glue_post(y.reshape(1, 1, 1, 16).cuda(), g.reshape(1, 1, 1, 16).cuda())
    torch.cuda.synchronize()
    ref = oracle.glue_gelu_gate(y.double().numpy(), g.double().numpy())
    got = out.reshape(-1).cpu().double().numpy()
    _check(got, ref, _gate_rel(g.double().numpy()) * np.abs(ref) + 1e-38, "tails")


@pytest.mark.parametrize("C", [4, 16])
def test_layer_pipeline_glue_forward_glue(C):
    """glue_pre -> lattice_osr_fwd_chunked -> glue_post, every call through the C ABI with one
    descriptor's layouts.  The forward is checked against the oracle run on the glue's own bf16
    outputs (q, k, gamma as the GPU produced them, which the tests above pin to the glue oracle), at
    the bf16 forward bar (max error 2e-2 of the oracle's RMS); the post-gate against the oracle's
    gate of the GPU's y, at the gate's bar.  C = 4 runs the token loop, C = 16 the matrix-core path."""
    B, T, H, m, d = 2, 64, 2, 16, 32
    g = synth.make_glue_inputs(B, T, H, m, d, seed=1200 + C)
    base = synth.make_inputs(B, T, H, m, d, seed=1300 + C)
    print(f"layer pipeline C={C}", flush=True)
    q, k, gamma = osr.lattice_osr_glue_pre(_dev(g.xq), _dev(g.xk), _dev(g.logit), _dev(g.wq), _dev(g.wk),
                                           _dev(g.bq), _dev(g.bk))
    t = osr.to_device(base)
    y, S = osr.lattice_osr_fwd_chunked(q, k, t["v"], gamma, t["mu"], t["state"], C)
    out = osr.lattice_osr_glue_post(y, _dev(g.gate))
    torch.cuda.synchronize()

    qv, kv, gv = _f64(q), _f64(k), _f64(gamma)
    v64, mu64, s64 = (base.value(n).astype(np.float64) for n in ("v", "mu", "state"))
    yr, Sr = oracle.osr_forward(qv, kv, v64, gv, mu64, s64, chunk_size=C)
    yg, Sg = _f64(y), S.cpu().numpy().astype(np.float64)
    for got, ref, what in ((yg, yr, "y"), (Sg, Sr, "state")):
        err = np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2))
        print(f"  {what} err/rms {err:.3e}", flush=True)
        assert np.isfinite(got).all() and err <= 2e-2, (what, err)
    gate = g.value("gate")
    ref = oracle.glue_gelu_gate(yg, gate)
    _check(_f64(out), ref, _gate_rel(gate) * np.abs(ref) + 1e-30, "out")


# ------------------------------------------- post-gate fused into the forward --
# lattice_osr_fwd_chunked_gated: y = OSR(...) * GeLU(gate) written once.  With
# fp32 y it is bit for bit the unfused forward followed by glue_post (the same
# fp32 product, rounded once); against the oracle (the fp64 forward, then the
# fp64 gate) the stated forward bar applies to the gated output relative to its
# RMS: 2e-2 for bf16 inputs, 1e-4 for fp32 (here the gate is N(0, 2^2), and
# the forward's error relative to y's RMS is 1e-4 - 1e-6 on these paths, far
# below the bars after the gate's scaling).
GATED = [("split", synth.BF16, 64, osr.SCHED_SPLIT, 2, 256, 2, 64, 128),
         ("fused", synth.BF16, 32, osr.SCHED_FUSED, 2, 256, 2, 64, 128),
         ("split-wgs", synth.BF16, 128, osr.SCHED_AUTO, 1, 512, 4, 128, 128),
         # 64 chunks: the read-out overlapped by chunk ranges (one and four workgroups per sequence)
         ("overlap", synth.BF16, 32, osr.SCHED_AUTO, 1, 2048, 2, 64, 64),
         ("overlap-wgs", synth.BF16, 128, osr.SCHED_AUTO, 1, 8192, 2, 128, 128),
         ("tokenloop-bf16", synth.BF16, 4, osr.SCHED_AUTO, 2, 64, 2, 32, 64),
         ("tokenloop-f32", synth.F32, 4, osr.SCHED_AUTO, 2, 64, 2, 32, 64)]


@pytest.mark.parametrize("case", GATED, ids=[c[0] for c in GATED])
@pytest.mark.parametrize("mode", [osr.MODE_DEC, osr.MODE_SIM])
def test_forward_with_fused_post_gate(case, mode):
    name, dt, C, sched, B, T, H, m, d = case
    print(f"[case] gated forward {name} B{B} T{T} H{H} m{m} d{d} C{C} mode{mode}", flush=True)
    inp = synth.make_inputs(B, T, H, m, d, seed=3100 + C + m + mode, in_dtype=dt)
    g32 = np.random.default_rng(31).standard_normal((B, T, H, d)).astype(np.float32) * np.float32(2)
    gate_store = synth.bf16_round_bits(g32) if dt == synth.BF16 else g32
    gate_vals = synth.bf16_bits_to_f32(gate_store) if dt == synth.BF16 else g32
    t = osr.to_device(inp)
    gate = _dev(gate_store)
    args = (t["q"], t["k"], t["v"], t["gamma"], t["mu"])
    yg, Sg = osr.lattice_osr_fwd_chunked_gated(*args, gate, t["state"], C, mode=mode, schedule=sched)
    y, S = osr.lattice_osr_fwd_chunked(*args, t["state"], C, mode=mode, schedule=sched)
    post = osr.lattice_osr_glue_post(y, gate)
    torch.cuda.synchronize()
    assert torch.equal(yg, post), "fused gate differs from forward + glue_post"
    assert torch.equal(Sg, S)
    yr, _ = oracle.osr_forward(*inp.values_f64(), chunk_size=C, mode=mode)
    ref = oracle.glue_gelu_gate(yr, gate_vals.astype(np.float64))
    got = _f64(yg)
    e = float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2)))
    tol = 2e-2 if dt == synth.BF16 else 1e-4
    print(f"[case]   gated y err/rms {e:.3e} (tol {tol:g})", flush=True)
    assert e <= tol


def test_forward_with_fused_post_gate_bf16_output():
    """bf16 y: the fused product rounded once to bf16 (round to nearest even)."""
    print("[case] gated forward, bf16 y, split schedule", flush=True)
    inp = synth.make_inputs(2, 256, 2, 64, 128, seed=3200, in_dtype=synth.BF16)
    g = synth.bf16_round_bits(np.random.default_rng(32).standard_normal((2, 256, 2, 128)).astype(np.float32))
    t = osr.to_device(inp)
    gate = _dev(g)
    args = (t["q"], t["k"], t["v"], t["gamma"], t["mu"], gate, t["state"])
    y16, _ = osr.lattice_osr_fwd_chunked_gated(*args, 64, y_dtype=torch.bfloat16)
    y32, _ = osr.lattice_osr_fwd_chunked_gated(*args, 64)
    torch.cuda.synchronize()
    rounded = synth.bf16_bits_to_f32(synth.bf16_round_bits(y32.cpu().numpy()))
    assert np.array_equal(rounded, y16.float().cpu().numpy())
