"""Pins of the layer-glue oracle (oracle/osr_glue.c) to what fixes it from outside.

The glue is the Lattice block's short causal convolution of q and k (width 4),
the sigmoid writing intensity and the GeLU post-gate ("Lattice: Learning to
Efficiently Compress the Memory", section "Experiments", paragraph on the
Lattice block; the experiment-details appendix gives the width 4).  Each pin
checks the oracle against something other than its own formula: library
routines (torch's grouped conv1d and exact gelu, scipy's expit and normal CDF),
delta filters whose output is known, and the split-sequence invariant of a
causal filter with carried history.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle

W = oracle.CONV_WIDTH


def _rng(seed):
    return np.random.default_rng(seed)


def _torch_conv(x, w, b):
    """Depthwise causal convolution through torch's grouped conv1d (fp64)."""
    B, T, N = x.shape
    xt = torch.from_numpy(x).permute(0, 2, 1)  # [B, N, T]
    wt = torch.from_numpy(w).reshape(N, 1, W)
    bt = None if b is None else torch.from_numpy(b)
    out = torch.nn.functional.conv1d(xt, wt, bt, padding=W - 1, groups=N)[..., :T]
    return out.permute(0, 2, 1).numpy()


@pytest.mark.parametrize("B,T,N,bias", [(2, 37, 24, True), (1, 5, 8, False), (3, 1, 16, True), (2, 3, 4, True)])
def test_conv_matches_torch_grouped_conv1d(B, T, N, bias):
    r = _rng(B * 1000 + T * 10 + N)
    x = r.standard_normal((B, T, N))
    w = r.standard_normal((N, W))
    b = r.standard_normal(N) if bias else None
    got = oracle.glue_conv(x, w, b)
    np.testing.assert_allclose(got, _torch_conv(x, w, b), rtol=1e-13, atol=1e-13)


def test_conv_delta_filters():
    r = _rng(1)
    x = r.standard_normal((2, 11, 6))
    w = np.zeros((6, W))
    w[:, W - 1] = 1.0  # the current token only: identity
    np.testing.assert_array_equal(oracle.glue_conv(x, w), x)
    w = np.zeros((6, W))
    w[:, 0] = 1.0  # the token three back: a shift with zeros in front
    shifted = np.zeros_like(x)
    shifted[:, 3:] = x[:, :-3]
    np.testing.assert_array_equal(oracle.glue_conv(x, w), shifted)
    b = r.standard_normal(6)
    np.testing.assert_array_equal(oracle.glue_conv(x, np.zeros((6, W)), b), np.broadcast_to(b, x.shape))


def test_conv_history_reaches_the_first_tokens():
    """The 3 carried tokens stand in front of x: a filter that reads only the oldest
    tap returns the history for t < 3."""
    r = _rng(2)
    x = r.standard_normal((2, 5, 4))
    hist = r.standard_normal((2, W - 1, 4))
    w = np.zeros((4, W))
    w[:, 0] = 1.0
    got = oracle.glue_conv(x, w, None, hist)
    np.testing.assert_array_equal(got[:, :3], hist)
    np.testing.assert_array_equal(got[:, 3:], x[:, :2])


@pytest.mark.parametrize("T1", [0, 1, 2, 3, 7])
def test_conv_split_sequence_equals_one_call(T1):
    r = _rng(3 + T1)
    B, T, N = 2, 12, 8
    x = r.standard_normal((B, T, N))
    w = r.standard_normal((N, W))
    b = r.standard_normal(N)
    whole, hwhole = oracle.glue_conv(x, w, b, return_hist=True)
    first, h1 = oracle.glue_conv(x[:, :T1], w, b, return_hist=True)
    second, h2 = oracle.glue_conv(x[:, T1:], w, b, h1, return_hist=True)
    np.testing.assert_allclose(np.concatenate([first, second], axis=1), whole, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(h2, hwhole)
    np.testing.assert_array_equal(hwhole, x[:, T - 3:])


def test_conv_history_of_short_calls():
    """Fewer than 3 tokens: the history shifts by T and keeps the older rows."""
    r = _rng(4)
    hist = r.standard_normal((1, 3, 5))
    x = r.standard_normal((1, 2, 5))
    _, h = oracle.glue_conv(x, r.standard_normal((5, W)), None, hist, return_hist=True)
    np.testing.assert_array_equal(h[:, 0], hist[:, 2])
    np.testing.assert_array_equal(h[:, 1:], x)
    _, h0 = oracle.glue_conv(np.zeros((1, 0, 5)), r.standard_normal((5, W)), None, hist, return_hist=True)
    np.testing.assert_array_equal(h0, hist)


def test_sigmoid_pins():
    r = _rng(5)
    x = np.concatenate([r.standard_normal(1000) * 4, [0.0, 30.0, -30.0, 700.0, -700.0]])
    got = oracle.glue_sigmoid(x)
    np.testing.assert_allclose(got, scipy.special.expit(x), rtol=1e-14, atol=1e-300)
    assert got[1000] == 0.5
    np.testing.assert_allclose(got[:1000] + oracle.glue_sigmoid(-x[:1000]), 1.0, rtol=0, atol=4.5e-16)
    assert np.all((got > 0) & (got <= 1))


def test_gelu_gate_pins():
    r = _rng(6)
    g = np.concatenate([r.standard_normal(2000) * 3, [0.0, 8.0, -8.0, 40.0, -40.0]])
    y = r.standard_normal(g.size)
    got = oracle.glue_gelu_gate(y, g)
    # GeLU(x) = x Phi(x), Phi the standard normal CDF
    np.testing.assert_allclose(got, y * g * scipy.special.ndtr(g), rtol=1e-13, atol=1e-300)
    # torch evaluates (1 + erf) and so only holds an absolute ~1e-16 in the negative tail
    ref = (torch.from_numpy(y) * torch.nn.functional.gelu(torch.from_numpy(g), approximate="none")).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)
    assert got[2000] == 0.0
    # far out the gate opens fully (GeLU(x) -> x) or shuts (-> 0)
    np.testing.assert_allclose(got[2003], y[2003] * 40.0, rtol=1e-15)
    assert abs(got[2004]) < 1e-300
    # GeLU(x) - GeLU(-x) = x
    np.testing.assert_allclose(oracle.glue_gelu_gate(np.ones(2000), g[:2000]) -
                               oracle.glue_gelu_gate(np.ones(2000), -g[:2000]), g[:2000], rtol=0, atol=1e-14)


def test_glue_pre_shapes_and_parts():
    r = _rng(7)
    B, T, H, m = 2, 9, 3, 4
    xq, xk = r.standard_normal((2, B, T, H, m))
    wq, wk = r.standard_normal((2, H, m, W))
    bq, bk = r.standard_normal((2, H, m))
    logit = r.standard_normal((B, T, H))
    q, k, gamma, hq, hk = oracle.glue_pre(xq, xk, logit, wq, wk, bq, bk)
    assert q.shape == k.shape == (B, T, H, m) and gamma.shape == (B, T, H)
    assert hq.shape == hk.shape == (B, 3, H, m)
    np.testing.assert_allclose(q.reshape(B, T, -1),
                               _torch_conv(xq.reshape(B, T, -1), wq.reshape(-1, W), bq.reshape(-1)), atol=1e-13)
    np.testing.assert_allclose(k.reshape(B, T, -1),
                               _torch_conv(xk.reshape(B, T, -1), wk.reshape(-1, W), bk.reshape(-1)), atol=1e-13)
    np.testing.assert_allclose(gamma, scipy.special.expit(logit), rtol=1e-14)
