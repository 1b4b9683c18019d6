"""Pins for the fp64 gradient oracle (oracle/osr_backward.py), CPU only.

The gradient oracle differentiates, by torch autograd, a torch transcription
of the forward.  It is pinned to things other than itself:

* its forward agrees with the C oracle (osr_oracle.c, pinned on its own in
  test_oracle_pins.py) to rounding, for every objective, both chunk
  linearisations, both gamma layouts and several chunk sizes;
* every gradient agrees with central finite differences of the C oracle's
  forward along random directions (the definition of a vector-Jacobian
  product; the C oracle shares no code with the torch transcription);
* closed forms: with gamma = 0 nothing is written, so y_t = sum_i q_{t,i} z_i
  with Z the projected initial state, and the gradients follow by hand;
* invariants: the forward does not change when a slot of the initial state
  is rescaled, so the initial-state gradient is orthogonal to every slot;
  slot permutation permutes the gradients;
* planted mistakes in copies of the oracle's source fail the finite-difference
  pin (a stop-gradient on beta, a state gradient not chained across segments,
  the returned state's projection left out of the backward).
"""
import os
import types

import numpy as np
import pytest

import oracle
from oracle import osr_backward as ob
from compressed_memory_linear_amd import synth

DEC, SIM, ENC = oracle.MODE_DEC, oracle.MODE_SIM, oracle.MODE_ENC
LIN2, LIN1 = oracle.LIN2, oracle.LIN1
NAMES = ("q", "k", "v", "gamma", "mu", "state")


def _problem(seed, B=1, T=12, H=2, m=4, d=5, per_slot=True):
    inp = synth.make_inputs(B, T, H, m, d, seed=seed, in_dtype=synth.F32, gamma_per_slot=per_slot)
    return list(inp.values_f64())


def _upstream(args, seed):
    rng = np.random.default_rng(seed + 77)
    return rng.standard_normal(args[2].shape), rng.standard_normal(args[5].shape)


def _loss_c(args, dy, dso, C, mode, lin):
    y, so = oracle.osr_forward(*args, chunk_size=C, mode=mode, linearisation=lin, nthreads=1)
    return float(np.sum(dy * y) + np.sum(dso * so))


def _fd_check(mod, seed, C, mode, lin, per_slot, which=NAMES, eps=1e-6, segment=None):
    """Largest relative gap between <grad, u> and the central difference of
    the C oracle's loss along u, over the inputs in `which`."""
    args = _problem(seed, per_slot=per_slot)
    dy, dso = _upstream(args, seed)
    g = mod.osr_backward(*args, dy, dso, chunk_size=C, mode=mode, linearisation=lin, segment=segment)
    rng = np.random.default_rng(seed + 5)
    worst = 0.0
    for name in which:
        i = NAMES.index(name)
        u = rng.standard_normal(args[i].shape)
        plus = [a.copy() for a in args]
        minus = [a.copy() for a in args]
        plus[i] = plus[i] + eps * u
        minus[i] = minus[i] - eps * u
        fd = (_loss_c(plus, dy, dso, C, mode, lin) - _loss_c(minus, dy, dso, C, mode, lin)) / (2 * eps)
        key = "dstate_in" if name == "state" else "d" + name
        an = float(np.sum(g[key] * u))
        scale = float(np.sum(np.abs(g[key] * u))) + 1e-12
        worst = max(worst, abs(fd - an) / scale)
    return worst


@pytest.mark.parametrize("mode", [DEC, SIM, ENC])
@pytest.mark.parametrize("lin", [LIN2, LIN1])
@pytest.mark.parametrize("C", [1, 2, 4, 12])
@pytest.mark.parametrize("per_slot", [True, False])
def test_torch_forward_matches_c_oracle(mode, lin, C, per_slot):
    args = _problem(3, T=24 if C != 12 else 12, per_slot=per_slot)
    y1, s1 = oracle.osr_forward(*args, chunk_size=C, mode=mode, linearisation=lin)
    y2, s2 = ob.osr_forward_torch(*args, chunk_size=C, mode=mode, linearisation=lin)
    assert np.max(np.abs(y1 - y2)) <= 1e-12 * max(1.0, np.max(np.abs(y1)))
    assert np.max(np.abs(s1 - s2)) <= 1e-12


@pytest.mark.parametrize("mode", [DEC, SIM, ENC])
@pytest.mark.parametrize("C", [1, 4])
@pytest.mark.parametrize("per_slot", [True, False])
@pytest.mark.parametrize("seed", [0, 1])
def test_gradient_matches_finite_differences(mode, C, per_slot, seed):
    # segment = C: the gradient is chained across several segments.
    assert _fd_check(ob, seed, C, mode, LIN2, per_slot, segment=C) <= 1e-6


@pytest.mark.parametrize("mode", [DEC, SIM, ENC])
def test_gradient_first_linearisation_matches_finite_differences(mode):
    assert _fd_check(ob, 2, 4, mode, LIN1, True) <= 1e-6


@pytest.mark.parametrize("mode", [DEC, SIM, ENC])
def test_gradient_whole_chunk_matches_finite_differences(mode):
    # one chunk of the whole sequence: every h, gate and projection frozen at S_0
    assert _fd_check(ob, 4, 12, mode, LIN2, True) <= 1e-6


@pytest.mark.parametrize("mode", [DEC, SIM, ENC])
@pytest.mark.parametrize("C", [1, 4])
def test_no_write_closed_form(mode, C):
    """gamma = 0: S stays at Z = projected S_0 and y_t = sum_i q_{t,i} z_i."""
    args = _problem(6)
    q, k, v, gamma, mu, S0 = args
    gamma = np.zeros_like(gamma)
    dy, dso = _upstream(args, 6)
    g = ob.osr_backward(q, k, v, gamma, mu, S0, dy, dso, chunk_size=C, mode=mode)
    n = np.linalg.norm(S0, axis=-1, keepdims=True)
    Z = S0 / n
    # y[b,t,h,:] = sum_i q[b,t,h,i] Z[b,h,i,:]
    assert np.allclose(g["dq"], np.einsum("bhid,bthd->bthi", Z, dy), rtol=0, atol=1e-12)
    for key in ("dk", "dv", "dmu"):
        assert np.max(np.abs(g[key])) <= 1e-12, key
    G = np.einsum("bthi,bthd->bhid", q, dy) + dso          # dL/dZ
    dS0 = (G - Z * np.sum(Z * G, axis=-1, keepdims=True)) / n
    assert np.allclose(g["dstate_in"], dS0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", [DEC, SIM, ENC])
def test_state_gradient_orthogonal_to_slots(mode):
    """Rescaling a slot of S_0 changes nothing, so dS_0 . s_i = 0 per slot."""
    args = _problem(7)
    args[5] = args[5] * np.random.default_rng(1).uniform(0.5, 2.0, size=args[5].shape[:-1] + (1,))
    dy, dso = _upstream(args, 7)
    g = ob.osr_backward(*args, dy, dso, chunk_size=4, mode=mode)
    dots = np.sum(g["dstate_in"] * args[5], axis=-1)
    assert np.max(np.abs(dots)) <= 1e-12 * np.max(np.abs(g["dstate_in"]))


@pytest.mark.parametrize("mode", [DEC, SIM, ENC])
def test_slot_permutation_permutes_gradients(mode):
    args = _problem(8)
    dy, dso = _upstream(args, 8)
    perm = np.random.default_rng(2).permutation(args[0].shape[-1])
    g = ob.osr_backward(*args, dy, dso, chunk_size=4, mode=mode)
    q, k, v, gamma, mu, S0 = args
    gp = ob.osr_backward(q[..., perm], k[..., perm], v, gamma[..., perm], mu, S0[:, :, perm],
                         dy, dso[:, :, perm], chunk_size=4, mode=mode)
    for key in ("dq", "dk", "dgamma"):
        assert np.allclose(gp[key], g[key][..., perm], rtol=0, atol=1e-12), key
    for key in ("dv", "dmu"):
        assert np.allclose(gp[key], g[key], rtol=0, atol=1e-12), key
    assert np.allclose(gp["dstate_in"], g["dstate_in"][:, :, perm], rtol=0, atol=1e-12)


def test_segments_chain_to_the_same_gradient():
    args = _problem(9, T=24)
    dy, dso = _upstream(args, 9)
    a = ob.osr_backward(*args, dy, dso, chunk_size=4, segment=4)
    b = ob.osr_backward(*args, dy, dso, chunk_size=4, segment=24)
    for key in a:
        assert np.allclose(a[key], b[key], rtol=0, atol=1e-12), key


_MUTANTS = {
    "beta_stop_gradient": ("beta = 1.0 / torch.sqrt(mut * mut + dsq)",
                           "beta = (1.0 / torch.sqrt(mut * mut + dsq)).detach()"),
    "state_gradient_not_chained": ("dS = g[0]\n", "dS = dS\n"),
    "final_projection_skipped": ("(dS,) = torch.autograd.grad(_project(Se), Se, grad_outputs=dSo)",
                                 "dS = dSo"),
    "mu_left_out_of_gate": ("R = (mut * beta + htil * khat)[..., None] * R",
                            "R = (mut.detach() * beta + htil * khat)[..., None] * R"),
}


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_planted_mistake_fails_finite_differences(name):
    src = open(os.path.join(os.path.dirname(ob.__file__), "osr_backward.py")).read()
    old, new = _MUTANTS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("osr_backward_mutant")
    exec(compile(src.replace(old, new), "osr_backward_mutant.py", "exec"), mod.__dict__)
    worst = max(_fd_check(mod, s, 4, DEC, LIN2, True, segment=4) for s in (0, 1))
    assert worst > 1e-3, (name, worst)


# ---------------------------------------------------------------------------
# The chunk-parallel form of the gradient, derived by hand, against autograd.
#
# Per chunk (eq. recurrence_linear2; the chunk-parallel form of "Parallel and
# Hardware Efficient Form"): with Z the projected chunk-start state,
#   H = K Z - V (decoding) or -V (similarity),  Ht = H Z^T,  nh = rowsum(H^2),
#   a = gamma k,  w = nh - Ht^2 (used where > 0),  beta = (mu^2 + a^2 w)^(-1/2),
#   kh = beta a,  G = beta (mu + a Ht),  A_t = prod_{u <= t} G_u (per slot),
#   Y = (Q A) Z - tril((Q A)(kh / A)^T) H,   R_end = diag(A_C) Z - (kh A_C / A)^T H.
# Its vector-Jacobian product is taken matrix by matrix (the products above,
# then the gate cumulative products through the reverse recursion
# E_t = dA_t + G_{t+1} E_{t+1}, dG_t = A_{t-1} E_t, with no division by G),
# and the chunks are chained backwards through the projection of their start
# states.  This is a second, independent evaluation of the gradient (matrix
# products instead of autograd of the token loop); it is also the form a
# chunk-parallel matrix-core backward would compute.

def _chunk_form_grad(q, k, v, g, mu, S0, dy, dso, C, mode):
    """fp64 numpy, one (b,h): q, k, g [T,m]; v, dy [T,d]; mu [T]; S0, dso [m,d]."""
    T, m = q.shape
    d = v.shape[1]
    NC = T // C
    # forward: chunk-start states (before projection)
    starts, S = [], S0.copy()
    for n in range(NC):
        starts.append(S.copy())
        sl = slice(n * C, (n + 1) * C)
        Z = S / np.linalg.norm(S, axis=1, keepdims=True)
        H = k[sl] @ Z - v[sl] if mode == DEC else -v[sl]
        Ht = H @ Z.T
        nh = np.sum(H * H, axis=1)
        a = g[sl] * k[sl]
        w = np.maximum(nh[:, None] - Ht * Ht, 0.0)
        beta = 1.0 / np.sqrt(mu[sl][:, None] ** 2 + a * a * w)
        kh = beta * a
        G = beta * (mu[sl][:, None] + a * Ht)
        A = np.cumprod(G, axis=0)
        S = A[-1][:, None] * Z - (kh * A[-1] / A).T @ H
    # the returned state is the end state projected
    nS = np.linalg.norm(S, axis=1, keepdims=True)
    Zo = S / nS
    dR = (dso - Zo * np.sum(Zo * dso, axis=1, keepdims=True)) / nS
    out = {key: np.zeros_like(x) for key, x in (("dq", q), ("dk", k), ("dv", v), ("dgamma", g), ("dmu", mu))}
    for n in reversed(range(NC)):
        sl = slice(n * C, (n + 1) * C)
        S = starts[n]
        nZ = np.linalg.norm(S, axis=1, keepdims=True)
        Z = S / nZ
        Q, K, V, Gm, Mu, dY = q[sl], k[sl], v[sl], g[sl], mu[sl], dy[sl]
        H = K @ Z - V if mode == DEC else -V
        Ht = H @ Z.T
        nh = np.sum(H * H, axis=1)
        a = Gm * K
        wraw = nh[:, None] - Ht * Ht
        Mk = wraw > 0
        w = np.where(Mk, wraw, 0.0)
        beta = 1.0 / np.sqrt(Mu[:, None] ** 2 + a * a * w)
        kh = beta * a
        G = beta * (Mu[:, None] + a * Ht)
        A = np.cumprod(G, axis=0)
        AC = A[-1]
        QA, KA = Q * A, kh / A
        P = np.tril(QA @ KA.T)
        W = KA * AC
        # read-out
        dZ = QA.T @ dY
        dQA = dY @ Z.T
        dH = -P.T @ dY
        dP = -np.tril(dY @ H.T)
        dQA += dP @ KA
        dKA = dP.T @ QA
        # chunk-end state
        dZ += AC[:, None] * dR
        dAC = np.sum(Z * dR, axis=1)
        dH += -W @ dR
        dW = -H @ dR.T
        dKA += dW * AC
        dAC += np.sum(dW * KA, axis=0)
        # Q A and kh / A
        out["dq"][sl] = dQA * A
        dA = dQA * Q - dKA * KA / A
        dA[-1] += dAC
        dkh = dKA / A
        # cumulative product, reverse recursion
        E = np.zeros_like(dA)
        E[-1] = dA[-1]
        for t in range(C - 2, -1, -1):
            E[t] = dA[t] + G[t + 1] * E[t + 1]
        Aprev = np.vstack([np.ones((1, m)), A[:-1]])
        dG = Aprev * E
        # gates
        dbeta = dG * (Mu[:, None] + a * Ht) + dkh * a
        dHt = dG * kh
        da = dG * beta * Ht + dkh * beta
        dmu = np.sum(dG * beta, axis=1)
        tb = -0.5 * beta ** 3 * dbeta
        dmu += np.sum(2.0 * Mu[:, None] * tb, axis=1)
        da += 2.0 * a * w * tb
        dw = np.where(Mk, a * a * tb, 0.0)
        dnh = np.sum(dw, axis=1)
        dHt += -2.0 * Ht * dw
        out["dgamma"][sl] = da * K
        dK = da * Gm
        dH += dHt @ Z + 2.0 * dnh[:, None] * H
        dZ += dHt.T @ H
        if mode == DEC:
            dK += dH @ Z.T
            dZ += K.T @ dH
        out["dk"][sl] = dK
        out["dv"][sl] = -dH
        out["dmu"][sl] = dmu
        # chunk-start projection
        dR = (dZ - Z * np.sum(Z * dZ, axis=1, keepdims=True)) / nZ
    out["dstate_in"] = dR
    return out


@pytest.mark.parametrize("C,T", [(1, 6), (4, 16), (8, 24), (16, 32)])
@pytest.mark.parametrize("mode", [DEC, SIM])
def test_chunk_parallel_gradient_form(C, T, mode):
    """The hand-derived chunk-parallel gradient equals the autograd gradient of
    the chunk-wise forward to rounding (per-slot gamma, several chunks)."""
    inp = synth.make_inputs(1, T, 2, 6, 5, seed=900 + C + T + mode, in_dtype=synth.F32, gamma_per_slot=True)
    q, k, v, g, mu, S0 = inp.values_f64()
    rng = np.random.default_rng(901 + C)
    dy = rng.standard_normal(v.shape)
    dso = rng.standard_normal(S0.shape)
    ref = ob.osr_backward(q, k, v, g, mu, S0, dy, dso, chunk_size=C, mode=mode)
    for h in range(2):
        got = _chunk_form_grad(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h], mu[0, :, h], S0[0, h],
                               dy[0, :, h], dso[0, h], C, mode)
        for key, ref_key in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dgamma", "dgamma"), ("dmu", "dmu")):
            r = ref[ref_key][0, :, h]
            scale = max(1.0, float(np.max(np.abs(r))))
            assert np.max(np.abs(got[key] - r)) <= 1e-9 * scale, (key, C, mode)
        r = ref["dstate_in"][0, h]
        assert np.max(np.abs(got["dstate_in"] - r)) <= 1e-9 * max(1.0, float(np.max(np.abs(r))))


# The same gradient at the tile level the matrix-core backward computes it:
# 16-token tiles, gate products running from the tile start relative to
# a_ref (their product over the tile's first 8 tokens, which cancels and is
# held constant), the tile-start states R_b, lambda swept over the tiles in
# reverse, and the gate gradients by a forward recursion (W's suffix
# products) and a reverse one (E_t = dA_t + g_{t+1} E_{t+1}).

TILE = 16


def _tile_form_grad(q, k, v, g, mu, S0, dy, dso, C, mode):
    """fp64 numpy, one (b,h): q, k, g [T,m]; v, dy [T,d]; mu [T]; S0, dso [m,d]."""
    T, m = q.shape
    NC, NT = T // C, C // TILE

    def gates(Z, sl):
        H = k[sl] @ Z - v[sl] if mode == DEC else -v[sl]
        Ht = H @ Z.T
        nh = np.sum(H * H, axis=1)
        a = g[sl] * k[sl]
        wraw = nh[:, None] - Ht * Ht
        w = np.where(wraw > 0, wraw, 0.0)
        beta = 1.0 / np.sqrt(mu[sl][:, None] ** 2 + a * a * w)
        return H, Ht, a, wraw > 0, w, beta, beta * a, beta * (mu[sl][:, None] + a * Ht)

    def suffix(Gt):
        return np.vstack([np.cumprod(Gt[::-1], axis=0)[::-1][1:], np.ones((1, Gt.shape[1]))])

    starts, S = [], S0.copy()
    for n in range(NC):
        starts.append(S.copy())
        sl = slice(n * C, (n + 1) * C)
        Z = S / np.linalg.norm(S, axis=1, keepdims=True)
        H, _, _, _, _, _, kap, G = gates(Z, sl)
        R = Z
        for b in range(NT):
            tb = slice(b * TILE, (b + 1) * TILE)
            R = np.prod(G[tb], axis=0)[:, None] * R - (kap[tb] * suffix(G[tb])).T @ H[tb]
        S = R
    nS = np.linalg.norm(S, axis=1, keepdims=True)
    Zo = S / nS
    lam = (dso - Zo * np.sum(Zo * dso, axis=1, keepdims=True)) / nS
    out = {x: np.zeros_like(y) for x, y in (("dq", q), ("dk", k), ("dv", v), ("dgamma", g), ("dmu", mu))}
    for n in reversed(range(NC)):
        sl = slice(n * C, (n + 1) * C)
        nZ = np.linalg.norm(starts[n], axis=1, keepdims=True)
        Z = starts[n] / nZ
        Q, K, Mu, dY = q[sl], k[sl], mu[sl], dy[sl]
        H, Ht, a, Mk, w, beta, kap, G = gates(Z, sl)
        tiles, R = [], Z
        for b in range(NT):
            tb = slice(b * TILE, (b + 1) * TILE)
            A = np.cumprod(G[tb], axis=0)
            ar = A[TILE // 2 - 1]
            tiles.append((tb, A, ar, R, Q[tb] * A / ar, kap[tb] * ar / A, kap[tb] * suffix(G[tb])))
            R = A[-1][:, None] * R - tiles[-1][6].T @ H[tb]
        dG, dkap, dH = np.zeros_like(G), np.zeros_like(kap), np.zeros_like(H)
        for tb, A, ar, Rb, QA, KA, Wt in reversed(tiles):
            Gt = G[tb]
            P = np.tril(QA @ KA.T)
            dP = -np.tril(dY[tb] @ H[tb].T)
            dQA = dY[tb] @ (ar[:, None] * Rb).T + dP @ KA
            dKA = dP.T @ QA
            dH[tb] += -P.T @ dY[tb] - Wt @ lam
            dW = -H[tb] @ lam.T
            dAE = np.sum(Rb * lam, axis=1)
            lam = A[-1][:, None] * lam + ar[:, None] * (QA.T @ dY[tb])
            out["dq"][sl][tb] = dQA * A / ar
            dA = dQA * Q[tb] / ar - dKA * KA / A
            dA[-1] += dAE
            sfx = suffix(Gt)
            dkap[tb] += dKA * ar / A + dW * sfx
            F = np.zeros_like(Gt)           # sum_{s<t} dW_s kappa_s prod_{s<l<t} g_l
            for t in range(1, TILE):
                F[t] = Gt[t - 1] * F[t - 1] + dW[t - 1] * kap[tb][t - 1]
            E = np.zeros_like(Gt)           # E_t = dA_t + g_{t+1} E_{t+1}
            E[-1] = dA[-1]
            for t in range(TILE - 2, -1, -1):
                E[t] = dA[t] + Gt[t + 1] * E[t + 1]
            dG[tb] = F * sfx + np.vstack([np.ones((1, m)), A[:-1]]) * E
        dbeta = dG * (Mu[:, None] + a * Ht) + dkap * a
        dHt = dG * kap
        da = dG * beta * Ht + dkap * beta
        tbeta = -0.5 * beta ** 3 * dbeta
        dmu = np.sum(dG * beta + 2.0 * Mu[:, None] * tbeta, axis=1)
        da += 2.0 * a * w * tbeta
        dw = np.where(Mk, a * a * tbeta, 0.0)
        dHt += -2.0 * Ht * dw
        dH += dHt @ Z + 2.0 * np.sum(dw, axis=1)[:, None] * H
        dZ = lam + dHt.T @ H
        dK = da * g[sl]
        if mode == DEC:
            dK += dH @ Z.T
            dZ += K.T @ dH
        out["dgamma"][sl] = da * K
        out["dk"][sl] = dK
        out["dv"][sl] = -dH
        out["dmu"][sl] = dmu
        lam = (dZ - Z * np.sum(Z * dZ, axis=1, keepdims=True)) / nZ
    out["dstate_in"] = lam
    return out


@pytest.mark.parametrize("C,T", [(16, 48), (32, 64), (64, 128)])
@pytest.mark.parametrize("mode", [DEC, SIM])
@pytest.mark.parametrize("mu_mean", [3.0, -2.0])
def test_tile_level_gradient_form(C, T, mode, mu_mean):
    """The tile-level evaluation (the matrix-core backward's own formulation)
    equals the autograd gradient of the chunk-wise forward to rounding, with
    large and small forget gates (mu = sigmoid(N(3, 1)) and sigmoid(N(-2, 1)))."""
    inp = synth.make_inputs(1, T, 2, 8, 6, seed=950 + C + mode, in_dtype=synth.F32, gamma_per_slot=True,
                            mu_mean=mu_mean)
    q, k, v, g, mu, S0 = inp.values_f64()
    rng = np.random.default_rng(951 + C)
    dy = rng.standard_normal(v.shape)
    dso = rng.standard_normal(S0.shape)
    ref = ob.osr_backward(q, k, v, g, mu, S0, dy, dso, chunk_size=C, mode=mode)
    for h in range(2):
        got = _tile_form_grad(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h], mu[0, :, h], S0[0, h],
                              dy[0, :, h], dso[0, h], C, mode)
        for key in ("dq", "dk", "dv", "dgamma", "dmu"):
            r = ref[key][0, :, h]
            assert np.max(np.abs(got[key] - r)) <= 1e-9 * max(1.0, float(np.max(np.abs(r)))), (key, C, mode)
        r = ref["dstate_in"][0, h]
        assert np.max(np.abs(got["dstate_in"] - r)) <= 1e-9 * max(1.0, float(np.max(np.abs(r))))
