"""Pins for the oracle's DP-GRAPE step (CPU only).

Each test ties one part of oracle.dpgrape to something outside it: brute force
on tiny inputs, closed forms, mathematical identities, statistics over many
seeds, and a reduction of the whole step (with an injected identity
projection) to textbook DP-Adam built from torch autograd per-sample
gradients and torch.optim.Adam.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from oracle.dpgrape import clip_scale


def _layers(rng, B, T, shapes, ids=None):
    ids = ids if ids is not None else list(range(len(shapes)))
    return [{"A": rng.standard_normal((B, T, a)),
             "dY": rng.standard_normal((B, T, b)), "layer_id": i}
            for (a, b), i in zip(shapes, ids)]


def _run(layers, r, C=math.inf, sigma=0.0, seed=0, step=1, proj_step=1, **kw):
    return oracle.project_clip_noise(layers, r, C, sigma, seed, step,
                                     proj_step, **kw)


# --- contraction ----------------------------------------------------------

def test_brute_force_tiny_both_associations():
    """Ghat = P (A^T dY) equals (A P^T)^T dY, both written as explicit loops
    over every index ([GRAPE] design choice 2: project the raw per-sample
    gradient; the second association is the one the GPU path uses)."""
    rng = np.random.default_rng(0)
    T, d_in, d_out, r = 3, 4, 5, 2
    lay = _layers(rng, 1, T, [(d_in, d_out)], ids=[9])
    A, dY = lay[0]["A"][0], lay[0]["dY"][0]
    P = oracle.projection_matrix(11, 9, 4, r, d_in)
    want1 = np.zeros((r, d_out))
    for j, n in itertools.product(range(r), range(d_out)):
        s = 0.0
        for k in range(d_in):
            g = 0.0
            for t in range(T):
                g += A[t][k] * dY[t][n]
            s += P[j][k] * g
        want1[j][n] = s
    X = np.zeros((T, r))
    for t, j in itertools.product(range(T), range(r)):
        X[t][j] = sum(A[t][k] * P[j][k] for k in range(d_in))
    want2 = np.zeros((r, d_out))
    for j, n in itertools.product(range(r), range(d_out)):
        want2[j][n] = sum(X[t][j] * dY[t][n] for t in range(T))
    got = _run(lay, r, seed=11, proj_step=4)["G_priv"][0]
    np.testing.assert_allclose(got, want1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got, want2, rtol=1e-12, atol=1e-12)


def test_per_sample_gradient_trace_identity():
    """||A^T G||_F^2 = tr(G^T A A^T G) ([RC] core mechanism), for the
    materialised per-sample gradient, plus an explicit loop check of one
    entry (catches a transposed operand)."""
    rng = np.random.default_rng(1)
    A = rng.standard_normal((7, 5))
    G = rng.standard_normal((7, 3))
    g = oracle.per_sample_gradient(A, G)
    assert g.shape == (5, 3)
    assert math.isclose(float(np.sum(g * g)),
                        float(np.trace(G.T @ A @ A.T @ G)), rel_tol=1e-12)
    assert math.isclose(g[4, 2], sum(A[t, 4] * G[t, 2] for t in range(7)),
                        rel_tol=1e-12)


def test_linearity():
    """Ghat(A, dY1 + dY2) = Ghat(A, dY1) + Ghat(A, dY2); Ghat(aA, dY) = a Ghat."""
    rng = np.random.default_rng(2)
    L1 = _layers(rng, 1, 6, [(12, 9), (9, 4)])
    L2 = [{"A": l["A"], "dY": rng.standard_normal(l["dY"].shape),
           "layer_id": l["layer_id"]} for l in L1]
    Ls = [{"A": a["A"], "dY": a["dY"] + b["dY"], "layer_id": a["layer_id"]}
          for a, b in zip(L1, L2)]
    La = [{"A": -2.5 * a["A"], "dY": a["dY"], "layer_id": a["layer_id"]}
          for a in L1]
    g1, g2, gs, ga = (_run(L, 5)["G_priv"] for L in (L1, L2, Ls, La))
    for l in range(2):
        np.testing.assert_allclose(gs[l], g1[l] + g2[l], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(ga[l], -2.5 * g1[l], rtol=1e-12, atol=1e-12)


def test_closed_form_single_token():
    """B = T = 1: ||P a d^T||_F = ||P a|| ||d||."""
    rng = np.random.default_rng(3)
    lay = _layers(rng, 1, 1, [(10, 6)], ids=[4])
    res = _run(lay, 3, seed=5)
    P = oracle.projection_matrix(5, 4, 1, 3, 10)
    a, d = lay[0]["A"][0, 0], lay[0]["dY"][0, 0]
    want = np.linalg.norm(P @ a) * np.linalg.norm(d)
    assert math.isclose(res["norms"][0], want, rel_tol=1e-12)
    assert math.isclose(np.linalg.norm(res["G_priv"][0]), want, rel_tol=1e-12)


# --- norms and clipping ----------------------------------------------------

def test_norm_is_global_over_layers():
    rng = np.random.default_rng(4)
    lay = _layers(rng, 3, 4, [(8, 5), (5, 7), (6, 2)])
    res = _run(lay, 4)
    per_layer = [np.array([np.linalg.norm(
        oracle.projection_matrix(0, l["layer_id"], 1, 4, l["A"].shape[2])
        @ oracle.per_sample_gradient(l["A"][i], l["dY"][i]))
        for i in range(3)]) for l in lay]
    want = np.sqrt(sum(p ** 2 for p in per_layer))
    np.testing.assert_allclose(res["norms"], want, rtol=1e-12)
    np.testing.assert_allclose(
        oracle.sample_norms(lay, 4, 0, 1, samples=[2]), want[2:], rtol=1e-12)


@pytest.mark.parametrize("C_factor", [0.01, 0.5, 0.999, 1.0, 2.0])
def test_clip_bound(C_factor):
    """With B = 1 and sigma = 0, the output is s * Ghat over all layers, so its
    global norm is min(n, C): equality when clipped, untouched otherwise
    ([GRAPE] Problem statement: per-sample clipping; [RC] flow step 4)."""
    rng = np.random.default_rng(5)
    lay = _layers(rng, 1, 5, [(9, 7), (7, 3)])
    n = _run(lay, 4)["norms"][0]
    C = C_factor * n
    res = _run(lay, 4, C=C)
    tot = math.sqrt(sum(float(np.sum(g * g)) for g in res["G_priv"]))
    assert tot <= C * (1 + 1e-12)
    assert math.isclose(tot, min(n, C), rel_tol=1e-12)


def test_clip_scale_special_cases():
    s = clip_scale(np.array([0.0, 0.5, 1.0, 2.0, 4.0]), 1.0)
    np.testing.assert_array_equal(s, [1.0, 1.0, 1.0, 0.5, 0.25])
    np.testing.assert_array_equal(clip_scale(np.array([0.0, 1e30]), math.inf),
                                  [1.0, 1.0])


def test_batch_mean_of_clipped():
    """Gpriv = mean_i(s_i Ghat_i) when sigma = 0; each sample clipped on its own."""
    rng = np.random.default_rng(6)
    lay = _layers(rng, 4, 3, [(6, 5)])
    lay[0]["A"][2] *= 100.0                       # one loud sample
    full = _run(lay, 3, C=1.0)
    parts = [_run([{"A": lay[0]["A"][i:i + 1], "dY": lay[0]["dY"][i:i + 1],
                    "layer_id": 0}], 3, C=1.0)["G_priv"][0] for i in range(4)]
    np.testing.assert_allclose(full["G_priv"][0], sum(parts) / 4, rtol=1e-12)
    assert full["scales"][2] < 0.05


# --- noise and ordering ------------------------------------------------------

def test_noise_only_in_projected_space():
    """A = 0: Gpriv is the noise alone, sigma C Z / B with Z i.i.d. N(0,1) in
    the [r, d_out] projected space ([GRAPE] design choice 2: noise is added
    in the compressed space). The naive privatise-then-project order instead
    gives P (sigma C Z_full) / B, whose entries have variance d_in / r times
    larger."""
    rng = np.random.default_rng(7)
    B, T, d_in, d_out, r, C, sigma = 4, 2, 400, 300, 8, 0.7, 1.3
    lay = [{"A": np.zeros((B, T, d_in)),
            "dY": rng.standard_normal((B, T, d_out)), "layer_id": 3}]
    g = _run(lay, r, C=C, sigma=sigma, seed=21, step=2)["G_priv"][0]
    z = g * B / (sigma * C)
    assert abs(z.std() - 1.0) < 0.03
    from scipy import stats
    assert stats.kstest(z.ravel(), "norm").pvalue > 1e-4
    naive = oracle.naive_privatise_then_project(lay, r, C, sigma, 21, 2, 1)[0]
    zn = naive * B / (sigma * C)
    assert abs(zn.std() / math.sqrt(d_in / r) - 1.0) < 0.05


def test_order_matters_constructed():
    """Projection before privatisation differs from the naive order on a
    constructed case where ||P G|| and ||G|| differ sharply (r = 1)."""
    rng = np.random.default_rng(8)
    lay = _layers(rng, 3, 4, [(16, 6)])
    ours = _run(lay, 1, C=0.5)["G_priv"][0]
    naive = oracle.naive_privatise_then_project(lay, 1, 0.5, 0.0, 0, 1, 1)[0]
    rel = np.linalg.norm(ours - naive) / np.linalg.norm(naive)
    assert rel > 0.05


def test_noise_key_and_determinism():
    rng = np.random.default_rng(9)
    lay = _layers(rng, 2, 3, [(5, 4)])
    a = _run(lay, 2, C=1.0, sigma=1.0, seed=1, step=3)["G_priv"][0]
    b = _run(lay, 2, C=1.0, sigma=1.0, seed=1, step=3)["G_priv"][0]
    c = _run(lay, 2, C=1.0, sigma=1.0, seed=1, step=4)["G_priv"][0]
    np.testing.assert_array_equal(a, b)
    assert not np.allclose(a, c)


# --- projection statistics ([RC] Hutchinson estimator) ---------------------

def test_projection_is_isotropic_in_expectation():
    """P with N(0, 1/r) entries: E[P^T P] = I and E||P G||^2 = ||G||^2
    (Hutchinson's estimator of the trace identity, [RC] core mechanism)."""
    rng = np.random.default_rng(10)
    d_in, r, S = 12, 6, 3000
    G = rng.standard_normal((d_in, 5))
    acc = np.zeros((d_in, d_in))
    ratios = np.empty(S)
    for s in range(S):
        P = oracle.projection_matrix(s, 0, 1, r, d_in)
        acc += P.T @ P
        ratios[s] = np.sum((P @ G) ** 2) / np.sum(G * G)
    M = acc / S
    assert np.abs(M - np.eye(d_in)).max() < 6 * math.sqrt(2.0 / (r * S))
    assert abs(ratios.mean() - 1.0) < 6 * ratios.std() / math.sqrt(S)


def test_projection_layout_and_keys():
    P = oracle.projection_matrix(3, 2, 5, 4, 7)
    z = oracle.gaussian_stream(3, 2, 5, oracle.TAG_PROJECTION, 28)
    np.testing.assert_array_equal(P, z.reshape(4, 7) / 2.0)
    assert not np.array_equal(P, oracle.projection_matrix(3, 2, 6, 4, 7))
    assert not np.array_equal(P, oracle.projection_matrix(3, 1, 5, 4, 7))
    assert not np.array_equal(P, oracle.projection_matrix(4, 2, 5, 4, 7))


# --- Adam ----------------------------------------------------------------------

def test_adam_first_step_closed_form():
    g = np.array([[1e-3, -2.0, 0.0, 5e-9]])
    m, v, U = oracle.adam_update(g, np.zeros_like(g), np.zeros_like(g), 1,
                                 0.9, 0.999, 1e-8)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v, 0.001 * g * g, rtol=1e-12)
    np.testing.assert_allclose(U, g / (np.abs(g) + 1e-8), rtol=1e-12)


def test_adam_constant_gradient_fixed_point():
    g = np.array([[0.3, -0.02, 4.0]])
    m = np.zeros_like(g)
    v = np.zeros_like(g)
    for t in range(1, 8):
        m, v, U = oracle.adam_update(g, m, v, t, 0.9, 0.999, 1e-8)
        np.testing.assert_allclose(U, g / (np.abs(g) + 1e-8), rtol=1e-12)


def test_backproject_delta_loop():
    rng = np.random.default_rng(11)
    P = rng.standard_normal((3, 4))
    U = rng.standard_normal((3, 5))
    dW = oracle.backproject_delta(P, U, 0.1)
    for i, j in itertools.product(range(4), range(5)):
        want = -0.1 * sum(P[k, i] * U[k, j] for k in range(3))
        assert math.isclose(dW[i, j], want, rel_tol=1e-12, abs_tol=1e-15)


# --- whole step reduces to textbook DP-Adam when P = I ----------------------

def test_identity_projection_reduces_to_dp_adam():
    """With P_l = I (r = d_in), DP-GRAPE is DP-Adam: per-sample gradients
    (torch autograd, vmap of grad), one global per-sample clip over both
    layers, noise, batch mean, and torch.optim.Adam on W. Three steps, so
    the moments carry over."""
    torch = pytest.importorskip("torch")
    from torch.func import grad, vmap

    rng = np.random.default_rng(12)
    B, T, r = 5, 4, 6
    douts = (3, 7)
    C, sigma, lr, b1, b2, eps, seed = 0.8, 0.6, 1e-2, 0.9, 0.999, 1e-8, 17
    Ws = [rng.standard_normal((r, d)) for d in douts]
    ms = [np.zeros((r, d)) for d in douts]
    vs = [np.zeros((r, d)) for d in douts]
    tW = [torch.tensor(W, dtype=torch.float64, requires_grad=True) for W in Ws]
    opt = torch.optim.Adam(tW, lr=lr, betas=(b1, b2), eps=eps)
    I = {0: np.eye(r), 1: np.eye(r)}
    for step in (1, 2, 3):
        A = [rng.standard_normal((B, T, r)) for _ in douts]
        dY = [rng.standard_normal((B, T, d)) for d in douts]
        lay = [{"A": A[l], "dY": dY[l], "layer_id": l} for l in range(2)]
        res = oracle.project_clip_noise(lay, r, C, sigma, seed, step, step,
                                        P_override=I)
        params = [{"W": Ws[l], "m": ms[l], "v": vs[l],
                   "G_priv": res["G_priv"][l], "layer_id": l} for l in range(2)]
        new = oracle.adam_backproject(params, r, lr, b1, b2, eps, seed, step,
                                      step, P_override=I)
        Ws = [n["W"] for n in new]
        ms = [n["m"] for n in new]
        vs = [n["v"] for n in new]

        # textbook DP-Adam
        def loss(W, a, d):
            return torch.sum((a @ W) * d)
        psg = [vmap(grad(loss), in_dims=(None, 0, 0))(
            tW[l].detach(), torch.tensor(A[l]), torch.tensor(dY[l]))
            for l in range(2)]
        norms = torch.sqrt(sum((g.reshape(B, -1) ** 2).sum(1) for g in psg))
        s = torch.clamp(C / norms, max=1.0)
        np.testing.assert_allclose(res["norms"], norms.numpy(), rtol=1e-12)
        opt.zero_grad()
        for l in range(2):
            Z = torch.tensor(oracle.noise_matrix(seed, l, step, r, douts[l]))
            tW[l].grad = ((s[:, None, None] * psg[l]).sum(0)
                          + sigma * C * Z) / B
        opt.step()
        for l in range(2):
            np.testing.assert_allclose(Ws[l], tW[l].detach().numpy(),
                                       rtol=1e-10, atol=1e-12)


# --- row-wise helpers used by the full-size sampled checks ------------------

def test_projection_and_noise_rows_match_full_matrices():
    """projection_rows / noise_rows are rows of projection_matrix /
    noise_matrix (same streams and element numbering)."""
    r, d_in, d_out = 7, 13, 11
    P = oracle.projection_matrix(5, 3, 2, r, d_in)
    Z = oracle.noise_matrix(5, 3, 4, r, d_out)
    rows = [0, 3, 6]
    np.testing.assert_array_equal(oracle.projection_rows(5, 3, 2, r, d_in, rows), P[rows])
    np.testing.assert_array_equal(oracle.noise_rows(5, 3, 4, r, d_out, rows), Z[rows])


@pytest.mark.parametrize("sigma", [0.0, 0.7])
def test_g_priv_rows_match_the_full_step(sigma):
    """g_priv_rows (given the step's clip factors) reproduces rows of the full
    oracle's G_priv, clipped samples and noise included."""
    rng = np.random.default_rng(11)
    B, T, r = 5, 6, 9
    layers = _layers(rng, B, T, [(10, 8), (8, 12)], ids=[4, 7])
    C = float(np.median(oracle.sample_norms(layers, r, 3, 2)))
    full = oracle.project_clip_noise(layers, r, C, sigma, 3, 5, 2)
    assert (full["scales"] < 1).any() and (full["scales"] == 1).any()
    rows = [0, 4, 8]
    for l, lay in enumerate(layers):
        d_in, d_out = lay["A"].shape[2], lay["dY"].shape[2]
        Pr = oracle.projection_rows(3, lay["layer_id"], 2, r, d_in, rows)
        Zr = oracle.noise_rows(3, lay["layer_id"], 5, r, d_out, rows)
        got = oracle.g_priv_rows(lay["A"], lay["dY"], Pr, full["scales"], C,
                                 sigma, Zr)
        np.testing.assert_allclose(got, full["G_priv"][l][rows], rtol=1e-12,
                                   atol=1e-14)
