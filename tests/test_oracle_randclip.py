"""Pins for the oracle's randomized-clipping norm estimate (CPU only).

Each test ties oracle.randclip to something outside it: the per-sample
gradient materialised and its Frobenius norm, the trace identity written as
explicit loops, an exact special case (probes sqrt(d_out) e_j), Hutchinson's
unbiasedness over many seeds, and the exact chi-square law of the estimate
when O has rank one. Source: [RC] "DP-SGD Eficiente para LLMs con Recorte
Aleatorizado", Methodology: DP-SGD-RC (trace identity, Hutchinson estimator)
and Algorithmic flow steps 3-4.
"""
import itertools
import math

import numpy as np
import pytest
from scipy import stats

from oracle import randclip
from oracle.dpgrape import per_sample_gradient


def _layers(rng, B, T, shapes, ids=None):
    ids = ids if ids is not None else list(range(len(shapes)))
    return [{"A": rng.standard_normal((B, T, a)),
             "dY": rng.standard_normal((B, T, b)), "layer_id": i}
            for (a, b), i in zip(shapes, ids)]


def test_trace_identity_by_loops():
    """||A^T G||_F^2 = tr(G^T A A^T G): the left side from the materialised
    per-sample gradient, the right side as explicit index loops."""
    rng = np.random.default_rng(1)
    T, d_in, d_out = 3, 4, 5
    A = rng.standard_normal((T, d_in))
    G = rng.standard_normal((T, d_out))
    lhs = float(np.sum(per_sample_gradient(A, G) ** 2))
    rhs = 0.0
    for c in range(d_out):            # O[c][c] = sum_t,s G[t][c] (A A^T)[t][s] G[s][c]
        for t, s in itertools.product(range(T), range(T)):
            aat = sum(A[t][k] * A[s][k] for k in range(d_in))
            rhs += G[t][c] * aat * G[s][c]
    assert lhs == pytest.approx(rhs, rel=1e-12)
    assert randclip.trace_of_O(A, G) == pytest.approx(lhs, rel=1e-12)


def test_exact_with_scaled_unit_probes():
    """With the k = d_out probes sqrt(d_out) e_j, (1/k) sum_j q_j^T O q_j is
    exactly tr(O): the estimate equals the exact norm over several layers."""
    rng = np.random.default_rng(2)
    B, T = 3, 4
    layers = _layers(rng, B, T, [(5, 6), (7, 3)], ids=[4, 9])
    Q = {lay["layer_id"]: math.sqrt(lay["dY"].shape[2]) * np.eye(lay["dY"].shape[2])
         for lay in layers}
    got = randclip.estimated_norms(layers, k=0, seed=0, step=1, Q_override=Q)
    for i in range(B):
        want = math.sqrt(sum(float(np.sum(per_sample_gradient(l["A"][i], l["dY"][i]) ** 2))
                             for l in layers))
        assert got[i] == pytest.approx(want, rel=1e-12)


def test_layer_estimate_by_loops():
    """hutchinson_layer against explicit loops over j, t, c and k."""
    rng = np.random.default_rng(3)
    T, d_in, d_out, k = 3, 2, 4, 3
    A = rng.standard_normal((T, d_in))
    G = rng.standard_normal((T, d_out))
    Q = rng.standard_normal((k, d_out))
    want = 0.0
    for j in range(k):
        for a in range(d_in):
            v = 0.0
            for t in range(T):
                gq = sum(G[t][c] * Q[j][c] for c in range(d_out))
                v += A[t][a] * gq
            want += v * v
    want /= k
    assert randclip.hutchinson_layer(A, G, Q) == pytest.approx(want, rel=1e-12)


def test_unbiased_over_seeds():
    """E[nhat^2] = n^2 (Hutchinson; E[q q^T] = I for the seeded Philox
    probes): the mean of nhat^2 / n^2 over 300 seeds is 1 within five
    standard errors, the standard error taken from the sample itself."""
    rng = np.random.default_rng(4)
    layers = _layers(rng, 2, 6, [(5, 7), (4, 3)], ids=[1, 2])
    n2 = np.array([sum(float(np.sum(per_sample_gradient(l["A"][i], l["dY"][i]) ** 2))
                       for l in layers) for i in range(2)])
    k = 4
    ratios = np.array([randclip.estimated_norms(layers, k, seed, step=3) ** 2 / n2
                       for seed in range(300)])
    mean = ratios.mean(axis=0)
    se = ratios.std(axis=0, ddof=1) / math.sqrt(ratios.shape[0])
    assert np.all(np.abs(mean - 1.0) < 5 * se)
    # and the spread is Hutchinson's: Var[nhat^2] = (2/k) ||O||_F^2 summed over layers
    var_want = []
    for i in range(2):
        v = 0.0
        for l in layers:
            A, G = l["A"][i], l["dY"][i]
            O = G.T @ A @ A.T @ G
            v += 2.0 / k * float(np.sum(O * O))
        var_want.append(v / n2[i] ** 2)
    assert np.allclose(ratios.var(axis=0, ddof=1), var_want, rtol=0.35)


def test_chi_square_law_rank_one():
    """T = 1 makes O = g g^T ||a||^2 rank one, so k nhat^2 / n^2 =
    sum_j (q_j . g / |g|)^2 is exactly chi-square with k degrees of freedom:
    a Kolmogorov-Smirnov test over 400 seeds (a wrong 1/k, a wrong probe
    variance or correlated probes all fail it)."""
    rng = np.random.default_rng(5)
    k = 6
    layers = _layers(rng, 1, 1, [(5, 9)], ids=[7])
    n2 = float(np.sum(per_sample_gradient(layers[0]["A"][0], layers[0]["dY"][0]) ** 2))
    x = np.array([k * randclip.estimated_norms(layers, k, seed, step=2)[0] ** 2 / n2
                  for seed in range(400)])
    assert stats.kstest(x, stats.chi2(k).cdf).pvalue > 1e-3


def test_probe_stream_keys():
    """Probes are keyed on (seed, layer, step) with tag 3: a different key
    draws different probes, the same key the same ones, and they are not the
    projection's tag-0 normals."""
    base = randclip.probe_matrix(5, 3, 7, 4, 6)
    assert base.shape == (4, 6)
    np.testing.assert_array_equal(base, randclip.probe_matrix(5, 3, 7, 4, 6))
    for other in (randclip.probe_matrix(6, 3, 7, 4, 6), randclip.probe_matrix(5, 4, 7, 4, 6),
                  randclip.probe_matrix(5, 3, 8, 4, 6)):
        assert not np.allclose(base, other)
    from oracle.philox import gaussian_stream
    assert not np.allclose(base.reshape(-1), gaussian_stream(5, 3, 7, 0, 24))


def test_clip_factors():
    """s = min(1, C / nhat), 1 at nhat = 0 ([RC] Algorithmic flow step 4)."""
    s = randclip.rc_clip_factors(np.array([0.0, 0.5, 1.0, 4.0]), 1.0)
    np.testing.assert_array_equal(s, [1.0, 1.0, 1.0, 0.25])
