"""Randomized clipping's per-sample norm estimate, written out plainly in
float64 (test infrastructure, like the rest of this package).

Source: [RC] "DP-SGD Eficiente para LLMs con Recorte Aleatorizado",
Methodology: DP-SGD-RC (core mechanism) and Algorithmic flow (steps 3-4).

For one sample of one linear layer, with activations A [T, d_in] and output
gradients G [T, d_out], the squared gradient norm is a trace:

    ||A^T G||_F^2 = tr(G^T A A^T G) = tr(O),   O = G^T A A^T G   [d_out, d_out].

Hutchinson's estimator replaces tr(O) by an average over k probe vectors q_j
with i.i.d. standard normal entries (E[q q^T] = I, so E[q^T O q] = tr(O)):

    tr(O) ~ (1/k) sum_j q_j^T O q_j = (1/k) sum_j ||A^T (G q_j)||^2,

which needs only the products G q_j [T] and A^T (G q_j) [d_in]: O is never
formed. The per-sample estimate adds the layers' estimates; the clip factor
is min(1, C / nhat).

Readings where the page is silent (listed again in the design notes):
  H1 The probes act on O's side, d_out (the page gives P in R^{p x k} with p
     the size of O); the identity tr(G^T A A^T G) = tr(A^T G G^T A) makes
     the d_in side an equal choice.
  H2 The probes are a seeded Philox stream like P and the noise: probe j of
     layer l has entries q_j[c] = z(seed, layer_id, step, tag 3,
     e = j*d_out + c); a fresh draw every step.
  H3 One estimate per sample summed over the layers of the call (as the
     exact norm is, reading R5 of oracle.dpgrape); n_hat = 0 gives s = 1.

Parity pins (tests/test_oracle_randclip.py): the trace identity against the
materialised per-sample gradient; exactness with the k = d_out probes
sqrt(d_out) e_j; unbiasedness over many seeds; the chi-square law of
k nhat^2 / n^2 when O has rank one.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

from .philox import gaussian_stream

TAG_PROBE = 3


def probe_matrix(seed: int, layer_id: int, step: int, k: int, d_out: int) -> np.ndarray:
    """Q_l [k, d_out]: row j is probe q_j, q_j[c] = z(seed, layer_id, step,
    tag 3, e = j*d_out + c) (reading H2)."""
    z = gaussian_stream(seed, layer_id, step, TAG_PROBE, k * d_out)
    return z.reshape(k, d_out)


def trace_of_O(A_i: np.ndarray, G_i: np.ndarray) -> float:
    """tr(G^T A A^T G), forming O explicitly (the identity's right side)."""
    A = np.asarray(A_i, np.float64)
    G = np.asarray(G_i, np.float64)
    O = G.T @ A @ A.T @ G
    return float(np.trace(O))


def hutchinson_layer(A_i: np.ndarray, G_i: np.ndarray, Q: np.ndarray) -> float:
    """(1/k) sum_j ||A^T (G q_j)||^2 for the probes q_j = rows of Q
    ([RC] Methodology, Hutchinson estimator)."""
    A = np.asarray(A_i, np.float64)
    G = np.asarray(G_i, np.float64)
    Q = np.asarray(Q, np.float64)
    k = Q.shape[0]
    total = 0.0
    for j in range(k):
        Gq = G @ Q[j]          # [T]
        v = A.T @ Gq           # [d_in]; q_j^T O q_j = ||v||^2
        total += float(v @ v)
    return total / k


def estimated_norms(layers: Sequence[dict], k: int, seed: int, step: int,
                    Q_override: Optional[Dict[int, np.ndarray]] = None) -> np.ndarray:
    """nhat_i = sqrt(sum_l (1/k) sum_j ||A_il^T dY_il q_lj||^2) for every
    sample i ([RC] Algorithmic flow step 3; readings H1-H3). `layers` holds
    dicts with A [B, T, d_in], dY [B, T, d_out] and layer_id; Q_override maps
    a layer id to explicit probes [k', d_out]."""
    B = layers[0]["A"].shape[0]
    Qs = []
    for lay in layers:
        lid = int(lay["layer_id"])
        if Q_override is not None and lid in Q_override:
            Qs.append(np.asarray(Q_override[lid], np.float64))
        else:
            Qs.append(probe_matrix(seed, lid, step, k, lay["dY"].shape[2]))
    out = np.zeros(B, dtype=np.float64)
    for i in range(B):
        acc = 0.0
        for Q, lay in zip(Qs, layers):
            acc += hutchinson_layer(lay["A"][i], lay["dY"][i], Q)
        out[i] = math.sqrt(acc)
    return out


def rc_clip_factors(nhat: np.ndarray, clip_C: float) -> np.ndarray:
    """s_i = min(1, C / nhat_i), 1 when nhat_i = 0 ([RC] Algorithmic flow
    step 4; reading H3)."""
    n = np.asarray(nhat, np.float64)
    s = np.ones_like(n)
    over = n > clip_C
    s[over] = clip_C / n[over]
    return s
