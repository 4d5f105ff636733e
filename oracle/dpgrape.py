"""The DP-GRAPE private update step, written out plainly in float64.

Test infrastructure: a slow, obviously correct reference that the GPU library
is compared against. It never rounds to bf16 and materialises every
per-sample gradient G_i = A_i^T dY_i explicitly.

The step, in the order the pages give it ([GRAPE] Methodology, closing
paragraph: per-sample gradients are projected layer by layer during the
backward pass, then aggregated, clipped and noised, and the privatised
projected gradients drive a projected Adam update of the parameters):

 1. P_l = Z_P / sqrt(r), Z_P a seeded Gaussian [r, d_in] matrix regenerated
    from (seed, layer, proj_step) ([GRAPE] design choice 1).
 2. Ghat_il = P_l (A_il^T dY_il) for every sample i, before any
    privatisation ([GRAPE] design choice 2; per-sample gradients of a batch,
    [GRAPE] Problem statement).
 3. n_i = sqrt(sum_l ||Ghat_il||_F^2); s_i = min(1, C / n_i) ([GRAPE] Problem
    statement: per-sample clipping before noise; the min(C/n, 1) form is the
    one [RC] Algorithmic flow step 4 states).
 4. Gpriv_l = (sum_i s_i Ghat_il + sigma C Z_l) / B, Z_l a seeded Gaussian
    [r, d_out] matrix keyed on (seed, layer, step).
 5. Adam with bias correction on the [r, d_out] projected gradient, moments
    kept in the projected space ([GRAPE] design choice 3).
 6. dW_l = -lr P_l^T U_l; W_l <- W_l + dW_l.

Readings where the pages are silent (each is a choice, listed again in the
design notes):
  R1 W is [d_in, d_out] with y = x W, so the per-sample gradient is A_i^T dY_i
     and P acts on the d_in side.
  R2 P has i.i.d. N(0, 1/r) entries (not orthonormalised), so E[P^T P] = I and
     E||P G||^2 = ||G||^2: the clip threshold keeps its full-space meaning.
  R3 Random streams: Philox4x32-10 + Box-Muller with the counter layout in
     oracle.philox.
  R4 P is keyed on proj_step (the caller passes proj_step = step to draw a
     fresh P every step, as the method's description implies).
  R5 "aggregation, clipping and noise": one global per-sample norm over all
     layers of the call, clip per sample, then batch sum and noise.
  R6 s_i = 1 when n_i <= C (including n_i = 0); C = +inf means no clipping.
  R7 Noise standard deviation sigma*C per entry of the projected space, added
     once to the clipped sum, then everything divided by B (DP-SGD
     convention). With sigma = 0 the noise term is absent (so C = +inf is
     allowed only with sigma = 0).
  R8 Adam (Kingma & Ba) with bias correction at t = step, eps added outside the
     square root, no weight decay; m and v start at zero.
  R9 Back-projection with no extra scale factor.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

from .philox import gaussian_stream

TAG_PROJECTION = 0
TAG_NOISE = 1
TAG_NAIVE_NOISE = 2     # only for the naive privatise-then-project comparator


def projection_matrix(seed: int, layer_id: int, proj_step: int, r: int,
                      d_in: int) -> np.ndarray:
    """P_l[j, k] = z(seed, layer_id, proj_step, tag 0, e = j*d_in + k) / sqrt(r).

    [GRAPE] design choice 1 (Gaussian projection regenerated from a seed);
    scale per reading R2. Pinned by tests/test_oracle_method.py (E[P^T P] = I
    and E||PG||^2 = ||G||^2 over many seeds, [RC] core mechanism)."""
    z = gaussian_stream(seed, layer_id, proj_step, TAG_PROJECTION, r * d_in)
    return z.reshape(r, d_in) / math.sqrt(r)


def noise_matrix(seed: int, layer_id: int, step: int, r: int,
                 d_out: int) -> np.ndarray:
    """Z_l[j, k] = z(seed, layer_id, step, tag 1, e = j*d_out + k)."""
    z = gaussian_stream(seed, layer_id, step, TAG_NOISE, r * d_out)
    return z.reshape(r, d_out)


def per_sample_gradient(A_i: np.ndarray, dY_i: np.ndarray) -> np.ndarray:
    """G_i = A_i^T dY_i, [d_in, d_out] (gradient of y = x W for one sample).

    Materialised explicitly (reading R1)."""
    return np.asarray(A_i, np.float64).T @ np.asarray(dY_i, np.float64)


def _projections(layers, r, seed, proj_step, P_override):
    Ps = []
    for lay in layers:
        lid = int(lay["layer_id"])
        if P_override is not None and lid in P_override:
            Ps.append(np.asarray(P_override[lid], np.float64))
        else:
            Ps.append(projection_matrix(seed, lid, proj_step, r,
                                        lay["A"].shape[2]))
    return Ps


def _projected(P, A, dY, i):
    return P @ per_sample_gradient(A[i], dY[i])


def sample_norms(layers: Sequence[dict], r: int, seed: int, proj_step: int,
                 P_override: Optional[Dict[int, np.ndarray]] = None,
                 samples: Optional[Iterable[int]] = None) -> np.ndarray:
    """n_i = sqrt(sum_l ||P_l A_il^T dY_il||_F^2) for the requested samples.

    [GRAPE] design choice 2 (project the raw per-sample gradients) and reading
    R5 (one norm over all layers)."""
    B = layers[0]["A"].shape[0]
    idx = list(range(B)) if samples is None else list(samples)
    Ps = _projections(layers, r, seed, proj_step, P_override)
    out = np.zeros(len(idx), dtype=np.float64)
    for a, i in enumerate(idx):
        acc = 0.0
        for P, lay in zip(Ps, layers):
            g = _projected(P, lay["A"], lay["dY"], i)
            acc += float(np.sum(g * g))
        out[a] = math.sqrt(acc)
    return out


def clip_scale(norms: np.ndarray, clip_C: float) -> np.ndarray:
    """s_i = 1 if n_i <= C else C / n_i (reading R6)."""
    n = np.asarray(norms, np.float64)
    s = np.ones_like(n)
    over = n > clip_C
    s[over] = clip_C / n[over]
    return s


def project_clip_noise(layers: Sequence[dict], r: int, clip_C: float,
                       sigma: float, seed: int, step: int, proj_step: int,
                       P_override: Optional[Dict[int, np.ndarray]] = None,
                       cache_bytes: int = 1 << 31) -> dict:
    """Steps 1-4: per-sample projection, global clip, batch sum and noise.

    layers: sequence of {"A": [B,T,d_in], "dY": [B,T,d_out], "layer_id": int}
    (float64 arrays holding the exact input values). Returns
    {"norms": n[B], "scales": s[B], "G_priv": [ [r, d_out] per layer ]}.
    Projected per-sample gradients are kept between the norm pass and the sum
    pass when they fit in cache_bytes, else recomputed (same arithmetic)."""
    if not (clip_C > 0):
        raise ValueError("clip_C must be > 0")
    if sigma < 0 or (sigma > 0 and math.isinf(clip_C)):
        raise ValueError("sigma must be >= 0, and 0 when clip_C is infinite")
    B = layers[0]["A"].shape[0]
    Ps = _projections(layers, r, seed, proj_step, P_override)
    total = sum(B * r * lay["dY"].shape[2] * 8 for lay in layers)
    cache = {} if total <= cache_bytes else None

    sq = np.zeros(B, dtype=np.float64)
    for i in range(B):
        for l, (P, lay) in enumerate(zip(Ps, layers)):
            g = _projected(P, lay["A"], lay["dY"], i)
            sq[i] += float(np.sum(g * g))
            if cache is not None:
                cache[(i, l)] = g
    norms = np.sqrt(sq)
    scales = clip_scale(norms, clip_C)

    G_priv = []
    for l, (P, lay) in enumerate(zip(Ps, layers)):
        acc = np.zeros((r, lay["dY"].shape[2]), dtype=np.float64)
        for i in range(B):
            g = cache[(i, l)] if cache is not None else _projected(
                P, lay["A"], lay["dY"], i)
            acc += scales[i] * g
        if sigma > 0:
            Z = noise_matrix(seed, int(lay["layer_id"]), step, r,
                             lay["dY"].shape[2])
            acc += sigma * clip_C * Z
        G_priv.append(acc / B)
    return {"norms": norms, "scales": scales, "G_priv": G_priv}


def adam_update(G: np.ndarray, m: np.ndarray, v: np.ndarray, step: int,
                beta1: float, beta2: float, eps: float):
    """Adam moments and step direction in the projected space (reading R8).

    m' = b1 m + (1-b1) G;  v' = b2 v + (1-b2) G^2;
    U = (m' / (1 - b1^t)) / (sqrt(v' / (1 - b2^t)) + eps).
    [GRAPE] design choice 3: the moments live in [r, d_out]."""
    G = np.asarray(G, np.float64)
    m1 = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * G
    v1 = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * G * G
    mhat = m1 / (1.0 - beta1 ** step)
    vhat = v1 / (1.0 - beta2 ** step)
    U = mhat / (np.sqrt(vhat) + eps)
    return m1, v1, U


def backproject_delta(P: np.ndarray, U: np.ndarray, lr: float) -> np.ndarray:
    """dW = -lr P^T U, [d_in, d_out] ([GRAPE] Methodology closing paragraph:
    the parameters are updated through the projected Adam rule; reading R9)."""
    return -lr * (np.asarray(P, np.float64).T @ np.asarray(U, np.float64))


def adam_backproject(params: Sequence[dict], r: int, lr: float, beta1: float,
                     beta2: float, eps: float, seed: int, step: int,
                     proj_step: int,
                     P_override: Optional[Dict[int, np.ndarray]] = None
                     ) -> List[dict]:
    """Steps 5-6 for every layer.

    params: sequence of {"W": [d_in,d_out], "m": [r,d_out], "v": [r,d_out],
    "G_priv": [r,d_out], "layer_id": int}. Returns per layer
    {"W", "m", "v", "dW", "U"} (new values; inputs are not modified)."""
    if step < 1:
        raise ValueError("step must be >= 1")
    out = []
    for p in params:
        lid = int(p["layer_id"])
        d_in = p["W"].shape[0]
        if P_override is not None and lid in P_override:
            P = np.asarray(P_override[lid], np.float64)
        else:
            P = projection_matrix(seed, lid, proj_step, r, d_in)
        m1, v1, U = adam_update(p["G_priv"], p["m"], p["v"], step,
                                beta1, beta2, eps)
        dW = backproject_delta(P, U, lr)
        out.append({"W": np.asarray(p["W"], np.float64) + dW, "m": m1,
                    "v": v1, "dW": dW, "U": U})
    return out


def projection_rows(seed: int, layer_id: int, proj_step: int, r: int,
                    d_in: int, rows: Sequence[int]) -> np.ndarray:
    """Rows `rows` of P_l (same stream as projection_matrix: row j holds
    elements j*d_in .. j*d_in + d_in - 1)."""
    out = np.empty((len(rows), d_in), dtype=np.float64)
    for a, j in enumerate(rows):
        out[a] = gaussian_stream(seed, layer_id, proj_step, TAG_PROJECTION,
                                 d_in, start=int(j) * d_in)
    return out / math.sqrt(r)


def noise_rows(seed: int, layer_id: int, step: int, r: int, d_out: int,
               rows: Sequence[int]) -> np.ndarray:
    """Rows `rows` of Z_l (same stream as noise_matrix)."""
    out = np.empty((len(rows), d_out), dtype=np.float64)
    for a, j in enumerate(rows):
        out[a] = gaussian_stream(seed, layer_id, step, TAG_NOISE, d_out,
                                 start=int(j) * d_out)
    return out


def g_priv_rows(A: np.ndarray, dY: np.ndarray, P_rows: np.ndarray,
                scales: np.ndarray, clip_C: float, sigma: float,
                Z_rows: Optional[np.ndarray]) -> np.ndarray:
    """Rows of G_priv_l = (sum_i s_i P_l G_il + sigma C Z_l) / B for given
    rows of P_l and Z_l and given clip factors s_i, for inputs too large to
    project whole.

    Row j of P_l G_il is p_j A_i^T dY_i; it is evaluated as (A_i p_j)^T dY_i,
    the same product associated the other way (exact in real arithmetic,
    pinned against project_clip_noise in the tests)."""
    A = np.asarray(A, np.float64)
    dY = np.asarray(dY, np.float64)
    B = A.shape[0]
    acc = np.zeros((P_rows.shape[0], dY.shape[2]), dtype=np.float64)
    for i in range(B):
        x = A[i] @ P_rows.T            # [T, rows]
        acc += scales[i] * (x.T @ dY[i])
    if sigma > 0:
        acc += sigma * clip_C * Z_rows
    return acc / B


def naive_privatise_then_project(layers: Sequence[dict], r: int,
                                 clip_C: float, sigma: float, seed: int,
                                 step: int, proj_step: int) -> List[np.ndarray]:
    """The contrasting order ([GRAPE] design choice 2, "naive" variant):
    clip the full per-sample gradients by their full-space global norm, sum,
    add full-space noise, divide by B, then project with the same P.

    Only used to show that the two orders give different results."""
    B = layers[0]["A"].shape[0]
    full_sq = np.zeros(B)
    for i in range(B):
        for lay in layers:
            g = per_sample_gradient(lay["A"][i], lay["dY"][i])
            full_sq[i] += float(np.sum(g * g))
    s = clip_scale(np.sqrt(full_sq), clip_C)
    out = []
    for lay in layers:
        d_in, d_out = lay["A"].shape[2], lay["dY"].shape[2]
        acc = np.zeros((d_in, d_out))
        for i in range(B):
            acc += s[i] * per_sample_gradient(lay["A"][i], lay["dY"][i])
        if sigma > 0:
            Zf = gaussian_stream(seed, int(lay["layer_id"]), step,
                                 TAG_NAIVE_NOISE, d_in * d_out)
            acc += sigma * clip_C * Zf.reshape(d_in, d_out)
        P = projection_matrix(seed, int(lay["layer_id"]), proj_step, r, d_in)
        out.append(P @ (acc / B))
    return out
