"""GPU parity of the streaming form (dpg_project_layer + dpg_clip_sum_noise,
and the autograd driver in dp_grape_projection_amd.streaming) against the
float64 oracle.

  * every layer's stored projections G_hat[i] = P A_i^T dY_i against the
    oracle's P_l (A_il^T dY_il), and the accumulated squared norms against
    the oracle's n_i^2;
  * G_priv from the stored projections (sigma = 0 and the workload's sigma)
    against oracle.project_clip_noise, and against the one-call form on the
    same inputs;
  * a two-layer network trained for two steps through GrapeOptimizer: the
    inputs the layers saw during backward are kept, and each step's G_priv,
    norms and update are checked against the oracle on those inputs.
Bars as in the other parity tests: fp32 1e-5, bf16 2e-2 (relative Frobenius).
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from _helpers import TOL, make_case, rel_err, rel_err_dw, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_and_library():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dp_grape_projection_amd as dpg
    dpg.load_library()     # fails loudly when libdpg.so is missing


CASES = {
    "tiny": W.workload("tiny"),
    "ragged_bf16": W.custom_workload("s_ragged_bf16", 31,
                                     [(200, 136), (136, 300), (72, 40)],
                                     B=3, T=40, r=40, layer_ids=[5, 17, 2]),
    "odd_fp32": W.custom_workload("s_odd_fp32", 32, [(37, 29), (29, 53)],
                                  B=2, T=13, r=7, dtype="fp32"),
    "full_bf16": W.custom_workload("s_full_bf16", 33, [(256, 256), (384, 128)],
                                   B=2, T=128, r=128),
    "long_t_bf16": W.custom_workload("s_long_t_bf16", 34, [(64, 96)], B=2,
                                     T=300, r=160),
    # r and B*T whole 256 x 256 tiles, d_in whole K steps: the per-layer
    # projection takes the large-tile kernel, the update the large-tile
    # back-projection
    "big_tiles_bf16": W.custom_workload("s_big_tiles_bf16", 35,
                                        [(256, 512), (512, 256)], B=2, T=256, r=256),
    # one layer with fewer 256 x 256 projection tiles (64) than CUs but as
    # many 128 x 128 ones (256): the plan gives the per-layer projection the
    # regular tiles instead of splitting d_in
    "regular_tiles_bf16": W.custom_workload("s_regular_tiles_bf16", 36, [(256, 320)],
                                            B=16, T=512, r=512),
}


def _stream(wl, host, sigma, C=None):
    import torch
    import dp_grape_projection_amd as dpg
    C = wl.clip_C if C is None else C
    norm_sq = torch.zeros(wl.B, dtype=torch.float32, device="cuda")
    G_hat = []
    for (a, d), L in zip(host, wl.layers):
        G_hat.append(dpg.dpg_project_layer(to_device(wl, a), to_device(wl, d), wl.r,
                                           wl.seed, wl.proj_step, L.layer_id, norm_sq))
    G_priv, n = dpg.dpg_clip_sum_noise(G_hat, wl.r, C, sigma, wl.seed, wl.step,
                                       norm_sq, layer_ids=[L.layer_id for L in wl.layers])
    torch.cuda.synchronize()
    return ([g.cpu().numpy() for g in G_hat], norm_sq.cpu().numpy(),
            [g.cpu().numpy() for g in G_priv], n.cpu().numpy())


@pytest.mark.parametrize("name", list(CASES))
def test_streaming_parity(name):
    import dp_grape_projection_amd as dpg
    wl = CASES[name]
    print(f"[stream] {name}: {len(wl.layers)} layers B={wl.B} T={wl.T} r={wl.r} "
          f"{wl.dtype}", flush=True)
    host, orc, _ = make_case(wl)
    tol = TOL[wl.dtype]
    Gh, nsq, G0, n = _stream(wl, host, 0.0)
    # stored projections, layer by layer
    worst = 0.0
    for g, lay in zip(Gh, orc):
        P = oracle.projection_matrix(wl.seed, lay["layer_id"], wl.proj_step, wl.r,
                                     lay["A"].shape[2])
        want = np.stack([P @ oracle.per_sample_gradient(lay["A"][i], lay["dY"][i])
                         for i in range(wl.B)])
        worst = max(worst, rel_err(g, want))
    want = oracle.project_clip_noise(orc, wl.r, wl.clip_C, 0.0, wl.seed, wl.step,
                                     wl.proj_step)
    e_sq = rel_err(nsq, want["norms"] ** 2)
    e_n = rel_err(n, want["norms"])
    e_g0 = max(rel_err(g, w) for g, w in zip(G0, want["G_priv"]))
    _, _, G1, _ = _stream(wl, host, wl.sigma)
    want1 = oracle.project_clip_noise(orc, wl.r, wl.clip_C, wl.sigma, wl.seed,
                                      wl.step, wl.proj_step)
    e_g1 = max(rel_err(g, w) for g, w in zip(G1, want1["G_priv"]))
    print(f"[stream] {name}: G_hat {worst:.2e} norm_sq {e_sq:.2e} norms {e_n:.2e} "
          f"G_priv sigma=0 {e_g0:.2e} sigma={wl.sigma} {e_g1:.2e}", flush=True)
    assert max(worst, e_sq, e_n, e_g0, e_g1) <= tol
    # the one-call form on the same inputs
    A = [to_device(wl, a) for a, _ in host]
    dY = [to_device(wl, d) for _, d in host]
    Gf, nf = dpg.dpg_project_clip_noise(A, dY, wl.r, wl.clip_C, 0.0, wl.seed, wl.step,
                                        wl.proj_step,
                                        layer_ids=[L.layer_id for L in wl.layers])
    e_f = max(rel_err(g, f.cpu().numpy()) for g, f in zip(G0, Gf))
    assert e_f <= tol and rel_err(n, nf.cpu().numpy()) <= tol


def test_streaming_mixed_clipping_and_no_clipping():
    wl = CASES["ragged_bf16"]
    host, orc, _ = make_case(wl)
    n_all = oracle.project_clip_noise(orc, wl.r, math.inf, 0.0, wl.seed, wl.step,
                                      wl.proj_step)["norms"]
    C = float(np.median(n_all))
    for c in (C, math.inf):
        _, _, G, n = _stream(wl, host, 0.0, C=c)
        want = oracle.project_clip_noise(orc, wl.r, c, 0.0, wl.seed, wl.step,
                                         wl.proj_step)
        assert max(rel_err(g, w) for g, w in zip(G, want["G_priv"])) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_autograd_driver_two_steps(dtype):
    """Two steps of a small network (ProjectedLinear -> tanh ->
    ProjectedLinear) through GrapeOptimizer; each step is checked against the
    oracle on the inputs and output gradients the layers actually saw."""
    import torch
    import dp_grape_projection_amd as dpg
    torch.manual_seed(0)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, T, d0, d1, d2, r = 4, 24, 48, 40, 24, 16
    l0 = dpg.ProjectedLinear(d0, d1, layer_id=3)
    l1 = dpg.ProjectedLinear(d1, d2, layer_id=8)
    C, sigma, seed, lr = 0.5, 0.6, 77, 1e-2
    opt = dpg.GrapeOptimizer([l0, l1], r=r, clip_C=C, sigma=sigma, seed=seed, lr=lr,
                             keep_inputs=True)
    x = torch.randn(B, T, d0, device="cuda").to(tdt)
    target = torch.randn(B, T, d2, device="cuda").to(tdt)
    m = {3: np.zeros((r, d1)), 8: np.zeros((r, d2))}
    v = {3: np.zeros((r, d1)), 8: np.zeros((r, d2))}
    tol = TOL[dtype]
    for step in (1, 2):
        W_old = {3: l0.W.cpu().numpy().astype(np.float64),
                 8: l1.W.cpu().numpy().astype(np.float64)}
        opt.zero_grad()
        xi = x.clone().requires_grad_(True)
        y = l1(torch.tanh(l0(xi)))
        loss = ((y.float() - target.float()) ** 2).sum()
        loss.backward()
        opt.step()
        torch.cuda.synchronize()
        layers = [{"A": opt.inputs[i][0].float().cpu().numpy().astype(np.float64),
                   "dY": opt.inputs[i][1].float().cpu().numpy().astype(np.float64),
                   "layer_id": i} for i in (3, 8)]
        want = oracle.project_clip_noise(layers, r, C, sigma, seed, step, step)
        e_n = rel_err(opt.last_norms.cpu().numpy(), want["norms"])
        e_g = max(rel_err(g.cpu().numpy(), w)
                  for g, w in zip(opt.last_G_priv, want["G_priv"]))
        # the update, stage-isolated on the GPU's G_priv
        params = [{"W": W_old[i], "m": m[i], "v": v[i],
                   "G_priv": g.cpu().numpy().astype(np.float64), "layer_id": i}
                  for i, g in zip((3, 8), opt.last_G_priv)]
        upd = oracle.adam_backproject(params, r, lr, 0.9, 0.999, 1e-8, seed, step, step)
        e_w = max(rel_err_dw(lw.W.cpu().numpy(), W_old[i], u["dW"])
                  for lw, i, u in zip((l0, l1), (3, 8), upd))
        e_m = max(rel_err(mm.cpu().numpy(), u["m"]) for mm, u in zip(opt.m, upd))
        print(f"[autograd {dtype}] step {step}: norms {e_n:.2e} G_priv {e_g:.2e} "
              f"dW {e_w:.2e} m {e_m:.2e}", flush=True)
        assert max(e_n, e_g, e_w, e_m) <= tol
        for i, u in zip((3, 8), upd):
            m[i], v[i] = u["m"], u["v"]
