"""GPU parity at the full sizes of the three large workloads, on sampled
outputs and on properties that hold at any size.

enc12 (72 layers, B=64, T=256, r=256), dec24 (144 layers, B=16, T=512,
r=512, Student-t output gradients) and long1 (6 layers, B=4, T=4096, r=256)
run through the C ABI exactly as a caller would, with inputs drawn in device
memory (workloads.device_layer_inputs). The float64 oracle cannot run these
steps whole, so each test checks:

  * the global per-sample norm is the root of the sum over layers of the
    per-layer squared norms, each taken from a single-layer call;
  * per-layer norms of sampled (layer, sample) pairs against the oracle's
    definition ||P_l A_il^T dY_il||_F (per-sample gradient materialised);
  * one whole row of G_priv in every layer (a different row in each) and
    three rows of the sampled layers, against oracle.g_priv_rows, with
    sigma = 0 and with the workload's sigma, stage-isolated on the clip
    factors that follow from the GPU's norms;
  * the update call stage-isolated: m and v of every layer, and sampled rows
    of dW, against oracle.adam_update / backproject_delta on the GPU's
    G_priv.

The bf16 bar (2e-2 relative) applies to every piece of a row (256 columns;
tests/_helpers.rel_err); the sum-of-squares property is checked at 1e-4 per
sample (both sides are fp32 sums of the same partial values in different
orders).
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from _helpers import TOL, rel_err, rel_err_dw

pytestmark = pytest.mark.gpu

# layers checked against the oracle (indices into the workload's layer list)
# and samples whose per-layer norms are checked
CHECKS = {
    "enc12": ([0, 5, 71], [0, 63]),   # blk0.q, blk0.down (3072->768), blk11.down
    "dec24": ([0, 5, 142], [0, 15]),  # blk0.q, blk0.down (8192->2048), blk23.up
    "long1": ([0, 3], [0, 3]),        # q, o (4096 x 4096, T = 4096)
}


@pytest.fixture(scope="module", autouse=True)
def gpu_and_library():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dp_grape_projection_amd as dpg
    dpg.load_library()     # fails loudly when libdpg.so is missing


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", list(CHECKS))
def test_full_size_sampled(name):
    import torch
    import dp_grape_projection_amd as dpg
    wl = W.workload(name)
    layers_chk, samples_chk = CHECKS[name]
    print(f"[full] {name}: {len(wl.layers)} layers B={wl.B} T={wl.T} r={wl.r} "
          f"{wl.dtype}", flush=True)
    A, dY = [], []
    for L in wl.layers:
        a, d = W.device_layer_inputs(wl, L)
        A.append(a)
        dY.append(d)
    ids = [L.layer_id for L in wl.layers]
    kw = dict(r=wl.r, seed=wl.seed, step=wl.step, proj_step=wl.proj_step,
              layer_ids=ids)
    C = wl.clip_C
    G0, n0 = dpg.dpg_project_clip_noise(A, dY, clip_C=C, sigma=0.0, **kw)
    G1, n1 = dpg.dpg_project_clip_noise(A, dY, clip_C=C, sigma=wl.sigma, **kw)
    torch.cuda.synchronize()
    assert torch.equal(n0, n1), "norms depend on sigma"
    n = _f64(n0)
    assert np.all(np.isfinite(n)) and np.all(n > 0)

    # global norm = root of the sum of per-layer squared norms
    sq = np.zeros(wl.B)
    per_layer = {}
    for l, L in enumerate(wl.layers):
        _, nl = dpg.dpg_project_clip_noise([A[l]], [dY[l]], clip_C=math.inf,
                                           sigma=0.0, r=wl.r, seed=wl.seed,
                                           step=wl.step, proj_step=wl.proj_step,
                                           layer_ids=[L.layer_id])
        nl = _f64(nl)
        sq += nl * nl
        if l in layers_chk:
            per_layer[l] = nl
    e_sq = rel_err(n * n, sq)
    print(f"[full] {name}: global vs per-layer squared norms {e_sq:.2e}", flush=True)
    assert e_sq <= 1e-4

    # per-layer norms of sampled (layer, sample) pairs
    Ps = {}
    worst = 0.0
    for l in layers_chk:
        L = wl.layers[l]
        Ps[l] = oracle.projection_matrix(wl.seed, L.layer_id, wl.proj_step,
                                         wl.r, L.d_in)
        for i in samples_chk:
            g = Ps[l] @ oracle.per_sample_gradient(_f64(A[l][i]), _f64(dY[l][i]))
            want = float(np.linalg.norm(g))
            worst = max(worst, abs(per_layer[l][i] - want) / want)
    print(f"[full] {name}: sampled per-layer norms, max rel error {worst:.2e}",
          flush=True)
    assert worst <= TOL[wl.dtype]

    # rows of G_priv, stage-isolated on the GPU's clip factors: one row of
    # every layer (row 37 l mod r), and three rows of the sampled layers
    s = oracle.clip_scale(n, C)
    worst0 = worst1 = 0.0
    for l, L in enumerate(wl.layers):
        rows = sorted({(37 * l) % wl.r} |
                      ({0, wl.r // 2, wl.r - 1} if l in layers_chk else set()))
        Pr = oracle.projection_rows(wl.seed, L.layer_id, wl.proj_step, wl.r,
                                    L.d_in, rows)
        if l in Ps:
            np.testing.assert_array_equal(Pr, Ps[l][rows])
        Zr = oracle.noise_rows(wl.seed, L.layer_id, wl.step, wl.r, L.d_out, rows)
        Af, dYf = _f64(A[l]), _f64(dY[l])
        want0 = oracle.g_priv_rows(Af, dYf, Pr, s, C, 0.0, None)
        want1 = oracle.g_priv_rows(Af, dYf, Pr, s, C, wl.sigma, Zr)
        del Af, dYf
        worst0 = max(worst0, rel_err(_f64(G0[l][rows]), want0))
        worst1 = max(worst1, rel_err(_f64(G1[l][rows]), want1))
    print(f"[full] {name}: G_priv rows of all {len(wl.layers)} layers, sigma=0 "
          f"{worst0:.2e}, sigma={wl.sigma} {worst1:.2e}", flush=True)
    assert worst0 <= TOL[wl.dtype] and worst1 <= TOL[wl.dtype]
    del A, dY

    # the update call, stage-isolated on the GPU's G_priv
    Ws, ms, vs = [], [], []
    for L in wl.layers:
        w, m, v = W.device_initial_state(wl, L)
        Ws.append(w)
        ms.append(m)
        vs.append(v)
    krows = {l: sorted({0, wl.layers[l].d_in // 2, wl.layers[l].d_in - 1})
             for l in layers_chk}
    W_old = {l: _f64(Ws[l][krows[l]]) for l in layers_chk}
    dpg.dpg_adam_backproject(G1, Ws, ms, vs, r=wl.r, lr=wl.lr, beta1=wl.beta1,
                             beta2=wl.beta2, eps=wl.eps, seed=wl.seed,
                             step=wl.step, proj_step=wl.proj_step,
                             layer_ids=ids, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    worst = worst_w = 0.0
    for l in range(len(wl.layers)):
        zero = np.zeros((wl.r, wl.layers[l].d_out))
        m1, v1, U = oracle.adam_update(_f64(G1[l]), zero, zero, wl.step,
                                       wl.beta1, wl.beta2, wl.eps)
        worst = max(worst, rel_err(_f64(ms[l]), m1), rel_err(_f64(vs[l]), v1))
        if l in layers_chk:
            dW = oracle.backproject_delta(Ps[l][:, krows[l]], U, wl.lr)
            worst_w = max(worst_w, rel_err_dw(Ws[l][krows[l]].cpu().numpy(), W_old[l], dW))
    print(f"[full] {name}: adam (m, v of every layer) {worst:.2e}, "
          f"back-projection rows (stage-isolated) {worst_w:.2e}", flush=True)
    assert worst <= TOL[wl.dtype] and worst_w <= TOL[wl.dtype]
