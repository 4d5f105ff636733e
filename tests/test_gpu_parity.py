"""GPU parity: libdpg (through its C ABI) against the float64 CPU oracle.

Each case feeds the same seeded inputs to both sides and compares, per layer
and per tensor, the largest relative Frobenius error over the pieces of the
tensor (one row cut into runs of 256 columns; each sample's norm on its own;
tests/_helpers.rel_err) against the bar for the input type (fp32 1e-5, bf16
2e-2):
  * sample norms n_i and the privatised projected gradient G_priv, with the
    workload's sigma and with sigma = 0 (with noise on, G_priv is dominated
    by the noise, so sigma = 0 is what checks the contraction);
  * the update call stage-isolated: both sides take the GPU's own G_priv and
    the same (W, m, v), and dW = W_new - W_old, m and v are compared. (At
    Adam's first step U is close to sign(G_priv); entries of G_priv within
    the bf16 rounding band of zero can flip sign, so an end-to-end dW check
    is only asserted for fp32 inputs.)
The random streams are compared word for word.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from _helpers import (TOL, make_case, rel_err, rel_err_dw, run_adam, run_project,
                      to_device, torch_dtype)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_and_library():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dp_grape_projection_amd as dpg
    dpg.load_library()     # fails loudly when libdpg.so is missing
    print(f"[gpu] {torch.cuda.get_device_name(0)}; lib {dpg.library_path()}",
          flush=True)


# ----------------------------------------------------------- random stream --

@pytest.mark.parametrize("seed,layer,stepw,tag,start,n", [
    (0, 0, 1, 0, 0, 4096),
    (0, 5, 1, 1, 3, 1001),
    (2 ** 40 + 7, 143, 99, 0, 12345, 777),
    (123456789, 7, 2 ** 32 - 1, 1, 2 ** 31, 64),
    # 2^23 values reach the tails: six with |z| > 5, max |z| = 5.47
    (0, 3, 1, 0, 0, 1 << 23),
])
def test_philox_stream(seed, layer, stepw, tag, start, n):
    """Philox words bit for bit; normals within 1e-6 absolute of the float64
    definition and, more tightly, within half an fp32 ulp (the kernels
    evaluate Box-Muller in float64 and round once) plus 1e-10."""
    import dp_grape_projection_amd as dpg
    from oracle.philox import philox_words
    z, w = dpg.dpg_philox_normals(seed, layer, stepw, tag, start, n, words=True)
    z32 = z.cpu().numpy()
    z = z32.astype(np.float64)
    w = w.cpu().numpy().view(np.uint32).reshape(-1, 4)
    c = np.arange(start >> 2, ((start + n - 1) >> 2) + 1, dtype=np.uint64)
    want_w = np.stack(philox_words(seed, layer, stepw, tag, c), axis=1)
    np.testing.assert_array_equal(w, want_w)
    want_z = oracle.gaussian_stream(seed, layer, stepw, tag, n, start=start)
    err = np.abs(z - want_z)
    print(f"[philox] n={n}: max |z| {np.abs(want_z).max():.3f}, "
          f"max abs error {err.max():.3e}", flush=True)
    assert err.max() <= 1e-6, err.max()
    half_ulp = 0.5 * np.spacing(np.abs(z32)).astype(np.float64)
    assert np.all(err <= half_ulp + 1e-10), (err - half_ulp).max()


# --------------------------------------------------------------- the step --

CASES = {
    "tiny": W.workload("tiny"),
    "ragged_bf16": W.custom_workload("ragged_bf16", 11,
                                     [(200, 136), (136, 300), (72, 40)],
                                     B=3, T=40, r=40, layer_ids=[5, 17, 2]),
    "ragged_fp32": W.custom_workload("ragged_fp32", 12,
                                     [(200, 136), (136, 300), (72, 40)],
                                     B=3, T=40, r=40, dtype="fp32",
                                     layer_ids=[5, 17, 2]),
    "odd_dims_bf16": W.custom_workload("odd_dims_bf16", 13,
                                       [(37, 29), (29, 53)], B=2, T=13, r=7),
    "odd_dims_fp32": W.custom_workload("odd_dims_fp32", 14,
                                       [(37, 29), (29, 53)], B=2, T=13, r=7,
                                       dtype="fp32"),
    "multi_tile_bf16": W.custom_workload("multi_tile_bf16", 15, [(300, 260)],
                                         B=5, T=70, r=150, clip_C=0.3,
                                         sigma=0.5),
    "single": W.custom_workload("single", 16, [(8, 8)], B=1, T=1, r=1),
    # more layers than one launch takes (48): two launches per kernel
    "many_layers": W.custom_workload("many_layers", 17,
                                     [(24, 16), (16, 24)] * 26, B=2, T=8,
                                     r=8, layer_ids=list(range(100, 152))),
    # bf16 projection on the LDS ring: full 128 x 64 tiles next to ragged
    # ones (r = 160, B*T = 600) and a ragged contraction tail (d_in = 200,
    # 328)
    "ring_edges_bf16": W.custom_workload("ring_edges_bf16", 21,
                                         [(200, 96), (328, 40)], B=2, T=300,
                                         r=160),
    # every tile and step full (r, B*T, d_in, d_out whole tiles, T and r
    # whole steps): the kernels compiled without edge code
    "full_tiles_bf16": W.custom_workload("full_tiles_bf16", 23,
                                         [(256, 256), (384, 128)], B=2, T=128,
                                         r=128),
    "full_tiles_fp32": W.custom_workload("full_tiles_fp32", 24,
                                         [(128, 256), (256, 128)], B=2, T=64,
                                         r=128, dtype="fp32"),
    # more than 1024 norm partials per sample: clip factors come from the
    # separate scale launch instead of the sum pass's prologue
    "wide_unfused_bf16": W.custom_workload("wide_unfused_bf16", 18,
                                           [(64, 17920), (48, 16640)], B=3,
                                           T=8, r=16),
    # many tiles x samples: the sum pass adds several samples per block,
    # each with its own clip factor
    "groups_bf16": W.custom_workload("groups_bf16", 19,
                                     [(32, 6400), (32, 6400)], B=33, T=8,
                                     r=16),
    "groups_fp32": W.custom_workload("groups_fp32", 20,
                                     [(32, 6400), (32, 6400)], B=33, T=8,
                                     r=16, dtype="fp32"),
    # the large-projection kernel (r and B*T multiples of 256, d_in of 64):
    # unsplit; split over d_in (partials and xsum); odd T (sample boundaries
    # between a lane's two columns)
    "big_bf16": W.custom_workload("big_bf16", 25, [(192, 160), (128, 96)], B=2,
                                  T=256, r=256),
    "big_split_bf16": W.custom_workload("big_split_bf16", 26, [(2048, 64)], B=2,
                                        T=256, r=256),
    "big_odd_t_bf16": W.custom_workload("big_odd_t_bf16", 27, [(64, 32)], B=256,
                                        T=3, r=256),
    # the large norm and sum kernel (r and d_out multiples of 256, T of 64):
    # two layers, several K steps per sample; r of two tiles with one K step
    # per sample; more than 1024 partials per sample (separate scale
    # launch); enough tiles that norm runs and sum groups hold 4 samples
    "samp_big_bf16": W.custom_workload("samp_big_bf16", 28, [(128, 256), (64, 512)],
                                       B=3, T=128, r=256),
    "samp_big_r512_bf16": W.custom_workload("samp_big_r512_bf16", 29,
                                            [(96, 256), (256, 768)], B=5, T=64,
                                            r=512),
    "samp_big_wide_bf16": W.custom_workload("samp_big_wide_bf16", 30, [(32, 33024)],
                                            B=2, T=64, r=256),
    "samp_big_groups_bf16": W.custom_workload("samp_big_groups_bf16", 31,
                                              [(32, 10240)], B=16, T=64, r=256),
    # the large back-projection kernel (d_in, d_out multiples of 256, r of 64
    # over one 128-step): two layers; r = 192; more than one round of
    # blocks, so that each block sweeps a run of two column tiles
    "back_big_bf16": W.custom_workload("back_big_bf16", 32, [(256, 512), (512, 256)],
                                       B=2, T=64, r=256),
    "back_big_r192_bf16": W.custom_workload("back_big_r192_bf16", 33, [(256, 256)],
                                            B=2, T=64, r=192),
    "back_big_runs_bf16": W.custom_workload("back_big_runs_bf16", 34, [(4096, 8192)],
                                            B=2, T=64, r=256),
    # runs of three column tiles over 34: the last run holds one tile
    "back_big_ragged_run_bf16": W.custom_workload("back_big_ragged_run_bf16", 38,
                                                  [(4096, 8704)], B=2, T=64, r=256),
    # T at least 8 r: the norm pass stores every sample's product and the
    # final pass sums them weighted by the clip factors (no second pass over
    # dY); with the large norm kernel, the regular one, and fp32
    "hat_big_bf16": W.custom_workload("hat_big_bf16", 35, [(128, 256), (64, 512)],
                                      B=3, T=2048, r=256),
    "hat_bf16": W.custom_workload("hat_bf16", 36, [(200, 136), (72, 40)], B=2,
                                  T=512, r=40),
    "hat_fp32": W.custom_workload("hat_fp32", 37, [(37, 29), (29, 53)], B=2, T=256,
                                  r=7, dtype="fp32"),
    # fewer tiles: sum groups of 2 samples (accumulator rescaled between
    # them), with a single-sample last group
    "groups4_bf16": W.custom_workload("groups4_bf16", 22,
                                      [(32, 1280), (32, 1280)], B=33, T=8,
                                      r=16),
}


def _check_project(wl, host, orc, sigma, C=None, tag=""):
    C = wl.clip_C if C is None else C
    G, n = run_project(wl, host, sigma=sigma, clip_C=C)
    want = oracle.project_clip_noise(orc, wl.r, C, sigma, wl.seed, wl.step,
                                     wl.proj_step)
    tol = TOL[wl.dtype]
    e_n = rel_err(n, want["norms"])
    assert e_n <= tol, f"{tag} norms {e_n}"
    errs = [rel_err(g, w) for g, w in zip(G, want["G_priv"])]
    print(f"[{wl.name}{tag} sigma={sigma}] norms {e_n:.2e} "
          f"G_priv max {max(errs):.2e}", flush=True)
    assert max(errs) <= tol, errs
    return G, want


def _check_adam(wl, G, state, tag=""):
    new = run_adam(wl, G, state)
    params = [{"W": s[0].astype(np.float64), "m": s[1].astype(np.float64),
               "v": s[2].astype(np.float64), "G_priv": g.astype(np.float64),
               "layer_id": L.layer_id}
              for s, g, L in zip(state, G, wl.layers)]
    want = oracle.adam_backproject(params, wl.r, wl.lr, wl.beta1, wl.beta2,
                                   wl.eps, wl.seed, wl.step, wl.proj_step)
    tol = TOL[wl.dtype]
    worst = 0.0
    for (Wn, mn, vn), s, w in zip(new, state, want):
        e = max(rel_err_dw(Wn, s[0], w["dW"]), rel_err(mn, w["m"]),
                rel_err(vn, w["v"]))
        worst = max(worst, e)
    print(f"[{wl.name}{tag}] adam+backproject (stage-isolated) {worst:.2e}",
          flush=True)
    assert worst <= tol
    return new, want


@pytest.mark.parametrize("name", list(CASES))
def test_step_parity(name):
    wl = CASES[name]
    print(f"[case] {name}: {len(wl.layers)} layers B={wl.B} T={wl.T} "
          f"r={wl.r} {wl.dtype}", flush=True)
    host, orc, state = make_case(wl)
    _check_project(wl, host, orc, sigma=0.0)
    G, _ = _check_project(wl, host, orc, sigma=wl.sigma)
    _check_adam(wl, G, state)


def test_tiny_end_to_end_fp32():
    """fp32 inputs: the whole step end to end, dW included."""
    wl = CASES["tiny"]
    host, orc, state = make_case(wl)
    G, n = run_project(wl, host)
    new = run_adam(wl, G, state)
    want = oracle.project_clip_noise(orc, wl.r, wl.clip_C, wl.sigma, wl.seed,
                                     wl.step, wl.proj_step)
    params = [{"W": s[0].astype(np.float64), "m": s[1].astype(np.float64),
               "v": s[2].astype(np.float64), "G_priv": g, "layer_id": L.layer_id}
              for s, g, L in zip(state, want["G_priv"], wl.layers)]
    w2 = oracle.adam_backproject(params, wl.r, wl.lr, wl.beta1, wl.beta2,
                                 wl.eps, wl.seed, wl.step, wl.proj_step)
    for (Wn, mn, vn), s, w in zip(new, state, w2):
        assert rel_err_dw(Wn, s[0], w["dW"]) <= TOL["fp32"]
        assert rel_err(mn, w["m"]) <= TOL["fp32"]
        assert rel_err(vn, w["v"]) <= TOL["fp32"]


def test_noise_alone_matches_stream():
    """A = 0: G_priv = sigma C Z / B exactly, Z the layer's noise stream in the
    projected [r, d_out] space."""
    wl = CASES["ragged_bf16"]
    host, orc, _ = make_case(wl, a_zero=True)
    G, n = run_project(wl, host)
    assert np.all(n == 0.0)
    for g, L in zip(G, wl.layers):
        Z = oracle.noise_matrix(wl.seed, L.layer_id, wl.step, wl.r, L.d_out)
        assert rel_err(g, wl.sigma * wl.clip_C * Z / wl.B) <= 1e-6


def test_no_clipping_is_plain_mean():
    """C = +inf and sigma = 0: G_priv is the batch mean of the projected
    per-sample gradients."""
    wl = CASES["multi_tile_bf16"]
    host, orc, _ = make_case(wl)
    G, n = run_project(wl, host, clip_C=math.inf, sigma=0.0)
    want = oracle.project_clip_noise(orc, wl.r, math.inf, 0.0, wl.seed,
                                     wl.step, wl.proj_step)
    for g, w in zip(G, want["G_priv"]):
        assert rel_err(g, w) <= TOL["bf16"]


@pytest.mark.parametrize("name", ["ragged_bf16", "groups_bf16", "groups_fp32",
                                  "groups4_bf16"])
def test_mixed_clipping(name):
    """C near the median norm: some samples clipped, some not."""
    wl = CASES[name]
    host, orc, _ = make_case(wl)
    n = oracle.project_clip_noise(orc, wl.r, math.inf, 0.0, wl.seed, wl.step,
                                  wl.proj_step)["norms"]
    C = float(np.median(n))
    s = oracle.dpgrape.clip_scale(n, C)
    assert (s < 1).any() and (s == 1).any()
    _check_project(wl, host, orc, sigma=0.0, C=C, tag=" mixed")


@pytest.mark.parametrize("name", ["multi_tile_bf16", "big_bf16", "samp_big_r512_bf16",
                                  "back_big_bf16"])
def test_deterministic_bitwise(name):
    """Two runs of the same step give the same bits: the regular tiles, the
    large projection, the large per-sample kernels (r = 512) and the large
    back-projection."""
    wl = CASES[name]
    host, _, state = make_case(wl)
    G1, n1 = run_project(wl, host)
    G2, n2 = run_project(wl, host)
    np.testing.assert_array_equal(n1, n2)
    for a, b in zip(G1, G2):
        np.testing.assert_array_equal(a, b)
    w1 = run_adam(wl, G1, state)
    w2 = run_adam(wl, G1, state)
    for a, b in zip(w1, w2):
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


def test_three_steps_and_resume():
    """Three steps with fresh P each step; state copied to the host and back
    between steps gives bit-identical results to keeping it on the device,
    and each step's update matches the oracle stage-isolated."""
    import torch
    import dp_grape_projection_amd as dpg
    wl = CASES["ragged_bf16"]
    host, orc, state = make_case(wl)
    A = [to_device(wl, a) for a, _ in host]
    dY = [to_device(wl, d) for _, d in host]
    ids = [L.layer_id for L in wl.layers]
    Wd = [torch.from_numpy(s[0].copy()).cuda() for s in state]
    md = [torch.from_numpy(s[1].copy()).cuda() for s in state]
    vd = [torch.from_numpy(s[2].copy()).cuda() for s in state]
    cur = [tuple(x.copy() for x in s) for s in state]
    for step in (1, 2, 3):
        G, _ = dpg.dpg_project_clip_noise(A, dY, wl.r, wl.clip_C, wl.sigma,
                                          wl.seed, step, step, layer_ids=ids)
        dpg.dpg_adam_backproject(G, Wd, md, vd, wl.r, wl.lr, wl.beta1,
                                 wl.beta2, wl.eps, wl.seed, step, step,
                                 layer_ids=ids, dtype=torch_dtype(wl))
        Gh = [g.cpu().numpy() for g in G]
        new = run_adam(wl, Gh, cur, step=step, proj_step=step)
        params = [{"W": c[0].astype(np.float64), "m": c[1].astype(np.float64),
                   "v": c[2].astype(np.float64), "G_priv": g.astype(np.float64),
                   "layer_id": i} for c, g, i in zip(cur, Gh, ids)]
        want = oracle.adam_backproject(params, wl.r, wl.lr, wl.beta1, wl.beta2,
                                       wl.eps, wl.seed, step, step)
        for (Wn, mn, vn), c, w in zip(new, cur, want):
            assert rel_err_dw(Wn, c[0], w["dW"]) <= TOL["bf16"]
            assert rel_err(mn, w["m"]) <= TOL["bf16"]
        cur = new
    torch.cuda.synchronize()
    for (Wn, mn, vn), w, m, v in zip(cur, Wd, md, vd):
        np.testing.assert_array_equal(Wn, w.cpu().numpy())
        np.testing.assert_array_equal(mn, m.cpu().numpy())
        np.testing.assert_array_equal(vn, v.cpu().numpy())


# ------------------------------------------------- bench workload, full size --

def test_mlp4_full_size():
    """The 4-layer MLP workload the bench times, at its full size and in the
    same launch configuration: the whole oracle runs (a few seconds)."""
    wl = W.workload("mlp4")
    host, orc, state = make_case(wl)
    _check_project(wl, host, orc, sigma=0.0)
    G, want = _check_project(wl, host, orc, sigma=wl.sigma)
    _check_adam(wl, G, state)
    # end to end dW, reported only (sign flips of near-zero G_priv entries)
    new = run_adam(wl, G, state)
    params = [{"W": s[0].astype(np.float64), "m": s[1].astype(np.float64),
               "v": s[2].astype(np.float64), "G_priv": g, "layer_id": L.layer_id}
              for s, g, L in zip(state, want["G_priv"], wl.layers)]
    w2 = oracle.adam_backproject(params, wl.r, wl.lr, wl.beta1, wl.beta2,
                                 wl.eps, wl.seed, wl.step, wl.proj_step)
    e2e = max(rel_err_dw(n[0], s[0], w["dW"])
              for n, s, w in zip(new, state, w2))
    print(f"[mlp4] end-to-end dW rel error (reported) {e2e:.3e}", flush=True)
