"""GPU parity of the one-call step (dpg_private_step).

The one-call step is the projection call followed by the update call with P
shared and the moments computed where G_priv is formed, so its results are
those of the two calls bit for bit. Each case checks:

  * G_priv, the norms, W, m and v bitwise against dpg_project_clip_noise +
    dpg_adam_backproject on copies of the same state;
  * G_priv and the norms against the float64 oracle;
  * the update stage-isolated on the GPU's G_priv (oracle.adam_backproject).

Two steps run in a row with proj_step held at 1, so the second uses the
first step's P with fresh noise and bias corrections of t = 2.
Bars as in the other parity tests: fp32 1e-5, bf16 2e-2 (relative Frobenius).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from _helpers import TOL, make_case, rel_err, rel_err_dw, to_device, torch_dtype

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
    "ragged_bf16": W.custom_workload("o_ragged_bf16", 41,
                                     [(200, 136), (136, 300), (72, 40)],
                                     B=3, T=40, r=40, layer_ids=[5, 17, 2]),
    "odd_fp32": W.custom_workload("o_odd_fp32", 42, [(37, 29), (29, 53)],
                                  B=2, T=13, r=7, dtype="fp32"),
    # whole tiles everywhere: the kernels without edge code, and P resident
    # in LDS for the back-projection (r within one step)
    "full_bf16": W.custom_workload("o_full_bf16", 43, [(256, 256), (384, 128)],
                                   B=2, T=128, r=128),
    "full_fp32": W.custom_workload("o_full_fp32", 44, [(128, 256), (256, 128)],
                                   B=2, T=64, r=128, dtype="fp32"),
    # r over one contraction step: the streamed back-projection
    "long_r_bf16": W.custom_workload("o_long_r_bf16", 45, [(300, 200)], B=2,
                                     T=100, r=272),
    # more than 1024 norm partials per sample: separate scale launch
    "wide_bf16": W.custom_workload("o_wide_bf16", 46, [(64, 17920), (48, 16640)],
                                   B=3, T=8, r=16),
    "groups_bf16": W.custom_workload("o_groups_bf16", 47, [(32, 6400), (32, 6400)],
                                     B=33, T=8, r=16),
    # T at least 8 r: products stored by the norm pass, summed in the final
    # pass
    "hat_bf16": W.custom_workload("o_hat_bf16", 49, [(200, 136), (72, 40)], B=3,
                                  T=400, r=40),
    # the large norm and sum kernel
    "samp_big_bf16": W.custom_workload("o_samp_big_bf16", 48, [(128, 256), (64, 512)],
                                       B=3, T=128, r=256),
}


def _state(state):
    import torch
    return ([torch.from_numpy(s[0].copy()).cuda() for s in state],
            [torch.from_numpy(s[1].copy()).cuda() for s in state],
            [torch.from_numpy(s[2].copy()).cuda() for s in state])


def _np(ts):
    return [t.cpu().numpy() for t in ts]


@pytest.mark.parametrize("name", list(CASES))
def test_one_call_step(name):
    import torch
    import dp_grape_projection_amd as dpg
    wl = CASES[name]
    print(f"[one-call] {name}: {len(wl.layers)} layers B={wl.B} T={wl.T} r={wl.r} "
          f"{wl.dtype}", flush=True)
    host, orc, state = make_case(wl)
    A = [to_device(wl, a) for a, _ in host]
    dY = [to_device(wl, d) for _, d in host]
    ids = [L.layer_id for L in wl.layers]
    W1, m1, v1 = _state(state)
    W2, m2, v2 = _state(state)
    hyper = dict(r=wl.r, clip_C=wl.clip_C, sigma=wl.sigma, seed=wl.seed)
    adam = dict(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps)
    tol = TOL[wl.dtype]
    cur = [tuple(x.astype(np.float64) for x in s) for s in state]
    for step in (1, 2):
        G1, n1 = dpg.dpg_private_step(A, dY, W1, m1, v1, step=step, proj_step=1,
                                      layer_ids=ids, **hyper, **adam)
        G2, n2 = dpg.dpg_project_clip_noise(A, dY, step=step, proj_step=1,
                                            layer_ids=ids, **hyper)
        dpg.dpg_adam_backproject(G2, W2, m2, v2, wl.r, seed=wl.seed, step=step,
                                 proj_step=1, layer_ids=ids, dtype=torch_dtype(wl),
                                 **adam)
        torch.cuda.synchronize()
        # bitwise against the two calls
        assert torch.equal(n1, n2)
        for a, b in zip(G1 + W1 + m1 + v1, G2 + W2 + m2 + v2):
            assert torch.equal(a, b)
        # G_priv and norms against the oracle
        want = oracle.project_clip_noise(orc, wl.r, wl.clip_C, wl.sigma, wl.seed,
                                         step, 1)
        e_n = rel_err(n1.cpu().numpy(), want["norms"])
        e_g = max(rel_err(g, w) for g, w in zip(_np(G1), want["G_priv"]))
        # the update, stage-isolated on the GPU's G_priv
        params = [{"W": c[0], "m": c[1], "v": c[2],
                   "G_priv": g.astype(np.float64), "layer_id": L.layer_id}
                  for c, g, L in zip(cur, _np(G1), wl.layers)]
        upd = oracle.adam_backproject(params, wl.r, wl.lr, wl.beta1, wl.beta2,
                                      wl.eps, wl.seed, step, 1)
        Wn, mn, vn = _np(W1), _np(m1), _np(v1)
        e_w = max(rel_err_dw(w, c[0], u["dW"])
                  for w, c, u in zip(Wn, cur, upd))
        e_m = max(rel_err(m, u["m"]) for m, u in zip(mn, upd))
        e_v = max(rel_err(v, u["v"]) for v, u in zip(vn, upd))
        print(f"[one-call] {name} step {step}: norms {e_n:.2e} G_priv {e_g:.2e} "
              f"dW {e_w:.2e} m {e_m:.2e} v {e_v:.2e}", flush=True)
        assert max(e_n, e_g, e_w, e_m, e_v) <= tol
        cur = [(w.astype(np.float64), m.astype(np.float64), v.astype(np.float64))
               for w, m, v in zip(Wn, mn, vn)]


def test_prepared_step_one_call_equals_two_calls():
    """PreparedStep (the bench's driver) gives the same state either way."""
    import torch
    import dp_grape_projection_amd as dpg
    wl = CASES["ragged_bf16"]
    host, _, state = make_case(wl)
    A = [to_device(wl, a) for a, _ in host]
    dY = [to_device(wl, d) for _, d in host]
    out = []
    for one_call in (True, False):
        Ws, ms, vs = _state(state)
        ps = dpg.PreparedStep(A, dY, Ws, ms, vs, wl.r, wl.clip_C, wl.sigma,
                              wl.seed, wl.lr, wl.beta1, wl.beta2, wl.eps,
                              layer_ids=[L.layer_id for L in wl.layers],
                              one_call=one_call)
        for step in (1, 2, 3):
            ps.run(step)
        torch.cuda.synchronize()
        out.append(_np(ps.G_priv) + [ps.sample_norms.cpu().numpy()] + _np(Ws)
                   + _np(ms) + _np(vs))
    for a, b in zip(*out):
        np.testing.assert_array_equal(a, b)


# Caller tensors that start one element past an aligned address: the
# large-tile kernels (which need 16-byte rows) and every vector access to a
# caller pointer step aside for their element-wise forms. The bf16 case has
# shapes that take all three large-tile kernels when aligned.
UNALIGNED = {
    "big_bf16": W.custom_workload("u_big_bf16", 50, [(256, 512), (512, 256)], B=4,
                                  T=128, r=256),
    "fp32": W.custom_workload("u_fp32", 51, [(64, 96), (96, 40)], B=2, T=24, r=16,
                              dtype="fp32"),
}


def _offset_copy(t):
    """A copy of t whose data starts one element past t's allocation start."""
    import torch
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("name", list(UNALIGNED))
def test_unaligned_caller_tensors(name):
    import torch
    import dp_grape_projection_amd as dpg
    wl = UNALIGNED[name]
    print(f"[unaligned] {name}: {len(wl.layers)} layers B={wl.B} T={wl.T} r={wl.r} "
          f"{wl.dtype}", flush=True)
    host, orc, state = make_case(wl)
    A = [_offset_copy(to_device(wl, a)) for a, _ in host]
    dY = [_offset_copy(to_device(wl, d)) for _, d in host]
    assert all(t.data_ptr() % 16 != 0 for t in A + dY)
    ids = [L.layer_id for L in wl.layers]
    hyper = dict(r=wl.r, clip_C=wl.clip_C, sigma=wl.sigma, seed=wl.seed)
    adam = dict(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps)
    W1, m1, v1 = [[_offset_copy(x) for x in xs] for xs in _state(state)]
    W2, m2, v2 = [[_offset_copy(x) for x in xs] for xs in _state(state)]
    G1, n1 = dpg.dpg_private_step(A, dY, W1, m1, v1, step=1, proj_step=1,
                                  layer_ids=ids, **hyper, **adam)
    G2 = [_offset_copy(torch.zeros(wl.r, L.d_out, device="cuda")) for L in wl.layers]
    G2, n2 = dpg.dpg_project_clip_noise(A, dY, step=1, proj_step=1, layer_ids=ids,
                                        G_priv=G2, **hyper)
    dpg.dpg_adam_backproject(G2, W2, m2, v2, wl.r, seed=wl.seed, step=1, proj_step=1,
                             layer_ids=ids, dtype=torch_dtype(wl), **adam)
    torch.cuda.synchronize()
    tol = TOL[wl.dtype]
    want = oracle.project_clip_noise(orc, wl.r, wl.clip_C, wl.sigma, wl.seed, 1, 1)
    params = [{"W": s[0].astype(np.float64), "m": s[1].astype(np.float64),
               "v": s[2].astype(np.float64), "G_priv": g.astype(np.float64),
               "layer_id": L.layer_id}
              for s, g, L in zip(state, _np(G1), wl.layers)]
    upd = oracle.adam_backproject(params, wl.r, wl.lr, wl.beta1, wl.beta2, wl.eps,
                                  wl.seed, 1, 1)
    for G, n, Ws, ms, vs in ((G1, n1, W1, m1, v1), (G2, n2, W2, m2, v2)):
        e_n = rel_err(n.cpu().numpy(), want["norms"])
        e_g = max(rel_err(g, w) for g, w in zip(_np(G), want["G_priv"]))
        e_w = max(rel_err_dw(w, s[0], u["dW"])
                  for w, s, u in zip(_np(Ws), state, upd))
        e_m = max(rel_err(m, u["m"]) for m, u in zip(_np(ms), upd))
        e_v = max(rel_err(v, u["v"]) for v, u in zip(_np(vs), upd))
        print(f"[unaligned] {name}: norms {e_n:.2e} G_priv {e_g:.2e} dW {e_w:.2e} "
              f"m {e_m:.2e} v {e_v:.2e}", flush=True)
        assert max(e_n, e_g, e_w, e_m, e_v) <= tol
    # the one-call and two-call forms agree bit for bit here too
    assert torch.equal(n1, n2)
    for a, b in zip(G1 + W1 + m1 + v1, G2 + W2 + m2 + v2):
        assert torch.equal(a, b)


def test_side_stream_matches_default_stream():
    """A call given a stream other than torch's current one: its outputs and
    temporary workspace are allocated for that stream, and the results equal
    the default-stream call's bit for bit."""
    import torch
    import dp_grape_projection_amd as dpg
    wl = CASES["ragged_bf16"]
    host, _, state = make_case(wl)
    A = [to_device(wl, a) for a, _ in host]
    dY = [to_device(wl, d) for _, d in host]
    ids = [L.layer_id for L in wl.layers]
    kw = dict(r=wl.r, clip_C=wl.clip_C, sigma=wl.sigma, seed=wl.seed,
              step=wl.step, proj_step=wl.proj_step, layer_ids=ids)
    G0, n0 = dpg.dpg_project_clip_noise(A, dY, **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    G1, n1 = dpg.dpg_project_clip_noise(A, dY, stream=side, **kw)
    Wd, md, vd = _state(state)
    Wd2, md2, vd2 = _state(state)
    dpg.dpg_adam_backproject(G0, Wd, md, vd, wl.r, wl.lr, wl.beta1, wl.beta2,
                             wl.eps, wl.seed, wl.step, wl.proj_step,
                             layer_ids=ids, dtype=torch_dtype(wl))
    side.wait_stream(torch.cuda.current_stream())
    dpg.dpg_adam_backproject(G1, Wd2, md2, vd2, wl.r, wl.lr, wl.beta1, wl.beta2,
                             wl.eps, wl.seed, wl.step, wl.proj_step,
                             layer_ids=ids, dtype=torch_dtype(wl), stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(n0, n1)
    for a, b in zip(G0, G1):
        assert torch.equal(a, b)
    for x, y in zip(Wd + md + vd, Wd2 + md2 + vd2):
        assert torch.equal(x, y)
