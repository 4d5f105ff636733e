"""Shared helpers of the GPU parity tests: seeded inputs from `workloads`,
device copies, and the relative Frobenius error used as the parity metric."""
import math

import numpy as np

import workloads as W

# Parity bars (max relative Frobenius error per tensor per layer): fp32
# inputs 1e-5, bf16 inputs 2e-2.
TOL = {"fp32": 1e-5, "bf16": 2e-2}


def rel_fro(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    if den == 0.0:
        return float(num)
    return float(num / den)


def to_device(wl, arr):
    import torch
    if wl.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
        return t.view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def torch_dtype(wl):
    import torch
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def make_case(wl, dy_zero=False, a_zero=False):
    """Host inputs of a workload: per layer (A, dY) in the workload's dtype,
    the oracle's float64 views, and the initial (W, m, v)."""
    host, orc, state = [], [], []
    for L in wl.layers:
        A, dY = W.layer_inputs(wl, L)
        if a_zero:
            A = np.zeros_like(A)
        if dy_zero:
            dY = np.zeros_like(dY)
        host.append((A, dY))
        orc.append({"A": W.as_float64(wl, A), "dY": W.as_float64(wl, dY),
                    "layer_id": L.layer_id})
        state.append(W.initial_state(wl, L))
    return host, orc, state


def run_project(wl, host, **kw):
    import dp_grape_projection_amd as dpg
    A = [to_device(wl, a) for a, _ in host]
    dY = [to_device(wl, d) for _, d in host]
    args = dict(r=wl.r, clip_C=wl.clip_C, sigma=wl.sigma, seed=wl.seed,
                step=wl.step, proj_step=wl.proj_step,
                layer_ids=[L.layer_id for L in wl.layers])
    args.update(kw)
    G, n = dpg.dpg_project_clip_noise(A, dY, **args)
    return [g.cpu().numpy() for g in G], n.cpu().numpy()


def run_adam(wl, G_priv, state, step=None, proj_step=None):
    """Runs dpg_adam_backproject on copies of `state`; returns new (W, m, v)
    per layer as float64 arrays."""
    import torch
    import dp_grape_projection_amd as dpg
    Wd = [torch.from_numpy(s[0].copy()).cuda() for s in state]
    md = [torch.from_numpy(s[1].copy()).cuda() for s in state]
    vd = [torch.from_numpy(s[2].copy()).cuda() for s in state]
    Gd = [torch.from_numpy(np.ascontiguousarray(g, np.float32)).cuda()
          for g in G_priv]
    step = wl.step if step is None else step
    proj_step = wl.proj_step if proj_step is None else proj_step
    dpg.dpg_adam_backproject(Gd, Wd, md, vd, r=wl.r, lr=wl.lr,
                             beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                             seed=wl.seed, step=step, proj_step=proj_step,
                             layer_ids=[L.layer_id for L in wl.layers],
                             dtype=torch_dtype(wl))
    torch.cuda.synchronize()
    return [(w.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy())
            for w, m, v in zip(Wd, md, vd)]
