"""Shared helpers of the GPU parity tests: seeded inputs from `workloads`,
device copies, and the relative Frobenius error used as the parity metric."""
import math

import numpy as np

import workloads as W

# Parity bars: fp32 inputs 1e-5, bf16 inputs 2e-2, applied by rel_err to
# every piece of a tensor (below), not to the tensor as a whole.
TOL = {"fp32": 1e-5, "bf16": 2e-2}

# Width of the row pieces rel_err compares.
SEG = 256


def rel_fro(got, want) -> float:
    """Relative Frobenius error of a whole tensor (reported beside rel_err)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    if den == 0.0:
        return float(num)
    return float(num / den)


def rel_err(got, want, width: int = SEG) -> float:
    """The parity metric: the largest relative Frobenius error over the
    pieces of a tensor. A matrix is cut into pieces of one row and `width`
    consecutive columns (the last piece of a row is its last `width`
    columns, overlapping the one before, so that no piece is a short tail
    whose few elements make the ratio noisy; rows narrower than `width` are
    one piece); each element of a vector (per-sample norms) is a piece of
    its own. A localised mistake (one wrong column of an 8192-wide layer,
    one wrong row, one sample) then shows at full size instead of being
    averaged over the whole tensor. A piece whose reference is all zeros
    contributes its absolute error."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    if want.ndim <= 1:
        got, want = got.reshape(-1, 1), want.reshape(-1, 1)
    else:
        got, want = got.reshape(-1, want.shape[-1]), want.reshape(-1, want.shape[-1])
    worst = 0.0
    n = want.shape[1]
    for c0 in range(0, n, width):
        c0 = min(c0, max(n - width, 0))
        w, g = want[:, c0:c0 + width], got[:, c0:c0 + width]
        den = np.linalg.norm(w, axis=1)
        num = np.linalg.norm(g - w, axis=1)
        r = np.where(den > 0.0, num / np.where(den > 0.0, den, 1.0), num)
        worst = max(worst, float(r.max()))
    return worst


def rel_err_dw(W_new, W_old, dW_want, width: int = SEG) -> float:
    """rel_err of the weight update dW = W_new - W_old against dW_want, with
    the one fp32 rounding of the stored weights taken out. W_new is
    fl32(W_old + dW): it is off the exact sum by up to half an ulp of W_new,
    which for |W| near 0.1 and |dW| near 1e-3 is already 1e-5 of dW, the
    whole fp32 bar. Each element's error is reduced by that half ulp (never
    below zero) before the pieces are measured, so the figure is the error of
    the update itself, understated by at most half an ulp per element."""
    Wn = np.asarray(W_new, np.float32)
    got = Wn.astype(np.float64) - np.asarray(W_old, np.float64)
    want = np.asarray(dW_want, np.float64)
    half = 0.5 * np.spacing(np.abs(Wn)).astype(np.float64)
    diff = got - want
    return rel_err(want + np.sign(diff) * np.maximum(np.abs(diff) - half, 0.0),
                   want, width)


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
