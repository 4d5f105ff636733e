"""The streaming form of the DP-GRAPE step, driven by autograd.

"Memory-Efficient Differentially Private Training with Gradient Random
Projection" (technical summary, Methodology, closing paragraph): the
per-sample gradients are projected layer by layer during the backward pass,
then aggregated, clipped and noised, and a projected Adam rule updates the
parameters.

Each ProjectedLinear keeps its input A from the forward pass. When autograd
produces the gradient dY of the layer's output, GrapeOptimizer projects that
layer's per-sample gradients at once (dpg_project_layer: the projections go
to a [B, r, d_out] fp32 buffer and the squared norms into a per-sample sum)
and drops its reference to A. After backward, GrapeOptimizer.step() clips,
sums and noises the stored projections (dpg_clip_sum_noise) and runs the
projected Adam update with the back-projection into every layer's W
(dpg_adam_backproject). All of it runs in libdpg's kernels; this module only
wires tensors to those calls.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import torch

from . import binding as _b


class ProjectedLinear(torch.nn.Module):
    """y = x W with W of shape [d_in, d_out] kept in fp32, the layout the
    update call writes in place. The product runs in the input's dtype. W is
    a buffer, not a parameter: it gets no gradient of its own, since the
    private update replaces the plain gradient step."""

    def __init__(self, d_in: int, d_out: int, layer_id: int,
                 W: Optional[torch.Tensor] = None, device="cuda"):
        super().__init__()
        if W is None:
            W = torch.randn(d_in, d_out, device=device) / math.sqrt(d_in)
        if tuple(W.shape) != (d_in, d_out):
            raise ValueError("W must be [d_in, d_out]")
        self.register_buffer("W", W.detach().to(torch.float32).contiguous())
        self.layer_id = int(layer_id)
        self._grape = None  # the GrapeOptimizer driving this layer, if any

    @property
    def d_in(self) -> int:
        return int(self.W.shape[0])

    @property
    def d_out(self) -> int:
        return int(self.W.shape[1])

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        y = x @ self.W.to(x.dtype)
        if self._grape is not None and torch.is_grad_enabled() and y.requires_grad:
            self._grape._capture(self, x, y)
        return y


class GrapeOptimizer:
    """Private update of a set of ProjectedLinear layers in the streaming form.

    Usage per step:
        opt.zero_grad()            # starts the step (resets the norm sums)
        loss = f(model(x)); loss.backward()   # layers are projected as
                                              # their dY appear
        opt.step()                 # clip, sum, noise, Adam, back-project
    The inputs of every layer are [B, T, d] in bf16 or fp32; the output of
    the first projected layer must require grad (for instance x.requires_grad_
    on the model input) so that autograd reaches every layer.
    proj_step = step when proj_period = 1, else (step - 1) // proj_period + 1
    (P then changes every proj_period steps)."""

    def __init__(self, layers: Sequence[ProjectedLinear], r: int, clip_C: float,
                 sigma: float, seed: int, lr: float, beta1: float = 0.9,
                 beta2: float = 0.999, eps: float = 1e-8, proj_period: int = 1,
                 keep_inputs: bool = False):
        self.layers: List[ProjectedLinear] = list(layers)
        ids = [l.layer_id for l in self.layers]
        if len(set(ids)) != len(ids):
            raise ValueError("layer ids must be unique")
        self.r, self.clip_C, self.sigma, self.seed = int(r), clip_C, sigma, int(seed)
        self.lr, self.beta1, self.beta2, self.eps = lr, beta1, beta2, eps
        self.proj_period = int(proj_period)
        self.keep_inputs = keep_inputs
        dev = self.layers[0].W.device
        self.m = [torch.zeros((self.r, l.d_out), device=dev) for l in self.layers]
        self.v = [torch.zeros((self.r, l.d_out), device=dev) for l in self.layers]
        self.t = 0
        self.norm_sq: Optional[torch.Tensor] = None
        self.G_hat: Dict[int, torch.Tensor] = {}  # layer id -> [B, r, d_out], reused
        self._done: set = set()                   # layers projected this step
        self.inputs: Dict[int, tuple] = {}  # layer id -> (A, dY) when keep_inputs
        self.dtype: Optional[torch.dtype] = None
        self.last_norms: Optional[torch.Tensor] = None
        self.last_G_priv: Optional[List[torch.Tensor]] = None
        for l in self.layers:
            l._grape = self

    @property
    def proj_step(self) -> int:
        return (self.t - 1) // self.proj_period + 1

    def zero_grad(self) -> None:
        self.t += 1
        self._done.clear()
        self.inputs.clear()
        if self.norm_sq is not None:
            self.norm_sq.zero_()

    def _capture(self, layer: ProjectedLinear, x: torch.Tensor, y: torch.Tensor):
        if self.t == 0:
            raise RuntimeError("call zero_grad() before the forward pass of a step")
        A = x.detach().contiguous()
        B = int(A.shape[0])
        if self.norm_sq is None or int(self.norm_sq.shape[0]) != B:
            self.norm_sq = torch.zeros(B, dtype=torch.float32, device=A.device)
        if self.dtype is None:
            self.dtype = A.dtype

        def on_grad(g: torch.Tensor):
            if layer.layer_id in self._done:
                raise RuntimeError(f"layer {layer.layer_id} ran twice in one step")
            dY = g.detach().contiguous()
            buf = self.G_hat.get(layer.layer_id)
            if buf is not None and tuple(buf.shape) != (B, self.r, layer.d_out):
                buf = None
            self.G_hat[layer.layer_id] = _b.dpg_project_layer(
                A, dY, self.r, self.seed, self.proj_step, layer.layer_id,
                self.norm_sq, G_hat=buf)
            self._done.add(layer.layer_id)
            if self.keep_inputs:
                self.inputs[layer.layer_id] = (A, dY)
            return None

        y.register_hook(on_grad)

    def step(self) -> None:
        missing = [l.layer_id for l in self.layers if l.layer_id not in self._done]
        if missing:
            raise RuntimeError(f"no gradient reached layers {missing}")
        ids = [l.layer_id for l in self.layers]
        G_priv, norms = _b.dpg_clip_sum_noise(
            [self.G_hat[i] for i in ids], self.r, self.clip_C, self.sigma,
            self.seed, self.t, self.norm_sq, layer_ids=ids)
        _b.dpg_adam_backproject(G_priv, [l.W for l in self.layers], self.m, self.v,
                                self.r, self.lr, self.beta1, self.beta2, self.eps,
                                self.seed, self.t, self.proj_step, layer_ids=ids,
                                dtype=self.dtype or torch.bfloat16)
        self.last_norms, self.last_G_priv = norms, G_priv
