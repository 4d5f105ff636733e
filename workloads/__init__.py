"""Seeded synthetic workloads for the DP-GRAPE private update step.

This module only describes shapes and draws seeded random inputs. It holds
none of the method's arithmetic (no projection, norm, clip, noise or Adam),
so both the CPU oracle's tests and the GPU path may take their inputs from it.

Shapes and value distributions follow the five synthetic workloads of the
DP-GRAPE step (the pages name ViT, RoBERTa and OPT models and MNIST/CIFAR/SST-2
data; those are not available, and these Gaussian / Student-t tensors stand in
for one step's layer activations A and output gradients dY):

  tiny      one 64x64 layer, B=8, T=16, r=8, fp32, A~N(0,1), dY~N(0,1/T)
  mlp4      768->3072->768->3072->768 (4 layers), B=32, T=128, r=128, bf16
  enc12     12 blocks x [q,k,v,o 768x768, up 768->3072, down 3072->768],
            B=64, T=256, r=256, bf16
  dec24     24 blocks x [q,k,v,o 2048^2, up 2048->8192, down 8192->2048],
            B=16, T=512, r=512, bf16, dY Student-t(3) / sqrt(T*d_out)
  long1     1 block x [q,k,v,o 4096^2, up 4096->11008, down 11008->4096],
            B=4, T=4096, r=256, bf16, C=0.5, sigma=1.2

A ~ N(0, 1/d_in) and dY ~ N(0, 1/(T*d_out)) for the bf16 workloads. W starts
as N(0, 1/d_in) in fp32 and the Adam moments start at zero.

Random draws use numpy's PCG64 seeded with [workload index, layer id,
tensor id] (tensor id 0 = A, 1 = dY, 2 = W), so any one layer can be
regenerated on its own. bf16 values are produced from fp32 draws by
round-to-nearest-even on the bit pattern; the exact bf16 values (upcast) are
what the oracle reads.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

__all__ = [
    "Layer", "Workload", "WORKLOADS", "workload", "custom_workload",
    "bf16_bits_from_f32", "f32_from_bf16_bits", "layer_inputs",
    "initial_state",
]


@dataclasses.dataclass(frozen=True)
class Layer:
    """One linear layer y = x W with W of shape [d_in, d_out]."""
    d_in: int
    d_out: int
    layer_id: int
    name: str = ""


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int              # first word of the PCG64 seed sequence
    layers: tuple
    B: int
    T: int
    r: int
    dtype: str              # "fp32" or "bf16": element type of A and dY
    a_kind: str             # "unit" -> N(0,1); "fan_in" -> N(0,1/d_in)
    dy_kind: str            # "inv_T" -> N(0,1/T); "inv_Tdout" -> N(0,1/(T d_out));
                            # "t3_inv_Tdout" -> Student-t(3)/sqrt(T d_out)
    clip_C: float
    sigma: float
    seed: int = 0
    step: int = 1
    proj_step: int = 1
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8

    @property
    def n_layers(self) -> int:
        return len(self.layers)

    def sum_din(self) -> int:
        return sum(l.d_in for l in self.layers)

    def sum_dout(self) -> int:
        return sum(l.d_out for l in self.layers)

    def n_params(self) -> int:
        return sum(l.d_in * l.d_out for l in self.layers)


def _blocks(n_blocks: int, d: int, d_ff: int) -> tuple:
    out = []
    names = ("q", "k", "v", "o", "up", "down")
    for b in range(n_blocks):
        shapes = [(d, d)] * 4 + [(d, d_ff), (d_ff, d)]
        for j, (di, do) in enumerate(shapes):
            out.append(Layer(di, do, 6 * b + j, f"blk{b}.{names[j]}"))
    return tuple(out)


WORKLOADS = {
    "tiny": Workload("tiny", 1, (Layer(64, 64, 0, "fc"),), B=8, T=16, r=8,
                     dtype="fp32", a_kind="unit", dy_kind="inv_T",
                     clip_C=1.0, sigma=1.0),
    "mlp4": Workload("mlp4", 2,
                     tuple(Layer(a, b, i, f"fc{i}") for i, (a, b) in enumerate(
                         [(768, 3072), (3072, 768), (768, 3072), (3072, 768)])),
                     B=32, T=128, r=128, dtype="bf16", a_kind="fan_in",
                     dy_kind="inv_Tdout", clip_C=1.0, sigma=0.8),
    "enc12": Workload("enc12", 3, _blocks(12, 768, 3072), B=64, T=256, r=256,
                      dtype="bf16", a_kind="fan_in", dy_kind="inv_Tdout",
                      clip_C=1.0, sigma=0.8),
    "dec24": Workload("dec24", 4, _blocks(24, 2048, 8192), B=16, T=512, r=512,
                      dtype="bf16", a_kind="fan_in", dy_kind="t3_inv_Tdout",
                      clip_C=1.0, sigma=0.8),
    "long1": Workload("long1", 5,
                      tuple(Layer(a, b, j, n) for j, (a, b, n) in enumerate(
                          [(4096, 4096, "q"), (4096, 4096, "k"),
                           (4096, 4096, "v"), (4096, 4096, "o"),
                           (4096, 11008, "up"), (11008, 4096, "down")])),
                      B=4, T=4096, r=256, dtype="bf16", a_kind="fan_in",
                      dy_kind="inv_Tdout", clip_C=0.5, sigma=1.2),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def custom_workload(name: str, index: int, shapes, B: int, T: int, r: int,
                    dtype: str = "bf16", a_kind: str = "fan_in",
                    dy_kind: str = "inv_Tdout", clip_C: float = 1.0,
                    sigma: float = 0.8, layer_ids: Optional[List[int]] = None,
                    **kw) -> Workload:
    """A workload of arbitrary layer shapes (parity cases, edge cases)."""
    ids = layer_ids if layer_ids is not None else list(range(len(shapes)))
    layers = tuple(Layer(int(a), int(b), int(i), f"l{i}")
                   for (a, b), i in zip(shapes, ids))
    return Workload(name, index, layers, B=B, T=T, r=r, dtype=dtype,
                    a_kind=a_kind, dy_kind=dy_kind, clip_C=clip_C,
                    sigma=sigma, **kw)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Inputs are finite draws, so no NaN handling is needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _rng(wl: Workload, layer_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([wl.index, layer_id, tensor_id])


def _draw_A(wl: Workload, layer: Layer) -> np.ndarray:
    g = _rng(wl, layer.layer_id, 0)
    x = g.standard_normal((wl.B, wl.T, layer.d_in), dtype=np.float32)
    if wl.a_kind == "fan_in":
        x *= np.float32(1.0 / np.sqrt(layer.d_in))
    elif wl.a_kind != "unit":
        raise ValueError(wl.a_kind)
    return x


def _draw_dY(wl: Workload, layer: Layer) -> np.ndarray:
    g = _rng(wl, layer.layer_id, 1)
    shape = (wl.B, wl.T, layer.d_out)
    if wl.dy_kind == "inv_T":
        x = g.standard_normal(shape, dtype=np.float32)
        x *= np.float32(1.0 / np.sqrt(wl.T))
    elif wl.dy_kind == "inv_Tdout":
        x = g.standard_normal(shape, dtype=np.float32)
        x *= np.float32(1.0 / np.sqrt(wl.T * layer.d_out))
    elif wl.dy_kind == "t3_inv_Tdout":
        x = g.standard_t(3.0, size=shape).astype(np.float32)
        x *= np.float32(1.0 / np.sqrt(wl.T * layer.d_out))
    else:
        raise ValueError(wl.dy_kind)
    return x


def layer_inputs(wl: Workload, layer: Layer):
    """(A, dY) for one layer in the workload's element type.

    fp32 workloads return float32 arrays; bf16 workloads return uint16 bf16
    bit patterns (use f32_from_bf16_bits for the exact values)."""
    A, dY = _draw_A(wl, layer), _draw_dY(wl, layer)
    if wl.dtype == "fp32":
        return A, dY
    if wl.dtype == "bf16":
        return bf16_bits_from_f32(A), bf16_bits_from_f32(dY)
    raise ValueError(wl.dtype)


def initial_state(wl: Workload, layer: Layer):
    """(W, m, v) before the first step: W ~ N(0, 1/d_in) fp32, m = v = 0."""
    g = _rng(wl, layer.layer_id, 2)
    W = g.standard_normal((layer.d_in, layer.d_out), dtype=np.float32)
    W *= np.float32(1.0 / np.sqrt(layer.d_in))
    m = np.zeros((wl.r, layer.d_out), dtype=np.float32)
    v = np.zeros((wl.r, layer.d_out), dtype=np.float32)
    return W, m, v


def as_float64(wl: Workload, x: np.ndarray) -> np.ndarray:
    """Exact float64 values of an input array of the workload's dtype."""
    if wl.dtype == "bf16":
        return f32_from_bf16_bits(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# ------------------------------------------------ draws in device memory --
#
# The large workloads (enc12, dec24, long1: 2 to 15 GB of A and dY) are drawn
# directly in device memory with torch's seeded generator, since drawing them
# on the host takes minutes. The values differ from the host draws above (a
# different generator) but follow the same distributions; checks read host
# copies of the slices they need. Seeds: (index << 40) | (layer id << 8) |
# tensor id.

def _device_gen(wl: Workload, layer_id: int, tensor_id: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((wl.index << 40) | (int(layer_id) << 8) | tensor_id)
    return g


def device_layer_inputs(wl: Workload, layer: Layer, device="cuda"):
    """(A, dY) for one layer as torch tensors on `device`, in the workload's
    element type (fp32 draws, rounded to bf16 by torch's round-to-nearest-even
    conversion for bf16 workloads)."""
    import torch
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    f32 = torch.float32
    gA = _device_gen(wl, layer.layer_id, 0, device)
    A = torch.randn((wl.B, wl.T, layer.d_in), generator=gA, device=device, dtype=f32)
    if wl.a_kind == "fan_in":
        A.mul_(1.0 / np.sqrt(layer.d_in))
    elif wl.a_kind != "unit":
        raise ValueError(wl.a_kind)
    gD = _device_gen(wl, layer.layer_id, 1, device)
    shape = (wl.B, wl.T, layer.d_out)
    if wl.dy_kind == "inv_T":
        dY = torch.randn(shape, generator=gD, device=device, dtype=f32)
        dY.mul_(1.0 / np.sqrt(wl.T))
    elif wl.dy_kind == "inv_Tdout":
        dY = torch.randn(shape, generator=gD, device=device, dtype=f32)
        dY.mul_(1.0 / np.sqrt(wl.T * layer.d_out))
    elif wl.dy_kind == "t3_inv_Tdout":
        # Student-t with 3 degrees of freedom: z / sqrt(chi2_3 / 3)
        dY = torch.randn(shape, generator=gD, device=device, dtype=f32)
        chi2 = torch.zeros(shape, device=device, dtype=f32)
        for _ in range(3):
            c = torch.randn(shape, generator=gD, device=device, dtype=f32)
            chi2.addcmul_(c, c)
        dY.div_(torch.sqrt(chi2 / 3.0))
        dY.mul_(1.0 / np.sqrt(wl.T * layer.d_out))
    else:
        raise ValueError(wl.dy_kind)
    return A.to(dt), dY.to(dt)


def device_initial_state(wl: Workload, layer: Layer, device="cuda"):
    """(W, m, v) on `device`: W ~ N(0, 1/d_in) fp32, m = v = 0."""
    import torch
    g = _device_gen(wl, layer.layer_id, 2, device)
    W = torch.randn((layer.d_in, layer.d_out), generator=g, device=device,
                    dtype=torch.float32)
    W.mul_(1.0 / np.sqrt(layer.d_in))
    m = torch.zeros((wl.r, layer.d_out), device=device, dtype=torch.float32)
    v = torch.zeros_like(m)
    return W, m, v
