"""ctypes binding of libdpg.so (include/dpg.h): argument marshalling only.

Every step of the DP-GRAPE update runs in the library's HIP kernels; this
module turns torch tensors into device pointers and the current HIP stream,
and allocates outputs and workspaces with torch when the caller does not pass
them. It never computes any part of the method itself, and it raises when the
library has not been built.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import math
import os
from typing import List, Optional, Sequence

import torch  # loaded first: libdpg.so then shares torch's HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdpg.so")

DPG_OK = 0
DPG_ERR_INVALID_ARG = 1
DPG_ERR_WORKSPACE = 2
DPG_ERR_UNSUPPORTED = 3
DPG_ERR_HIP = 4
DPG_FP32 = 0
DPG_BF16 = 1

EXPORTED = (
    "dpg_project_workspace_size", "dpg_project_clip_noise",
    "dpg_adam_workspace_size", "dpg_adam_backproject", "dpg_philox_normals",
    "dpg_project_layer_workspace_size", "dpg_project_layer",
    "dpg_clip_workspace_size", "dpg_clip_sum_noise",
    "dpg_step_workspace_size", "dpg_private_step", "dpg_private_step_static",
    "dpg_static_scratch_bytes", "dpg_rc_norms_workspace_size", "dpg_rc_norms",
    "dpg_status_string", "dpg_last_error", "dpg_version",
    "dpg_timing_enable", "dpg_timing_read", "dpg_kernel_name",
)
N_KERNEL_KINDS = 10


class DpgError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class LayerGrad(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_int64), ("d_out", ctypes.c_int64),
                ("layer_id", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("A", ctypes.c_void_p), ("dY", ctypes.c_void_p),
                ("G_priv", ctypes.c_void_p)]


class LayerHat(ctypes.Structure):
    _fields_ = [("d_out", ctypes.c_int64), ("layer_id", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32), ("G_hat", ctypes.c_void_p),
                ("G_priv", ctypes.c_void_p)]


class LayerParam(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_int64), ("d_out", ctypes.c_int64),
                ("layer_id", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("G_priv", ctypes.c_void_p), ("W", ctypes.c_void_p),
                ("m", ctypes.c_void_p), ("v", ctypes.c_void_p)]


_lib = None


def library_path() -> str:
    return LIB_PATH


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libdpg.so (once). Raises FileNotFoundError when it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} is missing: build it with `python -m dp_grape_projection_amd.build`")
    lib = ctypes.CDLL(p)
    i32, i64, u32, u64 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                          ctypes.c_uint64)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.dpg_project_workspace_size.argtypes = [
        ctypes.POINTER(LayerGrad), i32, i64, i64, i32, i32, ctypes.POINTER(sz)]
    f64 = ctypes.c_double
    lib.dpg_project_clip_noise.argtypes = [
        ctypes.POINTER(LayerGrad), i32, i64, i64, i32, i32, f64, f64, u64,
        u64, u64, vp, vp, sz, vp]
    lib.dpg_rc_norms_workspace_size.argtypes = [
        ctypes.POINTER(LayerGrad), i32, i64, i64, i32, i32, ctypes.POINTER(sz)]
    lib.dpg_rc_norms.argtypes = [
        ctypes.POINTER(LayerGrad), i32, i64, i64, i32, i32, f64, u64, u64, vp, vp,
        vp, sz, vp]
    lib.dpg_adam_workspace_size.argtypes = [
        ctypes.POINTER(LayerParam), i32, i32, i32, ctypes.POINTER(sz)]
    lib.dpg_adam_backproject.argtypes = [
        ctypes.POINTER(LayerParam), i32, i32, i32, f64, f64, f64, f64, u64,
        u64, u64, vp, sz, vp]
    lib.dpg_philox_normals.argtypes = [u64, u32, u32, u32, u64, u64, vp, vp, vp]
    lib.dpg_project_layer_workspace_size.argtypes = [
        ctypes.POINTER(LayerGrad), i64, i64, i32, i32, ctypes.POINTER(sz)]
    lib.dpg_project_layer.argtypes = [
        ctypes.POINTER(LayerGrad), i64, i64, i32, i32, u64, u64, vp, vp, vp, sz, vp]
    lib.dpg_clip_workspace_size.argtypes = [i64, ctypes.POINTER(sz)]
    lib.dpg_step_workspace_size.argtypes = [
        ctypes.POINTER(LayerGrad), i32, i64, i64, i32, i32, ctypes.POINTER(sz)]
    lib.dpg_private_step.argtypes = [
        ctypes.POINTER(LayerGrad), ctypes.POINTER(LayerParam), i32, i64, i64, i32,
        i32, f64, f64, f64, f64, f64, f64, u64, u64, u64, vp, vp, sz, vp]
    lib.dpg_private_step_static.argtypes = [
        ctypes.POINTER(LayerGrad), ctypes.POINTER(LayerParam), i32, i64, i64, i32,
        i32, f64, f64, f64, f64, f64, f64, u64, u64, u64, vp, vp]
    lib.dpg_static_scratch_bytes.argtypes = []
    lib.dpg_clip_sum_noise.argtypes = [
        ctypes.POINTER(LayerHat), i32, i64, i32, f64, f64, u64, u64, vp, vp, vp,
        sz, vp]
    for name in EXPORTED:
        getattr(lib, name).restype = ctypes.c_int
    lib.dpg_static_scratch_bytes.restype = ctypes.c_size_t
    lib.dpg_status_string.restype = ctypes.c_char_p
    lib.dpg_status_string.argtypes = [ctypes.c_int]
    lib.dpg_last_error.restype = ctypes.c_char_p
    lib.dpg_last_error.argtypes = []
    lib.dpg_timing_enable.argtypes = [ctypes.c_int]
    lib.dpg_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int64), i32,
                                    ctypes.c_int]
    lib.dpg_kernel_name.restype = ctypes.c_char_p
    lib.dpg_kernel_name.argtypes = [ctypes.c_int]
    if path is None:
        _lib = lib
    return lib


def _check(lib, status: int):
    if status != DPG_OK:
        msg = lib.dpg_last_error().decode() or lib.dpg_status_string(status).decode()
        raise DpgError(status, msg)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return DPG_BF16
    if t == torch.float32:
        return DPG_FP32
    raise TypeError(f"A/dY must be bfloat16 or float32, got {t}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _on_stream(fn):
    """Runs `fn` with its `stream` argument (when given) as torch's current
    stream, so that the outputs and temporary workspaces it allocates belong
    to the stream the library's kernels are enqueued on: the caching
    allocator then does not hand their memory to other work while those
    kernels may still use it."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kw):
        stream = sig.bind(*args, **kw).arguments.get("stream")
        if stream is None:
            return fn(*args, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, **kw)
    return wrapper


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if workspace is not None:
        _require(workspace, "workspace", torch.uint8)
        return workspace, workspace.numel()
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device), nbytes


def project_workspace_size(shapes: Sequence, B: int, T: int, r: int,
                           dtype: torch.dtype,
                           layer_ids: Optional[Sequence[int]] = None) -> int:
    """Workspace bytes dpg_project_clip_noise needs; shapes = [(d_in, d_out)]."""
    lib = load_library()
    n = len(shapes)
    ids = list(range(n)) if layer_ids is None else list(layer_ids)
    arr = (LayerGrad * n)()
    for i, ((di, do), lid) in enumerate(zip(shapes, ids)):
        arr[i].d_in, arr[i].d_out, arr[i].layer_id = int(di), int(do), int(lid)
    out = ctypes.c_size_t(0)
    _check(lib, lib.dpg_project_workspace_size(arr, n, int(B), int(T), int(r),
                                               _dtype_code(dtype),
                                               ctypes.byref(out)))
    return out.value


def adam_workspace_size(shapes: Sequence, r: int, dtype: torch.dtype,
                        layer_ids: Optional[Sequence[int]] = None) -> int:
    lib = load_library()
    n = len(shapes)
    ids = list(range(n)) if layer_ids is None else list(layer_ids)
    arr = (LayerParam * n)()
    for i, ((di, do), lid) in enumerate(zip(shapes, ids)):
        arr[i].d_in, arr[i].d_out, arr[i].layer_id = int(di), int(do), int(lid)
    out = ctypes.c_size_t(0)
    _check(lib, lib.dpg_adam_workspace_size(arr, n, int(r), _dtype_code(dtype),
                                            ctypes.byref(out)))
    return out.value


@_on_stream
def dpg_project_clip_noise(A: Sequence[torch.Tensor], dY: Sequence[torch.Tensor],
                           r: int, clip_C: float, sigma: float, seed: int,
                           step: int, proj_step: Optional[int] = None,
                           layer_ids: Optional[Sequence[int]] = None,
                           G_priv: Optional[List[torch.Tensor]] = None,
                           sample_norms: Optional[torch.Tensor] = None,
                           return_norms: bool = True,
                           workspace: Optional[torch.Tensor] = None,
                           stream=None):
    """Projection, global per-sample clip, batch sum and noise (libdpg).

    A[l]: [B, T, d_in_l], dY[l]: [B, T, d_out_l] (bf16 or fp32, on the GPU).
    Returns (G_priv list of [r, d_out_l] fp32, sample norms [B] or None)."""
    lib = load_library()
    n = len(A)
    if n < 1 or len(dY) != n:
        raise ValueError("A and dY must be non-empty lists of equal length")
    dt = A[0].dtype
    B, T = int(A[0].shape[0]), int(A[0].shape[1])
    ids = list(range(n)) if layer_ids is None else [int(x) for x in layer_ids]
    proj_step = step if proj_step is None else proj_step
    dev = A[0].device
    if G_priv is None:
        G_priv = [torch.empty((r, int(d.shape[2])), dtype=torch.float32,
                              device=dev) for d in dY]
    if sample_norms is None and return_norms:
        sample_norms = torch.empty(B, dtype=torch.float32, device=dev)
    arr = (LayerGrad * n)()
    for i in range(n):
        _require(A[i], f"A[{i}]", dt)
        _require(dY[i], f"dY[{i}]", dt)
        if A[i].dim() != 3 or dY[i].dim() != 3 or \
                tuple(A[i].shape[:2]) != (B, T) or tuple(dY[i].shape[:2]) != (B, T):
            raise ValueError(f"layer {i}: A and dY must be [B, T, d] with common B, T")
        d_in, d_out = int(A[i].shape[2]), int(dY[i].shape[2])
        _require(G_priv[i], f"G_priv[{i}]", torch.float32, (r, d_out))
        arr[i].d_in, arr[i].d_out, arr[i].layer_id = d_in, d_out, ids[i]
        arr[i].A, arr[i].dY, arr[i].G_priv = _ptr(A[i]), _ptr(dY[i]), _ptr(G_priv[i])
    if sample_norms is not None:
        _require(sample_norms, "sample_norms", torch.float32, (B,))
    need = ctypes.c_size_t(0)
    _check(lib, lib.dpg_project_workspace_size(arr, n, B, T, int(r),
                                               _dtype_code(dt), ctypes.byref(need)))
    ws, ws_bytes = _workspace(need.value, dev, workspace)
    _check(lib, lib.dpg_project_clip_noise(
        arr, n, B, T, int(r), _dtype_code(dt), float(clip_C), float(sigma),
        int(seed), int(step), int(proj_step), _ptr(sample_norms),
        ws.data_ptr(), ws_bytes, _stream_handle(stream)))
    return G_priv, sample_norms


@_on_stream
def dpg_adam_backproject(G_priv: Sequence[torch.Tensor], W: Sequence[torch.Tensor],
                         m: Sequence[torch.Tensor], v: Sequence[torch.Tensor],
                         r: int, lr: float, beta1: float, beta2: float,
                         eps: float, seed: int, step: int,
                         proj_step: Optional[int] = None,
                         layer_ids: Optional[Sequence[int]] = None,
                         dtype: torch.dtype = torch.bfloat16,
                         workspace: Optional[torch.Tensor] = None, stream=None):
    """Projected Adam and back-projection W -= lr P^T U, in place (libdpg).

    dtype is the operand precision of P^T U (bf16 or fp32)."""
    lib = load_library()
    n = len(W)
    ids = list(range(n)) if layer_ids is None else [int(x) for x in layer_ids]
    proj_step = step if proj_step is None else proj_step
    arr = (LayerParam * n)()
    for i in range(n):
        _require(W[i], f"W[{i}]", torch.float32)
        if W[i].dim() != 2:
            raise ValueError(f"W[{i}] must be [d_in, d_out]")
        d_in, d_out = int(W[i].shape[0]), int(W[i].shape[1])
        for name, t in (("G_priv", G_priv[i]), ("m", m[i]), ("v", v[i])):
            _require(t, f"{name}[{i}]", torch.float32, (r, d_out))
        arr[i].d_in, arr[i].d_out, arr[i].layer_id = d_in, d_out, ids[i]
        arr[i].G_priv, arr[i].W = _ptr(G_priv[i]), _ptr(W[i])
        arr[i].m, arr[i].v = _ptr(m[i]), _ptr(v[i])
    code = _dtype_code(dtype)
    need = ctypes.c_size_t(0)
    _check(lib, lib.dpg_adam_workspace_size(arr, n, int(r), code, ctypes.byref(need)))
    ws, ws_bytes = _workspace(need.value, W[0].device, workspace)
    _check(lib, lib.dpg_adam_backproject(
        arr, n, int(r), code, float(lr), float(beta1), float(beta2), float(eps),
        int(seed), int(step), int(proj_step), ws.data_ptr(), ws_bytes,
        _stream_handle(stream)))
    return W, m, v


@_on_stream
def dpg_private_step(A: Sequence[torch.Tensor], dY: Sequence[torch.Tensor],
                     W: Sequence[torch.Tensor], m: Sequence[torch.Tensor],
                     v: Sequence[torch.Tensor], r: int, clip_C: float, sigma: float,
                     lr: float, beta1: float, beta2: float, eps: float, seed: int,
                     step: int, proj_step: Optional[int] = None,
                     layer_ids: Optional[Sequence[int]] = None, stream=None):
    """The whole step in one call (libdpg): W, m, v updated in place.
    Returns (G_priv list of [r, d_out] fp32, sample norms [B])."""
    ps = PreparedStep(A, dY, W, m, v, r, clip_C, sigma, seed, lr, beta1, beta2,
                      eps, layer_ids=layer_ids)
    proj_step = step if proj_step is None else proj_step
    _check(ps.lib, ps.lib.dpg_private_step(
        ps.grads, ps.params, ps.n, ps.B, ps.T, ps.r, ps.dtype_code, float(clip_C),
        float(sigma), float(lr), float(beta1), float(beta2), float(eps), int(seed),
        int(step), int(proj_step), ps.sample_norms.data_ptr(), ps.ws3.data_ptr(),
        ps.ws3_bytes, _stream_handle(stream)))
    return ps.G_priv, ps.sample_norms


@_on_stream
def dpg_rc_norms(A: Sequence[torch.Tensor], dY: Sequence[torch.Tensor], k: int,
                 clip_C: float, seed: int, step: int,
                 layer_ids: Optional[Sequence[int]] = None,
                 norms: Optional[torch.Tensor] = None,
                 scales: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None):
    """Randomized clipping's per-sample norm estimate (libdpg): Hutchinson's
    estimator with k Gaussian probes per layer on the d_out side.
    A[l]: [B, T, d_in_l], dY[l]: [B, T, d_out_l] (bf16 or fp32, on the GPU).
    Returns (estimated norms [B], clip factors min(1, C / nhat) [B])."""
    lib = load_library()
    n = len(A)
    if n < 1 or len(dY) != n:
        raise ValueError("A and dY must be non-empty lists of equal length")
    dt = A[0].dtype
    B, T = int(A[0].shape[0]), int(A[0].shape[1])
    ids = list(range(n)) if layer_ids is None else [int(x) for x in layer_ids]
    dev = A[0].device
    norms = torch.empty(B, dtype=torch.float32, device=dev) if norms is None else norms
    scales = torch.empty(B, dtype=torch.float32, device=dev) if scales is None else scales
    _require(norms, "norms", torch.float32, (B,))
    _require(scales, "scales", torch.float32, (B,))
    arr = (LayerGrad * n)()
    for i in range(n):
        _require(A[i], f"A[{i}]", dt)
        _require(dY[i], f"dY[{i}]", dt)
        if A[i].dim() != 3 or dY[i].dim() != 3 or \
                tuple(A[i].shape[:2]) != (B, T) or tuple(dY[i].shape[:2]) != (B, T):
            raise ValueError(f"layer {i}: A and dY must be [B, T, d] with common B, T")
        arr[i].d_in, arr[i].d_out, arr[i].layer_id = int(A[i].shape[2]), int(dY[i].shape[2]), ids[i]
        arr[i].A, arr[i].dY, arr[i].G_priv = _ptr(A[i]), _ptr(dY[i]), None
    need = ctypes.c_size_t(0)
    _check(lib, lib.dpg_rc_norms_workspace_size(arr, n, B, T, int(k), _dtype_code(dt),
                                                ctypes.byref(need)))
    ws, ws_bytes = _workspace(need.value, dev, workspace)
    _check(lib, lib.dpg_rc_norms(arr, n, B, T, int(k), _dtype_code(dt), float(clip_C),
                                 int(seed), int(step), norms.data_ptr(), scales.data_ptr(),
                                 ws.data_ptr(), ws_bytes, _stream_handle(stream)))
    return norms, scales


def static_scratch_bytes() -> int:
    """Bytes of the library's static scratch (per GPU)."""
    return int(load_library().dpg_static_scratch_bytes())


@_on_stream
def dpg_private_step_static(A: Sequence[torch.Tensor], dY: Sequence[torch.Tensor],
                            W: Sequence[torch.Tensor], m: Sequence[torch.Tensor],
                            v: Sequence[torch.Tensor], G_priv: Sequence[torch.Tensor],
                            sample_norms: torch.Tensor, r: int, clip_C: float,
                            sigma: float, lr: float, beta1: float, beta2: float,
                            eps: float, seed: int, step: int,
                            proj_step: Optional[int] = None,
                            layer_ids: Optional[Sequence[int]] = None, stream=None):
    """The one-call step in the library's static scratch (libdpg
    dpg_private_step_static): nothing is allocated, here or in the library;
    the caller passes every output (G_priv [r, d_out] fp32 per layer,
    sample_norms [B] fp32). W, m, v are updated in place."""
    lib = load_library()
    grads, params, n, B, T, code = _step_tables(A, dY, W, m, v, G_priv, r, layer_ids)
    _require(sample_norms, "sample_norms", torch.float32, (B,))
    proj_step = step if proj_step is None else proj_step
    _check(lib, lib.dpg_private_step_static(
        grads, params, n, B, T, int(r), code, float(clip_C), float(sigma), float(lr),
        float(beta1), float(beta2), float(eps), int(seed), int(step), int(proj_step),
        sample_norms.data_ptr(), _stream_handle(stream)))
    return G_priv, sample_norms


def _step_tables(A, dY, W, m, v, G_priv, r, layer_ids):
    """Checked layer tables (dpg_layer_grad, dpg_layer_param) of one step."""
    n = len(A)
    if n < 1 or not (len(dY) == len(W) == len(m) == len(v) == len(G_priv) == n):
        raise ValueError("A, dY, W, m, v and G_priv must be lists of equal length >= 1")
    dt = A[0].dtype
    B, T = int(A[0].shape[0]), int(A[0].shape[1])
    ids = list(range(n)) if layer_ids is None else [int(x) for x in layer_ids]
    grads, params = (LayerGrad * n)(), (LayerParam * n)()
    for i in range(n):
        _require(A[i], f"A[{i}]", dt)
        _require(dY[i], f"dY[{i}]", dt)
        if A[i].dim() != 3 or dY[i].dim() != 3 or \
                tuple(A[i].shape[:2]) != (B, T) or tuple(dY[i].shape[:2]) != (B, T):
            raise ValueError(f"layer {i}: A and dY must be [B, T, d] with common B, T")
        d_in, d_out = int(A[i].shape[2]), int(dY[i].shape[2])
        _require(W[i], f"W[{i}]", torch.float32, (d_in, d_out))
        for name, t in (("G_priv", G_priv[i]), ("m", m[i]), ("v", v[i])):
            _require(t, f"{name}[{i}]", torch.float32, (r, d_out))
        g, p = grads[i], params[i]
        g.d_in = p.d_in = d_in
        g.d_out = p.d_out = d_out
        g.layer_id = p.layer_id = ids[i]
        g.A, g.dY, g.G_priv = A[i].data_ptr(), dY[i].data_ptr(), G_priv[i].data_ptr()
        p.G_priv, p.W = G_priv[i].data_ptr(), W[i].data_ptr()
        p.m, p.v = m[i].data_ptr(), v[i].data_ptr()
    return grads, params, n, B, T, _dtype_code(dt)


@_on_stream
def dpg_project_layer(A: torch.Tensor, dY: torch.Tensor, r: int, seed: int,
                      proj_step: int, layer_id: int, norm_sq: torch.Tensor,
                      G_hat: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """Streaming form, one layer (libdpg): G_hat[i] = P A_i^T dY_i
    ([B, r, d_out] fp32) and norm_sq[i] += ||G_hat[i]||^2. Returns G_hat."""
    lib = load_library()
    dt = A.dtype
    _require(A, "A", dt)
    _require(dY, "dY", dt)
    if A.dim() != 3 or dY.dim() != 3 or tuple(A.shape[:2]) != tuple(dY.shape[:2]):
        raise ValueError("A and dY must be [B, T, d] with common B, T")
    B, T = int(A.shape[0]), int(A.shape[1])
    d_in, d_out = int(A.shape[2]), int(dY.shape[2])
    if G_hat is None:
        G_hat = torch.empty((B, r, d_out), dtype=torch.float32, device=A.device)
    _require(G_hat, "G_hat", torch.float32, (B, r, d_out))
    _require(norm_sq, "norm_sq", torch.float32, (B,))
    arr = (LayerGrad * 1)()
    arr[0].d_in, arr[0].d_out, arr[0].layer_id = d_in, d_out, int(layer_id)
    arr[0].A, arr[0].dY = _ptr(A), _ptr(dY)
    need = ctypes.c_size_t(0)
    _check(lib, lib.dpg_project_layer_workspace_size(arr, B, T, int(r), _dtype_code(dt),
                                                     ctypes.byref(need)))
    ws, ws_bytes = _workspace(need.value, A.device, workspace)
    _check(lib, lib.dpg_project_layer(arr, B, T, int(r), _dtype_code(dt), int(seed),
                                      int(proj_step), _ptr(G_hat), _ptr(norm_sq),
                                      ws.data_ptr(), ws_bytes, _stream_handle(stream)))
    return G_hat


@_on_stream
def dpg_clip_sum_noise(G_hat: Sequence[torch.Tensor], r: int, clip_C: float,
                       sigma: float, seed: int, step: int, norm_sq: torch.Tensor,
                       layer_ids: Optional[Sequence[int]] = None,
                       G_priv: Optional[List[torch.Tensor]] = None,
                       sample_norms: Optional[torch.Tensor] = None,
                       return_norms: bool = True,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """Streaming form, after the last layer (libdpg): G_priv_l =
    (sum_i s_i G_hat_l[i] + sigma C Z_l) / B with s_i from norm_sq.
    Returns (G_priv list of [r, d_out] fp32, sample norms [B] or None)."""
    lib = load_library()
    n = len(G_hat)
    if n < 1:
        raise ValueError("G_hat must be a non-empty list")
    B = int(G_hat[0].shape[0])
    dev = G_hat[0].device
    ids = list(range(n)) if layer_ids is None else [int(x) for x in layer_ids]
    if G_priv is None:
        G_priv = [torch.empty((r, int(g.shape[2])), dtype=torch.float32, device=dev)
                  for g in G_hat]
    if sample_norms is None and return_norms:
        sample_norms = torch.empty(B, dtype=torch.float32, device=dev)
    _require(norm_sq, "norm_sq", torch.float32, (B,))
    arr = (LayerHat * n)()
    for i in range(n):
        d_out = int(G_hat[i].shape[2])
        _require(G_hat[i], f"G_hat[{i}]", torch.float32, (B, r, d_out))
        _require(G_priv[i], f"G_priv[{i}]", torch.float32, (r, d_out))
        arr[i].d_out, arr[i].layer_id = d_out, ids[i]
        arr[i].G_hat, arr[i].G_priv = _ptr(G_hat[i]), _ptr(G_priv[i])
    if sample_norms is not None:
        _require(sample_norms, "sample_norms", torch.float32, (B,))
    need = ctypes.c_size_t(0)
    _check(lib, lib.dpg_clip_workspace_size(B, ctypes.byref(need)))
    ws, ws_bytes = _workspace(need.value, dev, workspace)
    _check(lib, lib.dpg_clip_sum_noise(arr, n, B, int(r), float(clip_C), float(sigma),
                                       int(seed), int(step), _ptr(norm_sq),
                                       _ptr(sample_norms), ws.data_ptr(), ws_bytes,
                                       _stream_handle(stream)))
    return G_priv, sample_norms


@_on_stream
def dpg_philox_normals(seed: int, layer_id: int, step_word: int, tag: int,
                       start: int, n: int, device="cuda", words: bool = False,
                       stream=None):
    """The library's random stream z(e), e in [start, start+n) (and raw words)."""
    lib = load_library()
    z = torch.empty(n, dtype=torch.float32, device=device)
    w = None
    if words and n > 0:
        n_ctr = ((start + n - 1) >> 2) - (start >> 2) + 1
        w = torch.empty(4 * n_ctr, dtype=torch.int32, device=device)
    _check(lib, lib.dpg_philox_normals(int(seed), int(layer_id), int(step_word),
                                       int(tag), int(start), int(n), _ptr(z),
                                       _ptr(w), _stream_handle(stream)))
    return (z, w) if words else z


class PreparedStep:
    """One DP-GRAPE step with its layer tables and workspaces marshalled
    once, for callers that repeat the step on the same buffers (a training
    loop, the bench): dpg_private_step, or with one_call=False the two calls
    dpg_project_clip_noise and dpg_adam_backproject.

    run(step) enqueues the step on the current stream with
    step = proj_step = `step`."""

    def __init__(self, A, dY, W, m, v, r, clip_C, sigma, seed, lr, beta1,
                 beta2, eps, layer_ids=None, G_priv=None, sample_norms=None,
                 one_call=True):
        self.lib = load_library()
        self.one_call = one_call
        n = len(A)
        dt = A[0].dtype
        self.dtype_code = _dtype_code(dt)
        self.B, self.T = int(A[0].shape[0]), int(A[0].shape[1])
        ids = list(range(n)) if layer_ids is None else [int(x) for x in layer_ids]
        dev = A[0].device
        self.G_priv = G_priv or [torch.empty((r, int(d.shape[2])),
                                             dtype=torch.float32, device=dev)
                                 for d in dY]
        self.sample_norms = (torch.empty(self.B, dtype=torch.float32, device=dev)
                             if sample_norms is None else sample_norms)
        self.grads, self.params, _, _, _, _ = _step_tables(A, dY, W, m, v, self.G_priv,
                                                           r, ids)
        self.n = n
        self.r = int(r)
        self.hyper = (float(clip_C), float(sigma), int(seed), float(lr),
                      float(beta1), float(beta2), float(eps))
        need1, need2 = ctypes.c_size_t(0), ctypes.c_size_t(0)
        _check(self.lib, self.lib.dpg_project_workspace_size(
            self.grads, n, self.B, self.T, self.r, self.dtype_code,
            ctypes.byref(need1)))
        _check(self.lib, self.lib.dpg_adam_workspace_size(
            self.params, n, self.r, self.dtype_code, ctypes.byref(need2)))
        self.ws1, self.ws1_bytes = _workspace(need1.value, dev, None)
        self.ws2, self.ws2_bytes = _workspace(need2.value, dev, None)
        need3 = ctypes.c_size_t(0)
        _check(self.lib, self.lib.dpg_step_workspace_size(
            self.grads, n, self.B, self.T, self.r, self.dtype_code,
            ctypes.byref(need3)))
        self.ws3, self.ws3_bytes = _workspace(need3.value if one_call else 0, dev, None)
        self._keep = (A, dY, W, m, v)

    def _buffers(self):
        return [self.sample_norms, self.ws1, self.ws2, self.ws3, *self.G_priv]

    def _mark_stream(self, stream) -> None:
        """Buffers allocated on the construction stream and used on another
        one are marked as in use there, so that freeing this object does not
        release them to other work before that stream reaches this point."""
        if stream is not None and stream != torch.cuda.current_stream():
            for t in self._buffers():
                t.record_stream(stream)

    def run(self, step: int, stream=None) -> None:
        C, sigma, seed, lr, b1, b2, eps = self.hyper
        h = _stream_handle(stream)
        lib = self.lib
        self._mark_stream(stream)
        if self.one_call:
            _check(lib, lib.dpg_private_step(
                self.grads, self.params, self.n, self.B, self.T, self.r,
                self.dtype_code, C, sigma, lr, b1, b2, eps, seed, step, step,
                self.sample_norms.data_ptr(), self.ws3.data_ptr(), self.ws3_bytes, h))
            return
        _check(lib, lib.dpg_project_clip_noise(
            self.grads, self.n, self.B, self.T, self.r, self.dtype_code, C,
            sigma, seed, step, step, self.sample_norms.data_ptr(),
            self.ws1.data_ptr(), self.ws1_bytes, h))
        _check(lib, lib.dpg_adam_backproject(
            self.params, self.n, self.r, self.dtype_code, lr, b1, b2, eps,
            seed, step, step, self.ws2.data_ptr(), self.ws2_bytes, h))


class PreparedStreamingStep(PreparedStep):
    """The same step in the streaming form: dpg_project_layer for each layer
    in order (stored projections [B, r, d_out] fp32, squared norms summed
    over the layers), then dpg_clip_sum_noise and dpg_adam_backproject, with
    every table, buffer and workspace marshalled once."""

    def __init__(self, A, dY, W, m, v, r, clip_C, sigma, seed, lr, beta1,
                 beta2, eps, layer_ids=None):
        super().__init__(A, dY, W, m, v, r, clip_C, sigma, seed, lr, beta1,
                         beta2, eps, layer_ids=layer_ids)
        dev = A[0].device
        self.norm_sq = torch.zeros(self.B, dtype=torch.float32, device=dev)
        self.G_hat = [torch.empty((self.B, self.r, int(d.shape[2])),
                                  dtype=torch.float32, device=dev) for d in dY]
        self.one = []
        need = 0
        for i in range(self.n):
            g = (LayerGrad * 1)()
            ctypes.memmove(ctypes.addressof(g), ctypes.addressof(self.grads[i]),
                           ctypes.sizeof(LayerGrad))
            self.one.append(g)
            b = ctypes.c_size_t(0)
            _check(self.lib, self.lib.dpg_project_layer_workspace_size(
                g, self.B, self.T, self.r, self.dtype_code, ctypes.byref(b)))
            need = max(need, b.value)
        self.wsl, self.wsl_bytes = _workspace(need, dev, None)
        b = ctypes.c_size_t(0)
        _check(self.lib, self.lib.dpg_clip_workspace_size(self.B, ctypes.byref(b)))
        self.wsc, self.wsc_bytes = _workspace(b.value, dev, None)
        self.hats = (LayerHat * self.n)()
        for i in range(self.n):
            h = self.hats[i]
            h.d_out, h.layer_id = self.grads[i].d_out, self.grads[i].layer_id
            h.G_hat, h.G_priv = self.G_hat[i].data_ptr(), self.G_priv[i].data_ptr()

    def _buffers(self):
        return super()._buffers() + [self.norm_sq, self.wsl, self.wsc, *self.G_hat]

    def run(self, step: int, stream=None) -> None:
        C, sigma, seed, lr, b1, b2, eps = self.hyper
        h = _stream_handle(stream)
        lib = self.lib
        self._mark_stream(stream)
        with torch.cuda.stream(stream) if stream is not None else _nullctx():
            self.norm_sq.zero_()
        for i in range(self.n):
            _check(lib, lib.dpg_project_layer(
                self.one[i], self.B, self.T, self.r, self.dtype_code, seed, step,
                self.G_hat[i].data_ptr(), self.norm_sq.data_ptr(),
                self.wsl.data_ptr(), self.wsl_bytes, h))
        _check(lib, lib.dpg_clip_sum_noise(
            self.hats, self.n, self.B, self.r, C, sigma, seed, step,
            self.norm_sq.data_ptr(), self.sample_norms.data_ptr(),
            self.wsc.data_ptr(), self.wsc_bytes, h))
        _check(lib, lib.dpg_adam_backproject(
            self.params, self.n, self.r, self.dtype_code, lr, b1, b2, eps,
            seed, step, step, self.ws2.data_ptr(), self.ws2_bytes, h))


class _nullctx:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def timing_enable(on: bool = True) -> None:
    """Bracket every kernel launch of the two step calls with HIP events."""
    lib = load_library()
    _check(lib, lib.dpg_timing_enable(1 if on else 0))


def timing_read(reset: bool = True) -> dict:
    """{kernel name: (total ms, launches)} since the last reset."""
    lib = load_library()
    ms = (ctypes.c_double * N_KERNEL_KINDS)()
    cnt = (ctypes.c_int64 * N_KERNEL_KINDS)()
    _check(lib, lib.dpg_timing_read(ms, cnt, N_KERNEL_KINDS, 1 if reset else 0))
    return {lib.dpg_kernel_name(k).decode(): (ms[k], cnt[k])
            for k in range(N_KERNEL_KINDS)}


def version() -> int:
    return load_library().dpg_version()
