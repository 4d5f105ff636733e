"""The C-ABI library on the host (no GPU): it loads, exports every symbol that
include/dpg.h declares, and rejects invalid arguments before touching HIP."""
import ctypes
import math
import os
import re

import pytest

import dp_grape_projection_amd as dpg
from dp_grape_projection_amd.binding import LayerGrad, LayerHat, LayerParam

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dpg.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dpg.library_path()):
        pytest.skip("libdpg.so not built")
    return dpg.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dpg_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("dpg_project_clip_noise", "dpg_adam_backproject",
              "dpg_project_workspace_size", "dpg_adam_workspace_size",
              "dpg_philox_normals", "dpg_status_string", "dpg_last_error",
              "dpg_version", "dpg_project_layer", "dpg_clip_sum_noise",
              "dpg_project_layer_workspace_size", "dpg_clip_workspace_size",
              "dpg_step_workspace_size", "dpg_private_step",
              "dpg_private_step_static", "dpg_static_scratch_bytes"):
        assert n in names
    assert sorted(dpg.EXPORTED) == names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.dpg_version() == 10100


def test_struct_layout_matches_header():
    # int64 d_in, d_out; u32 layer_id, reserved; three / four pointers
    assert ctypes.sizeof(LayerGrad) == 8 + 8 + 4 + 4 + 3 * 8
    assert ctypes.sizeof(LayerParam) == 8 + 8 + 4 + 4 + 4 * 8
    assert LayerGrad.A.offset == 24 and LayerParam.G_priv.offset == 24
    # int64 d_out; u32 layer_id, reserved; two pointers
    assert ctypes.sizeof(LayerHat) == 8 + 4 + 4 + 2 * 8
    assert LayerHat.G_hat.offset == 16


def _grads(shapes, ids=None, ptr=0x1000):
    arr = (LayerGrad * len(shapes))()
    for i, (a, b) in enumerate(shapes):
        arr[i].d_in, arr[i].d_out = a, b
        arr[i].layer_id = i if ids is None else ids[i]
        arr[i].A = arr[i].dY = arr[i].G_priv = ptr
    return arr


def _params(shapes, ids=None, ptr=0x1000):
    arr = (LayerParam * len(shapes))()
    for i, (a, b) in enumerate(shapes):
        arr[i].d_in, arr[i].d_out = a, b
        arr[i].layer_id = i if ids is None else ids[i]
        arr[i].G_priv = arr[i].W = arr[i].m = arr[i].v = ptr
    return arr


def test_abi_names_and_status_codes():
    """The boundary as built: workspace queries named *_workspace_size that
    return a status and write the size through a pointer, and positive status
    codes (0 is success). The C header and the binding agree on both."""
    text = open(HEADER).read()
    codes = dict((k, int(v)) for k, v in re.findall(r"(DPG_[A-Z0-9_]+) = (\d+)", text))
    assert codes == {"DPG_OK": 0, "DPG_ERR_INVALID_ARG": 1, "DPG_ERR_WORKSPACE": 2,
                     "DPG_ERR_UNSUPPORTED": 3, "DPG_ERR_HIP": 4,
                     "DPG_FP32": 0, "DPG_BF16": 1}
    b = dpg.binding
    assert (b.DPG_OK, b.DPG_ERR_INVALID_ARG, b.DPG_ERR_WORKSPACE,
            b.DPG_ERR_UNSUPPORTED, b.DPG_ERR_HIP) == (0, 1, 2, 3, 4)
    for name in ("dpg_project_workspace_size", "dpg_adam_workspace_size",
                 "dpg_step_workspace_size", "dpg_project_layer_workspace_size",
                 "dpg_clip_workspace_size"):
        decl = re.search(r"int\s+" + name + r"\s*\(([^)]*)\)", text, re.S)
        assert decl and "size_t* bytes" in decl.group(1), name


def test_r_times_d_limit_in_size_queries(lib):
    """r*d_out = 2^31 is rejected by the workspace queries too."""
    out = ctypes.c_size_t(0)
    st = lib.dpg_project_workspace_size(_grads([(4, 2 ** 22)]), 1, 1, 1, 512, 1,
                                        ctypes.byref(out))
    assert st == dpg.binding.DPG_ERR_INVALID_ARG
    st = lib.dpg_adam_workspace_size(_params([(4, 2 ** 22)]), 1, 512, 1,
                                     ctypes.byref(out))
    assert st == dpg.binding.DPG_ERR_INVALID_ARG
    st = lib.dpg_project_workspace_size(_grads([(4, 2 ** 22 - 1)]), 1, 1, 1, 512, 1,
                                        ctypes.byref(out))
    assert st == 0


def test_status_strings(lib):
    for code in range(5):
        assert lib.dpg_status_string(code).startswith(b"DPG_")
    assert b"unknown" in lib.dpg_status_string(99)


def test_workspace_size_queries(lib):
    out = ctypes.c_size_t(0)
    st = lib.dpg_project_workspace_size(_grads([(768, 3072), (3072, 768)]), 2,
                                        32, 128, 128, 1, ctypes.byref(out))
    assert st == 0 and out.value > 0 and out.value % 256 == 0
    small = ctypes.c_size_t(0)
    assert lib.dpg_project_workspace_size(_grads([(8, 8)]), 1, 1, 1, 1, 0,
                                          ctypes.byref(small)) == 0
    assert 0 < small.value < out.value
    st = lib.dpg_adam_workspace_size(_params([(768, 3072)]), 1, 128, 1,
                                     ctypes.byref(out))
    assert st == 0 and out.value >= (768 + 3072) * 128 * 2


BAD_PROJECT = [
    # (description, overrides)
    ("zero batch", dict(B=0)),
    ("zero T", dict(T=0)),
    ("zero r", dict(r=0)),
    ("bad dtype", dict(dtype=7)),
    ("zero layers", dict(n=0)),
    ("negative C", dict(C=-1.0)),
    ("zero C", dict(C=0.0)),
    ("NaN C", dict(C=float("nan"))),
    ("negative sigma", dict(sigma=-0.1)),
    ("inf sigma", dict(sigma=float("inf"))),
    ("inf C with noise", dict(C=float("inf"), sigma=1.0)),
    ("step 0", dict(step=0)),
    ("step 2^32", dict(step=2 ** 32)),
    ("proj_step 2^32", dict(proj_step=2 ** 32)),
    ("duplicate ids", dict(ids=[3, 3])),
    ("zero d_in", dict(shapes=[(0, 4), (4, 4)])),
    ("huge r*d", dict(shapes=[(2 ** 30, 4), (4, 4)], r=8)),
    # r*d_out = 2^31: the element counts of the final and Adam passes are int32
    ("r*d_out 2^31", dict(shapes=[(4, 2 ** 22), (4, 4)], r=512)),
    ("r*d_in 2^31", dict(shapes=[(2 ** 22, 4), (4, 4)], r=512)),
    ("null data", dict(ptr=0)),
]


@pytest.mark.parametrize("desc,kw", BAD_PROJECT, ids=[d for d, _ in BAD_PROJECT])
def test_project_rejects_invalid_arguments(lib, desc, kw):
    shapes = kw.get("shapes", [(16, 8), (8, 16)])
    arr = _grads(shapes, kw.get("ids"), kw.get("ptr", 0x1000))
    st = lib.dpg_project_clip_noise(
        arr, kw.get("n", len(shapes)), kw.get("B", 2), kw.get("T", 3),
        kw.get("r", 4), kw.get("dtype", 1), kw.get("C", 1.0),
        kw.get("sigma", 0.5), 0, kw.get("step", 1), kw.get("proj_step", 1),
        None, 0x10000, 1 << 30, None)
    assert st == dpg.binding.DPG_ERR_INVALID_ARG, desc
    assert lib.dpg_last_error() != b""


def test_project_workspace_errors(lib):
    arr = _grads([(16, 8)])
    need = ctypes.c_size_t(0)
    assert lib.dpg_project_workspace_size(arr, 1, 2, 3, 4, 1,
                                          ctypes.byref(need)) == 0
    args = (arr, 1, 2, 3, 4, 1, 1.0, 0.5, 0, 1, 1, None)
    assert lib.dpg_project_clip_noise(*args, None, need.value, None) == 2
    assert lib.dpg_project_clip_noise(*args, 0x10000, need.value - 1, None) == 2
    assert lib.dpg_project_clip_noise(*args, 0x10010, need.value, None) == 2
    assert b"workspace" in lib.dpg_last_error()


BAD_ADAM = [
    ("zero lr", dict(lr=0.0)),
    ("inf lr", dict(lr=float("inf"))),
    ("beta1 = 1", dict(b1=1.0)),
    ("negative beta2", dict(b2=-0.1)),
    ("zero eps", dict(eps=0.0)),
    ("step 0", dict(step=0)),
    ("zero r", dict(r=0)),
    ("duplicate ids", dict(ids=[1, 1])),
    ("null data", dict(ptr=0)),
    ("bad dtype", dict(dtype=3)),
]


@pytest.mark.parametrize("desc,kw", BAD_ADAM, ids=[d for d, _ in BAD_ADAM])
def test_adam_rejects_invalid_arguments(lib, desc, kw):
    shapes = [(16, 8), (8, 16)]
    arr = _params(shapes, kw.get("ids"), kw.get("ptr", 0x1000))
    st = lib.dpg_adam_backproject(
        arr, 2, kw.get("r", 4), kw.get("dtype", 1), kw.get("lr", 1e-3),
        kw.get("b1", 0.9), kw.get("b2", 0.999), kw.get("eps", 1e-8), 0,
        kw.get("step", 1), 1, 0x10000, 1 << 30, None)
    assert st == dpg.binding.DPG_ERR_INVALID_ARG, desc


def test_philox_rejects_invalid_arguments(lib):
    assert lib.dpg_philox_normals(0, 0, 0, 0, 0, 0, None, None, None) == 0
    assert lib.dpg_philox_normals(0, 0, 0, 0, 0, 4, None, None, None) == 1
    assert lib.dpg_philox_normals(0, 0, 0, 0, 2 ** 32 - 2, 4, 0x1000, None,
                                  None) == 1


def test_binding_raises_without_library(tmp_path):
    with pytest.raises(FileNotFoundError):
        dpg.load_library(str(tmp_path / "missing.so"))


# --- streaming form ----------------------------------------------------------

def _hats(d_outs, ids=None, ptr=0x1000):
    arr = (LayerHat * len(d_outs))()
    for i, d in enumerate(d_outs):
        arr[i].d_out = d
        arr[i].layer_id = i if ids is None else ids[i]
        arr[i].G_hat = arr[i].G_priv = ptr
    return arr


def test_streaming_workspace_queries(lib):
    one = ctypes.c_size_t(0)
    assert lib.dpg_project_layer_workspace_size(_grads([(768, 3072)]), 32, 128, 128, 1,
                                                ctypes.byref(one)) == 0
    assert one.value > 0 and one.value % 256 == 0
    clip = ctypes.c_size_t(0)
    assert lib.dpg_clip_workspace_size(32, ctypes.byref(clip)) == 0
    assert clip.value >= 32 * 4 and clip.value % 256 == 0
    assert lib.dpg_clip_workspace_size(0, ctypes.byref(clip)) == 1


BAD_LAYER = [
    ("zero batch", dict(B=0)),
    ("zero r", dict(r=0)),
    ("bad dtype", dict(dtype=5)),
    ("proj_step 2^32", dict(proj_step=2 ** 32)),
    ("null G_hat", dict(ghat=None)),
    ("null norm_sq", dict(norm_sq=None)),
    ("null data", dict(ptr=0)),
]


@pytest.mark.parametrize("desc,kw", BAD_LAYER, ids=[d for d, _ in BAD_LAYER])
def test_project_layer_rejects_invalid_arguments(lib, desc, kw):
    arr = _grads([(16, 8)], ptr=kw.get("ptr", 0x1000))
    st = lib.dpg_project_layer(arr, kw.get("B", 2), 3, kw.get("r", 4), kw.get("dtype", 1),
                               0, kw.get("proj_step", 1), kw.get("ghat", 0x2000),
                               kw.get("norm_sq", 0x3000), 0x10000, 1 << 30, None)
    assert st == dpg.binding.DPG_ERR_INVALID_ARG, desc
    assert lib.dpg_last_error() != b""


BAD_CLIP = [
    ("zero layers", dict(n=0)),
    ("zero batch", dict(B=0)),
    ("zero r", dict(r=0)),
    ("zero C", dict(C=0.0)),
    ("inf C with noise", dict(C=float("inf"), sigma=1.0)),
    ("negative sigma", dict(sigma=-1.0)),
    ("step 0", dict(step=0)),
    ("duplicate ids", dict(ids=[2, 2])),
    ("null norm_sq", dict(norm_sq=None)),
    ("null data", dict(ptr=0)),
]


@pytest.mark.parametrize("desc,kw", BAD_CLIP, ids=[d for d, _ in BAD_CLIP])
def test_clip_sum_noise_rejects_invalid_arguments(lib, desc, kw):
    arr = _hats([8, 16], kw.get("ids"), kw.get("ptr", 0x1000))
    st = lib.dpg_clip_sum_noise(arr, kw.get("n", 2), kw.get("B", 2), kw.get("r", 4),
                                kw.get("C", 1.0), kw.get("sigma", 0.5), 0,
                                kw.get("step", 1), kw.get("norm_sq", 0x3000), None,
                                0x10000, 1 << 30, None)
    assert st == dpg.binding.DPG_ERR_INVALID_ARG, desc


def test_clip_sum_noise_workspace_errors(lib):
    arr = _hats([8])
    args = (arr, 1, 64, 4, 1.0, 0.5, 0, 1, 0x3000, None)
    assert lib.dpg_clip_sum_noise(*args, None, 256, None) == 2
    assert lib.dpg_clip_sum_noise(*args, 0x10000, 255, None) == 2
    assert lib.dpg_clip_sum_noise(*args, 0x10010, 256, None) == 2


# ------------------------------------------------------ the one-call step --

BAD_STEP = BAD_PROJECT + [
    ("zero lr", dict(lr=0.0)),
    ("beta1 = 1", dict(b1=1.0)),
    ("zero eps", dict(eps=0.0)),
    ("null params", dict(no_params=True)),
    ("params d_in differs", dict(pshapes=[(16, 8), (9, 16)])),
    ("params id differs", dict(pids=[0, 7])),
    ("null W", dict(pptr=0)),
]


@pytest.mark.parametrize("desc,kw", BAD_STEP, ids=[d for d, _ in BAD_STEP])
def test_private_step_rejects_invalid_arguments(lib, desc, kw):
    shapes = kw.get("shapes", [(16, 8), (8, 16)])
    arr = _grads(shapes, kw.get("ids"), kw.get("ptr", 0x1000))
    pshapes = kw.get("pshapes", shapes)
    par = None if kw.get("no_params") else _params(
        pshapes, kw.get("pids", kw.get("ids")), kw.get("pptr", 0x1000))
    st = lib.dpg_private_step(
        arr, par, kw.get("n", len(shapes)), kw.get("B", 2), kw.get("T", 3),
        kw.get("r", 4), kw.get("dtype", 1), kw.get("C", 1.0), kw.get("sigma", 0.5),
        kw.get("lr", 1e-3), kw.get("b1", 0.9), kw.get("b2", 0.999),
        kw.get("eps", 1e-8), 0, kw.get("step", 1), kw.get("proj_step", 1), None,
        0x10000, 1 << 30, None)
    assert st == dpg.binding.DPG_ERR_INVALID_ARG, desc
    assert lib.dpg_last_error() != b""


def test_private_step_workspace(lib):
    """The one-call step needs the projection's workspace plus room for the
    update direction U of every layer; too little, NULL or misaligned is an
    error before anything is enqueued."""
    shapes = [(16, 8), (8, 16)]
    arr, par = _grads(shapes), _params(shapes)
    need, proj = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.dpg_step_workspace_size(arr, 2, 2, 3, 4, 1, ctypes.byref(need)) == 0
    assert lib.dpg_project_workspace_size(arr, 2, 2, 3, 4, 1, ctypes.byref(proj)) == 0
    # U: [4, 8] and [4, 16] bf16, each 256-byte aligned
    assert need.value == proj.value + 256 + 256
    assert lib.dpg_step_workspace_size(arr, 2, 2, 3, 4, 1, None) == 1
    args = (arr, par, 2, 2, 3, 4, 1, 1.0, 0.5, 1e-3, 0.9, 0.999, 1e-8, 0, 1, 1, None)
    assert lib.dpg_private_step(*args, None, need.value, None) == 2
    assert lib.dpg_private_step(*args, 0x10000, need.value - 1, None) == 2
    assert lib.dpg_private_step(*args, 0x10010, need.value, None) == 2
    assert b"workspace" in lib.dpg_last_error()


def test_static_step_rejects_a_step_beyond_its_scratch(lib):
    """dpg_private_step_static: a step whose scratch exceeds the static array
    (enc12 needs about 1 GiB) fails with DPG_ERR_WORKSPACE before any HIP
    call; so does an invalid shape, with DPG_ERR_INVALID_ARG."""
    import workloads as W
    assert lib.dpg_static_scratch_bytes() == 64 << 20
    wl = W.workload("enc12")
    shapes = [(L.d_in, L.d_out) for L in wl.layers]
    ids = [L.layer_id for L in wl.layers]
    n = len(shapes)
    args = (_grads(shapes, ids), _params(shapes, ids), n, wl.B, wl.T, wl.r, 1,
            1.0, 0.5, 1e-3, 0.9, 0.999, 1e-8, 0, 1, 1, None, None)
    assert lib.dpg_private_step_static(*args) == dpg.binding.DPG_ERR_WORKSPACE
    assert b"static scratch" in lib.dpg_last_error()
    bad = list(args)
    bad[5] = 0   # r = 0
    assert lib.dpg_private_step_static(*bad) == dpg.binding.DPG_ERR_INVALID_ARG


BAD_RC = [
    ("zero batch", dict(B=0)),
    ("zero k", dict(k=0)),
    ("bad dtype", dict(dtype=7)),
    ("zero C", dict(C=0.0)),
    ("NaN C", dict(C=float("nan"))),
    ("step 0", dict(step=0)),
    ("step 2^32", dict(step=2 ** 32)),
    ("duplicate ids", dict(ids=[3, 3])),
    ("k*d_out 2^31", dict(shapes=[(4, 2 ** 22), (4, 4)], k=512)),
    ("null data", dict(ptr=0)),
    ("null norms", dict(norms=None)),
]


@pytest.mark.parametrize("desc,kw", BAD_RC, ids=[d for d, _ in BAD_RC])
def test_rc_norms_rejects_invalid_arguments(lib, desc, kw):
    """dpg_rc_norms validates before it enqueues anything (no GPU needed)."""
    shapes = kw.get("shapes", [(16, 8), (8, 16)])
    arr = _grads(shapes, kw.get("ids"), kw.get("ptr", 0x1000))
    st = lib.dpg_rc_norms(arr, len(shapes), kw.get("B", 2), kw.get("T", 3), kw.get("k", 4),
                          kw.get("dtype", 1), kw.get("C", 1.0), 0, kw.get("step", 1),
                          kw.get("norms", 0x20000), 0x30000, 0x10000, 1 << 30, None)
    assert st == dpg.binding.DPG_ERR_INVALID_ARG, desc
    assert lib.dpg_last_error() != b""


def test_rc_norms_workspace(lib):
    """The estimate's workspace query: positive and 256-aligned for valid
    shapes, growing with k; a short workspace is rejected."""
    arr = _grads([(768, 3072), (3072, 768)])
    small, big = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.dpg_rc_norms_workspace_size(arr, 2, 32, 128, 8, 1, ctypes.byref(small)) == 0
    assert lib.dpg_rc_norms_workspace_size(arr, 2, 32, 128, 64, 1, ctypes.byref(big)) == 0
    assert 0 < small.value < big.value and big.value % 256 == 0
    assert lib.dpg_rc_norms_workspace_size(arr, 2, 32, 128, 8, 1, None) == \
        dpg.binding.DPG_ERR_INVALID_ARG
    st = lib.dpg_rc_norms(arr, 2, 32, 128, 8, 1, 1.0, 0, 1, 0x20000, 0x30000, 0x10000,
                          small.value - 1, None)
    assert st == dpg.binding.DPG_ERR_WORKSPACE
