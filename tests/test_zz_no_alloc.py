"""dpg_private_step_static, the one-call step that allocates nothing (its
scratch is a static device array of the library), through the C ABI, against
dpg_private_step with a caller workspace: two calls in a row, the second on a
smaller input, each bit for bit against the workspace form on copies of the
same state. (A step too large for the static array is rejected on the CPU:
tests/test_abi_cpu.py.)

The file name sorts last so that it also runs after every other GPU test."""
import numpy as np
import pytest

import workloads as W
from _helpers import make_case, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_and_library():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dp_grape_projection_amd as dpg
    dpg.load_library()     # fails loudly when libdpg.so is missing


def _device_state(state):
    import torch
    return ([torch.from_numpy(s[0].copy()).cuda() for s in state],
            [torch.from_numpy(s[1].copy()).cuda() for s in state],
            [torch.from_numpy(s[2].copy()).cuda() for s in state])


CASES = [
    # mlp4: about 50 MiB of the 64 MiB scratch
    ("mlp4", W.workload("mlp4"), 3),
    # then a smaller ragged case, which runs in what the first call left
    ("small", W.custom_workload("static_small", 61, [(200, 136), (136, 300), (72, 40)],
                                B=3, T=40, r=40, layer_ids=[5, 17, 2]), 5),
]


@pytest.mark.parametrize("name,wl,step", CASES, ids=[c[0] for c in CASES])
def test_static_matches_workspace_form(name, wl, step):
    import torch
    import dp_grape_projection_amd as dpg
    print(f"[no-alloc] {name}: {len(wl.layers)} layers B={wl.B} T={wl.T} r={wl.r} "
          f"step {step}", flush=True)
    host, _, state = make_case(wl)
    A = [to_device(wl, a) for a, _ in host]
    dY = [to_device(wl, d) for _, d in host]
    ids = [L.layer_id for L in wl.layers]
    hyper = dict(r=wl.r, clip_C=wl.clip_C, sigma=wl.sigma, lr=wl.lr, beta1=wl.beta1,
                 beta2=wl.beta2, eps=wl.eps, seed=wl.seed, step=step, proj_step=step,
                 layer_ids=ids)
    Wa, ma, va = _device_state(state)
    Ga, na = dpg.dpg_private_step(A, dY, Wa, ma, va, **hyper)
    Wb, mb, vb = _device_state(state)
    Gb = [torch.empty((wl.r, L.d_out), dtype=torch.float32, device="cuda")
          for L in wl.layers]
    nb = torch.empty(wl.B, dtype=torch.float32, device="cuda")
    dpg.dpg_private_step_static(A, dY, Wb, mb, vb, Gb, nb, **hyper)
    torch.cuda.synchronize()
    for x, y in zip([na, *Ga, *Wa, *ma, *va], [nb, *Gb, *Wb, *mb, *vb]):
        np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy())
