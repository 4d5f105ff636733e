"""GPU parity of dpg_rc_norms, randomized clipping's per-sample norm estimate
([RC] "DP-SGD Eficiente para LLMs con Recorte Aleatorizado", Methodology:
DP-SGD-RC, Hutchinson estimator; Algorithmic flow steps 3-4), through the C
ABI, against oracle.randclip on the same seeded inputs and the same probe
stream: each sample's estimated norm is a piece of its own (rel_err), at the
bar of the input type; the clip factors follow min(1, C / nhat)."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from _helpers import TOL, make_case, rel_err, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_and_library():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dp_grape_projection_amd as dpg
    dpg.load_library()     # fails loudly when libdpg.so is missing


CASES = [
    # ragged shapes, odd k, fp32 and bf16 (the regular tile kernels)
    ("fp32_ragged_k7", W.custom_workload("rc_fp32", 71, [(200, 136), (136, 300), (72, 40)],
                                         B=3, T=37, r=7, dtype="fp32", layer_ids=[5, 17, 2]), 7),
    ("bf16_ragged_k32", W.custom_workload("rc_bf16", 72, [(200, 136), (136, 300), (72, 40)],
                                          B=3, T=40, r=32, layer_ids=[5, 17, 2]), 32),
    # k = 32 on mlp4's shapes (the page's example probe count)
    ("mlp4_k32", W.workload("mlp4"), 32),
    # k a multiple of 256 with whole 256-wide tiles: the large tile kernels
    ("bf16_big_k256", W.custom_workload("rc_big", 73, [(512, 768), (768, 256)],
                                        B=2, T=256, r=256, layer_ids=[3, 8]), 256),
]


def _run(wl, host, k, clip_C, step):
    import torch
    import dp_grape_projection_amd as dpg
    A = [to_device(wl, a) for a, _ in host]
    dY = [to_device(wl, d) for _, d in host]
    n, s = dpg.dpg_rc_norms(A, dY, k=k, clip_C=clip_C, seed=wl.seed, step=step,
                            layer_ids=[L.layer_id for L in wl.layers])
    torch.cuda.synchronize()
    return n.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("name,wl,k", CASES, ids=[c[0] for c in CASES])
def test_rc_norms_parity(name, wl, k):
    print(f"[rc_norms] {name}: {len(wl.layers)} layers B={wl.B} T={wl.T} k={k} {wl.dtype}",
          flush=True)
    host, orc, _ = make_case(wl)
    step = 3
    want = oracle.estimated_norms(orc, k, wl.seed, step)
    exact = oracle.sample_norms(orc, 1, 0, 1, P_override={
        l["layer_id"]: np.eye(l["A"].shape[2]) for l in orc})  # P = I: the exact norm
    # a clip threshold between the smallest and largest estimate, so that
    # both branches of the clip factor occur
    C = float(np.sort(want)[len(want) // 2])
    n, s = _run(wl, host, k, C, step)
    tol = TOL[wl.dtype]
    e = rel_err(n, want)
    print(f"  nhat rel_err {e:.3e}; nhat / n in [{(want / exact).min():.3f}, "
          f"{(want / exact).max():.3f}]", flush=True)
    assert e <= tol, f"{name} norms {e}"
    np.testing.assert_array_equal(s, np.where(n > np.float32(C), np.float32(C) / n,
                                              np.float32(1.0)).astype(np.float32))
    assert rel_err(s, oracle.rc_clip_factors(want, C)) <= tol


def test_rc_norms_new_probes_each_step():
    """The probes are keyed on the step: two steps give different estimates,
    each matching the oracle's for its own step."""
    wl = CASES[1][1]
    host, orc, _ = make_case(wl)
    for step in (1, 2):
        n, _ = _run(wl, host, 32, math.inf, step)
        assert rel_err(n, oracle.estimated_norms(orc, 32, wl.seed, step)) <= TOL["bf16"]
    n1, _ = _run(wl, host, 32, math.inf, 1)
    n2, _ = _run(wl, host, 32, math.inf, 2)
    assert not np.allclose(n1, n2)


def test_rc_norms_zero_gradient():
    """A = 0: every estimate is 0 and every clip factor 1."""
    wl = CASES[0][1]
    host, _, _ = make_case(wl, a_zero=True)
    n, s = _run(wl, host, 7, 0.5, 1)
    np.testing.assert_array_equal(n, np.zeros_like(n))
    np.testing.assert_array_equal(s, np.ones_like(s))
