"""CPU oracle for the DP-GRAPE private update step (test infrastructure).

A plain, slow, float64 numpy implementation of what the GPU library computes,
written from the method's description and sharing no code with the HIP path.
Only the tests, the smoke check and the bench's CPU-baseline leg may import
it; the product path never does.

Sources (gist.science pages; cited by page title and section):
  [GRAPE]  "Memory-Efficient Differentially Private Training with Gradient
           Random Projection" (arXiv 2506.15588 explainer, es/fr/it/hi),
           technical summary: Problem statement; Methodology design choices
           1 (random Gaussian projection regenerated from a seed), 2
           (projection before privatisation), 3 (projected optimizer states)
           and the closing paragraph of Methodology (training loop).
  [RC]     "DP-SGD Eficiente para LLMs con Recorte Aleatorizado" (arXiv
           2605.24879 explainer), Methodology - core mechanism (trace
           identity, Hutchinson estimator) and Algorithmic flow steps 3-4
           (norm estimation; clip factor min(C/n, 1)); oracle.randclip.

Parity status of each function is stated in its docstring. Readings where the
pages are silent are listed in the module docstring of oracle.dpgrape.
"""
from .philox import philox4x32_10, uniform_open01, gaussian_stream  # noqa: F401
from .dpgrape import (  # noqa: F401
    TAG_PROJECTION, TAG_NOISE,
    projection_matrix, noise_matrix, per_sample_gradient,
    project_clip_noise, adam_update, backproject_delta, adam_backproject,
    naive_privatise_then_project, sample_norms, clip_scale,
    projection_rows, noise_rows, g_priv_rows,
)
from .randclip import (  # noqa: F401
    TAG_PROBE, probe_matrix, hutchinson_layer, estimated_norms, rc_clip_factors,
)
