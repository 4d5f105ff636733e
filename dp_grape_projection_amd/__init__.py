"""DP-GRAPE private update step on one AMD MI355X (gfx950).

The compute lives in libdpg.so (C ABI in include/dpg.h, HIP kernels in
csrc/); this package is its thin Python binding.
"""
from .binding import (  # noqa: F401
    DPG_BF16, DPG_FP32, DpgError, EXPORTED, LayerGrad, LayerHat, LayerParam,
    PreparedStep, PreparedStreamingStep, adam_workspace_size, dpg_adam_backproject,
    dpg_clip_sum_noise, dpg_philox_normals, dpg_private_step, dpg_private_step_static,
    dpg_project_clip_noise, dpg_project_layer, dpg_rc_norms, library_path, load_library,
    project_workspace_size, static_scratch_bytes, timing_enable, timing_read, version,
)
from .streaming import GrapeOptimizer, ProjectedLinear  # noqa: F401
