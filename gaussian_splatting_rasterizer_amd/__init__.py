"""MI355X (gfx950) Gaussian-splat render + analytic score replay + renderer backward.

The compute path is the HIP library libgsr.so (C ABI in include/gsr.h); this
package holds its kernels (csrc/), the build step (build.py) and a thin ctypes
binding (binding.py).  Importing the package does not load the library; the
binding loads it on first use and raises if it is missing.
"""
from .binding import (GS_OK, GsrError, Rasterizer, gs_attribute, gs_backward, gs_bin_sort,  # noqa: F401
                      gs_context_create, gs_context_destroy, gs_debug_exp2, gs_debug_export, gs_default_params,
                      gs_gaussian_grads, gs_profile_enable, gs_profile_read, gs_project, gs_render,
                      gs_render_features, gs_score_replay, gs_workspace_size, load_library, rasterizer_for_scene)
