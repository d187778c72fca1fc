"""Thin ctypes binding over the C ABI of include/gsr.h.

Argument marshalling only: every step of the render and the score replay runs
in the HIP kernels of libgsr.so.  PyTorch is used for device memory (inputs,
outputs, the workspace) and for the current HIP stream.  The functions keep
the C names (gs_project, gs_bin_sort, gs_render, gs_score_replay, ...); the
`Rasterizer` class strings them together and sizes the workspace.

There is no fallback: if libgsr.so is missing or fails to load, every entry
point raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libgsr.so")

GS_OK = 0
GS_ERR_INVALID_ARGUMENT = 1
GS_ERR_WORKSPACE_TOO_SMALL = 2
GS_ERR_STATE = 3
GS_ERR_HIP = 4
GS_ERR_UNSUPPORTED = 5
GS_MAX_VIEWS = 32
GS_EXPORT_RECORDS = 1
GS_EXPORT_DEPTH_KEYS = 2
GS_EXPORT_SORTED_IDS = 3
GS_EXPORT_RANGES = 4
GS_EXPORT_PIXEL_STATS = 5
STAGES = ("project", "depth_sort", "scan", "emit", "tile_sort", "ranges", "render", "replay", "finalize",
          "backward", "backward_finalize", "features", "attribute")

ABI_SYMBOLS = ("gs_default_params", "gs_workspace_size", "gs_context_create", "gs_context_destroy",
               "gs_project", "gs_bin_sort", "gs_render", "gs_score_replay", "gs_backward", "gs_render_features",
               "gs_attribute", "gs_status_string",
               "gs_last_error", "gs_debug_exp2", "gs_debug_export", "gs_debug_topk", "gs_profile_enable",
               "gs_profile_stages", "gs_profile_read", "gs_render_score_noalloc")


class gs_gaussians(ctypes.Structure):
    _fields_ = [("means", ctypes.c_void_p), ("quats", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("opacities", ctypes.c_void_p), ("sh", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("sh_degree", ctypes.c_int32)]


class gs_gaussian_grads(ctypes.Structure):
    _fields_ = [("means", ctypes.c_void_p), ("quats", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("opacities", ctypes.c_void_p), ("sh", ctypes.c_void_p)]


class gs_camera(ctypes.Structure):
    _fields_ = [("R", ctypes.c_float * 9), ("t", ctypes.c_float * 3), ("fx", ctypes.c_float),
                ("fy", ctypes.c_float), ("cx", ctypes.c_float), ("cy", ctypes.c_float)]


class gs_dims(ctypes.Structure):
    _fields_ = [("n_gaussians", ctypes.c_int64), ("sh_degree", ctypes.c_int32), ("n_views", ctypes.c_int32),
                ("width", ctypes.c_int32), ("height", ctypes.c_int32), ("max_pairs", ctypes.c_uint64)]


class gs_params(ctypes.Structure):
    _fields_ = [("eps", ctypes.c_float), ("den_min", ctypes.c_float), ("lam", ctypes.c_float),
                ("near_plane", ctypes.c_float), ("far_plane", ctypes.c_float),
                ("background", ctypes.c_float * 3), ("antialiased", ctypes.c_int32)]


class GsrError(RuntimeError):
    def __init__(self, status, where, message):
        super().__init__(f"{where}: {status_name(status)}: {message}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libgsr.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P, St = ctypes.c_void_p, ctypes.c_int
    lib.gs_default_params.restype = St
    lib.gs_default_params.argtypes = [ctypes.POINTER(gs_params)]
    lib.gs_workspace_size.restype = St
    lib.gs_workspace_size.argtypes = [ctypes.POINTER(gs_dims), ctypes.POINTER(ctypes.c_size_t)]
    lib.gs_context_create.restype = St
    lib.gs_context_create.argtypes = [ctypes.POINTER(gs_dims), P, ctypes.c_size_t, ctypes.POINTER(P)]
    lib.gs_context_destroy.restype = St
    lib.gs_context_destroy.argtypes = [P]
    lib.gs_project.restype = St
    lib.gs_project.argtypes = [P, ctypes.POINTER(gs_gaussians), ctypes.POINTER(gs_camera),
                               ctypes.POINTER(gs_params), P]
    lib.gs_bin_sort.restype = St
    lib.gs_bin_sort.argtypes = [P, P, ctypes.POINTER(ctypes.c_uint64)]
    lib.gs_render.restype = St
    lib.gs_render.argtypes = [P, P, P, P, P]
    lib.gs_score_replay.restype = St
    lib.gs_score_replay.argtypes = [P, P, P, P]
    lib.gs_backward.restype = St
    lib.gs_backward.argtypes = [P, P, ctypes.POINTER(gs_gaussian_grads), P]
    lib.gs_render_features.restype = St
    lib.gs_render_features.argtypes = [P, P, ctypes.c_int32, P, P, P]
    lib.gs_attribute.restype = St
    lib.gs_attribute.argtypes = [P, P, ctypes.c_int32, P, P]
    lib.gs_status_string.restype = ctypes.c_char_p
    lib.gs_status_string.argtypes = [St]
    lib.gs_last_error.restype = ctypes.c_char_p
    lib.gs_last_error.argtypes = []
    lib.gs_debug_exp2.restype = St
    lib.gs_debug_exp2.argtypes = [P, P, ctypes.c_int64, P]
    lib.gs_debug_export.restype = St
    lib.gs_debug_export.argtypes = [P, ctypes.c_int32, P, ctypes.c_size_t, P]
    lib.gs_debug_topk.restype = St
    lib.gs_debug_topk.argtypes = [P, ctypes.c_int32, P, P, P]
    lib.gs_profile_enable.restype = St
    lib.gs_profile_enable.argtypes = [P, ctypes.c_int32]
    lib.gs_profile_stages.restype = St
    lib.gs_profile_stages.argtypes = [P, ctypes.c_uint32]
    lib.gs_profile_read.restype = St
    lib.gs_profile_read.argtypes = [P, P, P, ctypes.c_int32]
    lib.gs_render_score_noalloc.restype = St
    lib.gs_render_score_noalloc.argtypes = [ctypes.POINTER(gs_gaussians), ctypes.POINTER(gs_camera), ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(gs_params), P, P, P, P,
                                            P, P]
    _lib = lib
    return lib


def status_name(status: int) -> str:
    return load_library().gs_status_string(int(status)).decode()


def last_error() -> str:
    return load_library().gs_last_error().decode()


def _check(status, where):
    if status != GS_OK:
        raise GsrError(status, where, last_error())


def _stream_handle(stream=None) -> ctypes.c_void_p:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev_ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(None)


# ---- the ABI calls, same names as in C -------------------------------------------------------------
def gs_default_params() -> gs_params:
    p = gs_params()
    _check(load_library().gs_default_params(ctypes.byref(p)), "gs_default_params")
    return p


def gs_workspace_size(dims: gs_dims) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().gs_workspace_size(ctypes.byref(dims), ctypes.byref(out)), "gs_workspace_size")
    return int(out.value)


def gs_context_create(dims: gs_dims, workspace_ptr: int, nbytes: int) -> ctypes.c_void_p:
    ctx = ctypes.c_void_p()
    _check(load_library().gs_context_create(ctypes.byref(dims), ctypes.c_void_p(workspace_ptr), nbytes,
                                            ctypes.byref(ctx)), "gs_context_create")
    return ctx


def gs_context_destroy(ctx) -> None:
    load_library().gs_context_destroy(ctx)


def gs_project(ctx, gaussians: gs_gaussians, cams, params: gs_params, stream=None) -> None:
    _check(load_library().gs_project(ctx, ctypes.byref(gaussians), cams, ctypes.byref(params),
                                     _stream_handle(stream)), "gs_project")


def gs_bin_sort(ctx, stream=None, raise_on_overflow=True) -> tuple:
    n = ctypes.c_uint64(0)
    st = load_library().gs_bin_sort(ctx, _stream_handle(stream), ctypes.byref(n))
    if st == GS_ERR_WORKSPACE_TOO_SMALL and not raise_on_overflow:
        return st, int(n.value)
    _check(st, "gs_bin_sort")
    return st, int(n.value)


def gs_render(ctx, color, T_final, n_contrib, stream=None) -> None:
    _check(load_library().gs_render(ctx, _dev_ptr(color), _dev_ptr(T_final), _dev_ptr(n_contrib),
                                    _stream_handle(stream)), "gs_render")


def gs_score_replay(ctx, observed, tokens, stream=None) -> None:
    _check(load_library().gs_score_replay(ctx, _dev_ptr(observed), _dev_ptr(tokens), _stream_handle(stream)),
           "gs_score_replay")


def gs_render_score_noalloc(gauss: gs_gaussians, cams, n_views, width, height, params: gs_params, observed,
                            color, T_final, n_contrib, tokens, stream=None) -> None:
    _check(load_library().gs_render_score_noalloc(ctypes.byref(gauss), cams, int(n_views), int(width), int(height),
                                                  ctypes.byref(params), _dev_ptr(observed), _dev_ptr(color),
                                                  _dev_ptr(T_final), _dev_ptr(n_contrib), _dev_ptr(tokens),
                                                  _stream_handle(stream)), "gs_render_score_noalloc")


def gs_backward(ctx, grad_color, grads: gs_gaussian_grads, stream=None) -> None:
    _check(load_library().gs_backward(ctx, _dev_ptr(grad_color), ctypes.byref(grads), _stream_handle(stream)),
           "gs_backward")


def gs_render_features(ctx, features, n_channels, background, out, stream=None) -> None:
    """background: None or a host sequence of n_channels floats."""
    bg = None
    if background is not None:
        bg = (ctypes.c_float * n_channels)(*[float(x) for x in background])
    _check(load_library().gs_render_features(ctx, _dev_ptr(features), int(n_channels), bg, _dev_ptr(out),
                                             _stream_handle(stream)), "gs_render_features")


def gs_attribute(ctx, pixel_map, n_channels, out, stream=None) -> None:
    _check(load_library().gs_attribute(ctx, _dev_ptr(pixel_map), int(n_channels), _dev_ptr(out),
                                       _stream_handle(stream)), "gs_attribute")


def gs_debug_exp2(inp, out, stream=None) -> None:
    _check(load_library().gs_debug_exp2(_dev_ptr(inp), _dev_ptr(out), inp.numel(), _stream_handle(stream)),
           "gs_debug_exp2")


def gs_debug_export(ctx, kind, dst, stream=None) -> None:
    _check(load_library().gs_debug_export(ctx, int(kind), _dev_ptr(dst), dst.numel() * dst.element_size(),
                                          _stream_handle(stream)), "gs_debug_export")


def gs_debug_topk(ctx, k, ids, weights, stream=None) -> None:
    _check(load_library().gs_debug_topk(ctx, int(k), _dev_ptr(ids), _dev_ptr(weights), _stream_handle(stream)),
           "gs_debug_topk")


def gs_profile_enable(ctx, enable=True) -> None:
    _check(load_library().gs_profile_enable(ctx, int(bool(enable))), "gs_profile_enable")


def gs_profile_stages(ctx, stages) -> None:
    """Time only the named stages (names from STAGES)."""
    mask = 0
    for name in stages:
        mask |= 1 << STAGES.index(name)
    _check(load_library().gs_profile_stages(ctx, mask), "gs_profile_stages")


def gs_profile_read(ctx) -> dict:
    """{stage: (total ms, launches)} accumulated since the previous read."""
    ms = (ctypes.c_double * len(STAGES))()
    calls = (ctypes.c_int64 * len(STAGES))()
    _check(load_library().gs_profile_read(ctx, ms, calls, len(STAGES)), "gs_profile_read")
    return {name: (float(ms[i]), int(calls[i])) for i, name in enumerate(STAGES)}


# ---- convenience wrapper ----------------------------------------------------------------------------
def make_cameras(cams: np.ndarray):
    """[V, 16] float rows (R, t, fx, fy, cx, cy) -> ctypes array of gs_camera (host memory)."""
    cams = np.asarray(cams, dtype=np.float32)
    arr = (gs_camera * cams.shape[0])()
    for v, row in enumerate(cams):
        arr[v].R[:] = [float(x) for x in row[:9]]
        arr[v].t[:] = [float(x) for x in row[9:12]]
        arr[v].fx, arr[v].fy, arr[v].cx, arr[v].cy = (float(x) for x in row[12:16])
    return arr


class Rasterizer:
    """Device-resident scene + workspace; runs gs_project -> gs_bin_sort -> gs_render
    [-> gs_score_replay] on the current stream.  All buffers are torch tensors."""

    def __init__(self, means, quats, scales, opacities, sh, sh_degree, cams, width, height,
                 params: gs_params | None = None, max_pairs: int | None = None, device="cuda"):
        import torch
        load_library()
        self.torch = torch
        self.device = torch.device(device)
        f32 = dict(dtype=torch.float32, device=self.device)
        self.means = torch.as_tensor(means, **f32).contiguous()
        self.quats = torch.as_tensor(quats, **f32).contiguous()
        self.scales = torch.as_tensor(scales, **f32).contiguous()
        self.opacities = torch.as_tensor(opacities, **f32).contiguous()
        self.sh = torch.as_tensor(sh, **f32).contiguous()
        self.sh_degree = int(sh_degree)
        self.n = int(self.means.shape[0])
        self.cams_np = np.asarray(cams, dtype=np.float32).reshape(-1, 16)
        self.cams = make_cameras(self.cams_np)
        self.V = int(self.cams_np.shape[0])
        self.W, self.H = int(width), int(height)
        self.d = (self.sh_degree + 1) ** 2
        self.params = params if params is not None else gs_default_params()
        self.gauss = gs_gaussians(_dev_ptr(self.means), _dev_ptr(self.quats), _dev_ptr(self.scales),
                                  _dev_ptr(self.opacities), _dev_ptr(self.sh), self.n, self.sh_degree)
        self.ctx = None
        self.workspace = None
        self.n_pairs = None
        self._alloc(max_pairs if max_pairs else max(1, 4 * self.n * self.V))

    def _alloc(self, max_pairs: int):
        torch = self.torch
        self.close()
        self.max_pairs = int(max_pairs)
        dims = gs_dims(self.n, self.sh_degree, self.V, self.W, self.H, self.max_pairs)
        nbytes = gs_workspace_size(dims)
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        base = self.workspace.data_ptr()
        aligned = (base + 255) & ~255
        self.ctx = gs_context_create(dims, aligned, nbytes)

    def close(self):
        if self.ctx is not None:
            gs_context_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def project_and_bin(self, stream=None) -> int:
        while True:
            gs_project(self.ctx, self.gauss, self.cams, self.params, stream)
            st, n = gs_bin_sort(self.ctx, stream, raise_on_overflow=False)
            if st == GS_OK:
                self.n_pairs = n
                return n
            self._alloc(int(n * 1.25) + 1024)

    def new_outputs(self):
        torch = self.torch
        V, H, W = self.V, self.H, self.W
        color = torch.empty((V, H, W, 3), dtype=torch.float32, device=self.device)
        T = torch.empty((V, H, W), dtype=torch.float32, device=self.device)
        n = torch.empty((V, H, W), dtype=torch.int32, device=self.device)
        return color, T, n

    def render(self, outputs=None, stream=None):
        color, T, n = outputs if outputs is not None else self.new_outputs()
        gs_render(self.ctx, color, T, n, stream)
        return color, T, n

    def score_replay(self, observed, tokens=None, stream=None):
        torch = self.torch
        if tokens is None:
            tokens = torch.empty((self.n, 9 + 3 * self.d), dtype=torch.float32, device=self.device)
        obs = torch.as_tensor(observed, dtype=torch.float32, device=self.device).contiguous()
        gs_score_replay(self.ctx, obs, tokens, stream)
        return tokens

    def new_grads(self):
        """Gradient tensors shaped like the scene parameters."""
        torch = self.torch
        return {name: torch.empty_like(getattr(self, name))
                for name in ("means", "quats", "scales", "opacities", "sh")}

    def backward(self, grad_color, grads=None, stream=None):
        """Renderer backward: dL/d(means, quats, scales, opacities, sh) for dL/dC_hat = grad_color."""
        torch = self.torch
        grads = grads if grads is not None else self.new_grads()
        gC = torch.as_tensor(grad_color, dtype=torch.float32, device=self.device).contiguous()
        for name in ("means", "quats", "scales", "opacities", "sh"):
            t = grads.get(name)
            if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()
                                  or t.shape != getattr(self, name).shape):
                raise ValueError(f"gradient buffer {name} must be contiguous float32 of the parameter shape")
        ptrs = gs_gaussian_grads(*[grads[k].data_ptr() if grads.get(k) is not None else None
                                   for k in ("means", "quats", "scales", "opacities", "sh")])
        gs_backward(self.ctx, gC, ptrs, stream)
        return grads

    def render_features(self, features, background=None, out=None, stream=None):
        """Composite per-Gaussian features [n, C] with the render weights -> [V, H, W, C]."""
        torch = self.torch
        f = torch.as_tensor(features, dtype=torch.float32, device=self.device).contiguous()
        if f.dim() == 1:
            f = f.view(-1, 1)
        C = int(f.shape[1])
        if out is None:
            out = torch.empty((self.V, self.H, self.W, C), dtype=torch.float32, device=self.device)
        gs_render_features(self.ctx, f, C, background, out, stream)
        return out

    def attribute(self, pixel_map, out=None, stream=None):
        """Scatter a per-pixel map [V, H, W, C] back along the render weights -> [n, C]."""
        torch = self.torch
        m = torch.as_tensor(pixel_map, dtype=torch.float32, device=self.device).contiguous()
        C = int(m.shape[-1])
        if out is None:
            out = torch.empty((self.n, C), dtype=torch.float32, device=self.device)
        gs_attribute(self.ctx, m, C, out, stream)
        return out

    def topk(self, k, stream=None):
        """Debug: per pixel the k contributions of largest weight -> (ids [V,H,W,k] int32, weights [V,H,W,k])."""
        torch = self.torch
        ids = torch.empty((self.V, self.H, self.W, k), dtype=torch.int32, device=self.device)
        w = torch.empty((self.V, self.H, self.W, k), dtype=torch.float32, device=self.device)
        gs_debug_topk(self.ctx, k, ids, w, stream)
        return ids, w

    def step(self, observed, outputs=None, tokens=None, stream=None):
        """One pass of the whole path: project, bin/sort, render, replay -> tokens."""
        self.project_and_bin(stream)
        out = self.render(outputs, stream)
        tok = self.score_replay(observed, tokens, stream)
        return out, tok

    def export(self, kind):
        torch = self.torch
        VG = self.V * self.n
        if kind == GS_EXPORT_RECORDS:
            dst = torch.empty((4, VG, 4), dtype=torch.float32, device=self.device)
        elif kind == GS_EXPORT_DEPTH_KEYS:
            dst = torch.empty((VG,), dtype=torch.int32, device=self.device)
        elif kind == GS_EXPORT_SORTED_IDS:
            dst = torch.empty((max(self.n_pairs, 1),), dtype=torch.int32, device=self.device)
        elif kind == GS_EXPORT_RANGES:
            T = ((self.W + 15) // 16) * ((self.H + 15) // 16)
            dst = torch.empty((self.V * T, 2), dtype=torch.int32, device=self.device)
        elif kind == GS_EXPORT_PIXEL_STATS:
            dst = torch.empty((self.V, self.H, self.W, 2), dtype=torch.int32, device=self.device)
        else:
            raise ValueError(kind)
        gs_debug_export(self.ctx, kind, dst)
        return dst


def rasterizer_for_scene(scene, params: gs_params | None = None, max_pairs=None, device="cuda",
                         antialiased=False) -> Rasterizer:
    """Build a Rasterizer from a `scenes.Scene`-like object (means, quats, ... attributes)."""
    p = params if params is not None else gs_default_params()
    if params is None:
        p.background[:] = [float(x) for x in np.asarray(scene.background, dtype=np.float32)]
        p.antialiased = 1 if antialiased else 0
    return Rasterizer(scene.means, scene.quats, scene.scales, scene.opacities, scene.sh, scene.sh_degree,
                      scene.cams, scene.width, scene.height, params=p, max_pairs=max_pairs, device=device)
