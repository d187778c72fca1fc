"""CPU oracle for the Gaussian-splat render and the analytic score replay.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP path (``gaussian_splatting_rasterizer_amd``) and never
imports it; the two meet only through the seeded inputs of ``scenes``.

The arithmetic lives in ``gsr_oracle.c`` (plain C, float64 values, float32
canonical decisions, brute-force lists, explicit back-to-front suffix, literal
score sums, Jacobi eigenvalues, feature composite and attribution scatter, an
explicit chain-rule renderer backward);
this module builds it with gcc and wraps it
with ctypes.  Everything here follows the page "Research Proposal: Renderer
Score Tokens for Recurrent Gaussian Splatting" (Two-Stage Algorithm, Exact
Score Operators, Final Token and Updater).

Parity status: every function is pinned by a test under ``tests/`` (closed
forms, invariants, library routines, brute force, central finite differences)
except the numeric values of the constants the pages leave open (epsilon, the
suffix-denominator threshold, lambda, the 0.3 px dilation, the 0.1 eigenvalue
floor, the 1.3x field-of-view clamp, the near plane): those are our reading,
parity unpinned by the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gsr_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_OUT_DIR, "liboracle.so")
_lock = threading.Lock()
_lib = None

REC32_FIELDS = ["culled", "mx", "my", "mx_lo", "my_lo", "s1", "s2", "s3", "clip_bits", "opac", "pre_r", "pre_g",
                "pre_b", "depth", "radius", "x0", "y0", "x1", "y1", "clamp_bits"]
NACC_FIXED = 8  # W, A_alpha, A_mu_x, A_mu_y, |A_alpha|, |A_mu_x|, |A_mu_y|, n_pix
NACC_SENS = 9   # after the 6d SH sums: sensitivity of (A_alpha, A_mu_x, A_mu_y) to the residual, to the suffix,
                # and to the projected centre


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, OpenMP, no FMA contraction, no fast-math)."""
    os.makedirs(_OUT_DIR, exist_ok=True)
    if (not force and os.path.exists(_LIB_PATH)
            and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fno-finite-math-only", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64, I32, F32, F64 = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
        lib.orc_scene_new.restype = P
        lib.orc_scene_new.argtypes = [I32, I32, P, P, P, P, P, I32, P, I32, I32, F32, F32, P, I32]
        lib.orc_scene_free.argtypes = [P]
        lib.orc_get_records32.argtypes = [P, P]
        lib.orc_get_records64.argtypes = [P, P]
        lib.orc_build_lists.restype = I64
        lib.orc_build_lists.argtypes = [P]
        lib.orc_get_lists.argtypes = [P, P, P]
        lib.orc_tile_list_scan.restype = I64
        lib.orc_tile_list_scan.argtypes = [P, I64, P]
        lib.orc_select.argtypes = [P, P, I32]
        lib.orc_render_tiles.argtypes = [P, P, I64, P, F32, F32, P, P, P, P]
        lib.orc_pixel_work.argtypes = [P, P, I64, P]
        lib.orc_get_acc.argtypes = [P, P]
        lib.orc_tokens.argtypes = [P, F64, F64, P, P, P]
        lib.orc_eig3.argtypes = [P, P]
        lib.orc_exp2f.restype = F32
        lib.orc_exp2f.argtypes = [F32]
        lib.orc_exp2f_array.argtypes = [P, P, I64]
        lib.orc_constants.argtypes = [P]
        lib.orc_sh_basis64.argtypes = [P, I64, I32, P]
        lib.orc_values_reset.argtypes = [P]
        lib.orc_set_opacity64.argtypes = [P, I32, F64]
        lib.orc_set_sh64.argtypes = [P, I32, I32, I32, F64]
        lib.orc_set_mean2d64.argtypes = [P, I32, I32, F64, F64]
        lib.orc_set_mean3d64.argtypes = [P, I32, P]
        lib.orc_set_params64.argtypes = [P, I32, P]
        lib.orc_render_features.argtypes = [P, P, I32, P, P]
        lib.orc_attribute.argtypes = [P, P, I32, P]
        lib.orc_topk.argtypes = [P, I32, P, P]
        lib.orc_backward.argtypes = [P, P, P, I64, P, P]
        lib.orc_sh_basis_grad64.argtypes = [P, I64, I32, P]
        lib.orc_num_threads.restype = I32
        lib.orc_set_num_threads.argtypes = [I32]
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def exp2f(x: np.ndarray) -> np.ndarray:
    """The specified float32 2^x (decision exponential)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    lib.orc_exp2f_array(_ptr(x), _ptr(out), x.size)
    return out


def constants() -> dict:
    lib = _load()
    out = np.zeros(28, dtype=np.float32)
    lib.orc_constants(_ptr(out))
    return {"alpha_min": out[0], "exp2_coef": out[1:9].copy(), "half_log2e": out[9], "sh": out[11:27].copy()}


def sh_basis64(dirs: np.ndarray, d: int) -> np.ndarray:
    lib = _load()
    dirs = np.ascontiguousarray(dirs, dtype=np.float64).reshape(-1, 3)
    out = np.empty((dirs.shape[0], d), dtype=np.float64)
    lib.orc_sh_basis64(_ptr(dirs), dirs.shape[0], d, _ptr(out))
    return out


def sh_basis_grad64(dirs: np.ndarray, d: int) -> np.ndarray:
    """d B_k / d(x, y, z) of the SH polynomials, [n, d, 3] (no unit-norm projection)."""
    lib = _load()
    dirs = np.ascontiguousarray(dirs, dtype=np.float64).reshape(-1, 3)
    out = np.empty((dirs.shape[0], d, 3), dtype=np.float64)
    lib.orc_sh_basis_grad64(_ptr(dirs), dirs.shape[0], d, _ptr(out))
    return out


def eig3(A: np.ndarray) -> np.ndarray:
    lib = _load()
    A = np.ascontiguousarray(A, dtype=np.float64).reshape(3, 3)
    ev = np.empty(3, dtype=np.float64)
    lib.orc_eig3(_ptr(A), _ptr(ev))
    return ev


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on (used only to time it)."""
    _load().orc_set_num_threads(int(n))


class OracleScene:
    """One scene loaded into the oracle: per-(Gaussian, view) records, tile lists,
    per-pixel render/replay for chosen tiles, score sums for chosen Gaussians, tokens."""

    def __init__(self, scene, near=0.01, far=1e10, background=None, antialiased=False):
        lib = _load()
        self.lib = lib
        self.G, self.V = scene.n, scene.n_views
        self.W, self.H = scene.width, scene.height
        self.d = scene.d
        self.TX = (self.W + 15) // 16
        self.TY = (self.H + 15) // 16
        self.T = self.TX * self.TY
        bg = np.asarray(scene.background if background is None else background, dtype=np.float32)
        self._keep = [np.ascontiguousarray(a, dtype=np.float32) for a in
                      (scene.means, scene.quats, scene.scales, scene.opacities, scene.sh, scene.cams, bg)]
        m, q, s, o, sh, cams, bgc = self._keep
        self.handle = lib.orc_scene_new(self.G, scene.sh_degree, _ptr(m), _ptr(q), _ptr(s), _ptr(o), _ptr(sh),
                                        self.V, _ptr(cams), self.W, self.H, near, far, _ptr(bgc),
                                        1 if antialiased else 0)
        if not self.handle:
            raise ValueError("oracle rejected the scene")
        self.n_pairs = None
        self.n_sel = None
        self._sel = None

    def close(self):
        if self.handle:
            self.lib.orc_scene_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- records -------------------------------------------------------------
    def records32(self) -> np.ndarray:
        out = np.empty((self.V, self.G, 20), dtype=np.float32)
        self.lib.orc_get_records32(self.handle, _ptr(out))
        return out

    def records64(self) -> np.ndarray:
        out = np.empty((self.V, self.G, 15), dtype=np.float64)
        self.lib.orc_get_records64(self.handle, _ptr(out))
        return out

    # -- lists ---------------------------------------------------------------
    def build_lists(self) -> int:
        self.n_pairs = int(self.lib.orc_build_lists(self.handle))
        return self.n_pairs

    def lists(self):
        if self.n_pairs is None:
            self.build_lists()
        starts = np.empty(self.V * self.T + 1, dtype=np.int64)
        ids = np.empty(max(self.n_pairs, 1), dtype=np.int32)
        self.lib.orc_get_lists(self.handle, _ptr(starts), _ptr(ids))
        return starts, ids[: self.n_pairs]

    def tile_list_scan(self, tile: int) -> np.ndarray:
        out = np.empty(max(self.G, 1), dtype=np.int32)
        n = self.lib.orc_tile_list_scan(self.handle, int(tile), _ptr(out))
        return out[:n].copy()

    # -- render / replay -------------------------------------------------------
    def select(self, gids=None):
        if gids is None:
            self.lib.orc_select(self.handle, None, -1)
            self.n_sel = self.G
            self._sel = None
        else:
            gids = np.ascontiguousarray(gids, dtype=np.int32)
            self._sel = gids
            self.lib.orc_select(self.handle, _ptr(gids), gids.size)
            self.n_sel = gids.size

    def render(self, tiles=None, obs=None, eps=1e-6, den_min=1e-3):
        """Render (and replay when `obs` is given) the chosen tiles (all by default).
        Returns colour [V,H,W,3] f64, T_final [V,H,W] f32, n_contrib [V,H,W] i32,
        T_final64 [V,H,W] f64; pixels outside the chosen tiles are NaN / -1."""
        if self.n_pairs is None:
            self.build_lists()
        if tiles is None:
            tiles = np.arange(self.V * self.T, dtype=np.int64)
        tiles = np.ascontiguousarray(tiles, dtype=np.int64)
        if obs is not None:
            obs = np.ascontiguousarray(obs, dtype=np.float32)
            assert obs.shape == (self.V, self.H, self.W, 3)
            if self.n_sel is None:
                self.select(None)
        color = np.full((self.V, self.H, self.W, 3), np.nan, dtype=np.float64)
        T = np.full((self.V, self.H, self.W), np.nan, dtype=np.float32)
        n = np.full((self.V, self.H, self.W), -1, dtype=np.int32)
        T64 = np.full((self.V, self.H, self.W), np.nan, dtype=np.float64)
        self.lib.orc_render_tiles(self.handle, _ptr(tiles), tiles.size,
                                  _ptr(obs) if obs is not None else None, eps, den_min,
                                  _ptr(color), _ptr(T), _ptr(n), _ptr(T64))
        return color, T, n, T64

    def pixel_work(self, tiles=None) -> np.ndarray:
        """Work counts of the render pass per pixel of the chosen tiles (all by default):
        [V,H,W,2] uint32 = (list entries examined up to and including the one at which the
        pixel stopped, or the whole list; those of them past the distance cut).  Pixels
        outside the chosen tiles hold 0xffffffff."""
        if self.n_pairs is None:
            self.build_lists()
        if tiles is None:
            tiles = np.arange(self.V * self.T, dtype=np.int64)
        tiles = np.ascontiguousarray(tiles, dtype=np.int64)
        out = np.full((self.V, self.H, self.W, 2), 0xFFFFFFFF, dtype=np.uint32)
        self.lib.orc_pixel_work(self.handle, _ptr(tiles), tiles.size, _ptr(out))
        return out

    def acc(self) -> np.ndarray:
        na = NACC_FIXED + 6 * self.d + NACC_SENS
        out = np.empty((self.n_sel, self.V, na), dtype=np.float64)
        self.lib.orc_get_acc(self.handle, _ptr(out))
        return out

    def tokens(self, eps=1e-6, lam=1.0, with_A=False):
        D = 9 + 3 * self.d
        tok = np.empty((self.n_sel, D), dtype=np.float64)
        A = np.empty((self.n_sel, 9), dtype=np.float64) if with_A else None
        q = np.empty((self.n_sel, self.V), dtype=np.float64) if with_A else None
        self.lib.orc_tokens(self.handle, eps, lam, _ptr(tok), _ptr(A) if with_A else None,
                            _ptr(q) if with_A else None)
        if with_A:
            return tok, A.reshape(-1, 3, 3), q
        return tok

    def tiles_of(self, gids) -> np.ndarray:
        """Every tile (global id v*T + t) inside the rectangles of the given Gaussians."""
        rec = self.records32()
        out = set()
        for g in np.asarray(gids).ravel():
            for v in range(self.V):
                r = rec[v, int(g)]
                if r[0]:
                    continue
                x0, y0, x1, y1 = (int(r[15]), int(r[16]), int(r[17]), int(r[18]))
                for ty in range(y0, y1):
                    for tx in range(x0, x1):
                        out.add(v * self.T + ty * self.TX + tx)
        return np.array(sorted(out), dtype=np.int64)

    # -- feature composite and attribution scatter ----------------------------
    def render_features(self, features, background=None):
        """Composite per-Gaussian features [G, C] with the render weights:
        [V, H, W, C] float64 = sum_k T_k alpha_k f_k + T_final * background."""
        if self.n_pairs is None:
            self.build_lists()
        f = np.ascontiguousarray(features, dtype=np.float32).reshape(self.G, -1)
        C = f.shape[1]
        bg = None if background is None else np.ascontiguousarray(background, dtype=np.float32).reshape(C)
        out = np.empty((self.V, self.H, self.W, C), dtype=np.float64)
        self.lib.orc_render_features(self.handle, _ptr(f), C, _ptr(bg) if bg is not None else None, _ptr(out))
        return out

    def attribute(self, pixel_map):
        """Attribution scatter of a per-pixel map [V, H, W, C]: [G, C] float64 =
        sum over views and pixels of T alpha * map."""
        if self.n_pairs is None:
            self.build_lists()
        m = np.ascontiguousarray(pixel_map, dtype=np.float32)
        C = m.shape[-1]
        assert m.shape == (self.V, self.H, self.W, C)
        out = np.empty((self.G, C), dtype=np.float64)
        self.lib.orc_attribute(self.handle, _ptr(m), C, _ptr(out))
        return out

    def topk(self, K):
        """Per pixel the K contributions of largest weight T alpha (decreasing, list order
        on ties): ids [V, H, W, K] int32 (-1 unused), weights [V, H, W, K] float64."""
        if self.n_pairs is None:
            self.build_lists()
        ids = np.empty((self.V, self.H, self.W, K), dtype=np.int32)
        w = np.empty((self.V, self.H, self.W, K), dtype=np.float64)
        self.lib.orc_topk(self.handle, int(K), _ptr(ids), _ptr(w))
        return ids, w

    # -- renderer backward -----------------------------------------------------
    def backward(self, grad_color, with_image_sums=False, tiles=None):
        """Vector-Jacobian product of the colour image with `grad_color` [V,H,W,3]:
        gradients [G, 11 + 3 d] = [mean 3, quaternion 4, scale 3, opacity 1, SH d*3]
        (float64).  With `with_image_sums`, also the per-(view, Gaussian) image-space
        sums [V, G, 9] = dL/d(mx, my, ca, cb, cc, o, c_r, c_g, c_b).  With `tiles`
        (global tile ids), only those tiles are walked: exact for the Gaussians
        whose rectangles they cover (`tiles_of`)."""
        if self.n_pairs is None:
            self.build_lists()
        gC = np.ascontiguousarray(grad_color, dtype=np.float32)
        assert gC.shape == (self.V, self.H, self.W, 3)
        out = np.empty((self.G, 11 + 3 * self.d), dtype=np.float64)
        g2d = np.empty((self.V, self.G, 9), dtype=np.float64) if with_image_sums else None
        if tiles is not None:
            tiles = np.ascontiguousarray(tiles, dtype=np.int64)
        self.lib.orc_backward(self.handle, _ptr(gC), _ptr(tiles) if tiles is not None else None,
                              0 if tiles is None else tiles.size, _ptr(out),
                              _ptr(g2d) if with_image_sums else None)
        return (out, g2d) if with_image_sums else out

    def params64(self, g) -> np.ndarray:
        """The 11 float64 parameter values of Gaussian g: mean, quaternion, scale, opacity."""
        return np.concatenate([self._keep[0][g], self._keep[1][g], self._keep[2][g],
                               self._keep[3][g:g + 1]]).astype(np.float64)

    def set_params64(self, g, prm):
        prm = np.ascontiguousarray(prm, dtype=np.float64)
        assert prm.shape == (11,)
        self.lib.orc_set_params64(self.handle, int(g), _ptr(prm))

    # -- finite-difference probes ---------------------------------------------
    def values_reset(self):
        self.lib.orc_values_reset(self.handle)

    def set_opacity64(self, g, o):
        self.lib.orc_set_opacity64(self.handle, int(g), float(o))

    def set_sh64(self, g, k, ch, value):
        self.lib.orc_set_sh64(self.handle, int(g), int(k), int(ch), float(value))

    def set_mean2d64(self, g, v, mx, my):
        self.lib.orc_set_mean2d64(self.handle, int(g), int(v), float(mx), float(my))

    def set_mean3d64(self, g, mu):
        mu = np.ascontiguousarray(mu, dtype=np.float64)
        self.lib.orc_set_mean3d64(self.handle, int(g), _ptr(mu))


def render_observation(scene, **kw) -> np.ndarray:
    """Observed image of a workload: the oracle render of the scene with perturbed
    means plus the scene's pixel noise, rounded to float32."""
    o = OracleScene(scene.perturbed(), **kw)
    try:
        color, _, _, _ = o.render()
    finally:
        o.close()
    return (color + scene.pixel_noise.astype(np.float64)).astype(np.float32)


def full_reference(scene, obs, eps=1e-6, den_min=1e-3, lam=1.0, gids=None, tiles=None, antialiased=False):
    """Convenience: render + replay + tokens.  With `gids`, only those Gaussians'
    tokens are computed, from every tile their rectangles touch (plus `tiles`)."""
    o = OracleScene(scene, antialiased=antialiased)
    t0 = time.perf_counter()
    o.build_lists()
    if gids is None:
        o.select(None)
        render_tiles = tiles
    else:
        o.select(gids)
        render_tiles = o.tiles_of(gids)
        if tiles is not None:
            render_tiles = np.union1d(render_tiles, np.asarray(tiles, dtype=np.int64))
    color, T, n, T64 = o.render(tiles=render_tiles, obs=obs, eps=eps, den_min=den_min)
    tok = o.tokens(eps=eps, lam=lam)
    elapsed = time.perf_counter() - t0
    return {"oracle": o, "color": color, "T": T, "n": n, "T64": T64, "tokens": tok,
            "seconds": elapsed}


TOKEN_RTOL = 1e-3          # per block, relative to the block's own norm (Renderer Score Tokens plan, Block 0)
TERM_RTOL = 1e-4           # float32 rounding of one signed per-pixel score term, relative to its magnitude


CENTRE_ATOL = 2.0 ** -20    # px: half an ulp of a tile-relative coordinate below 16 (float32)


def token_block_errors(o, z, zr, eps=1e-6, catol=1e-5, term_rtol=TERM_RTOL, centre_atol=CENTRE_ATOL):
    """Per-block comparison of tokens `z` [n_sel, 9 + 3d] with the oracle's `zr` for the
    Gaussians selected in the OracleScene `o` (after its render + replay).

    Blocks (Final Token and Updater): b_mu (3), s_alpha (1), s_SH (3d), stats (log Q,
    e~ (3), log(tr A + eps)).  Each block's error norm is held to TOKEN_RTOL of the
    block's own norm plus a floor that bounds what a correct float32 evaluation may
    move it by:
      * the signed-sum blocks (b_mu, s_alpha, s_SH) are sums of per-pixel terms that may
        cancel: `term_rtol` (default TERM_RTOL) of the sum of the terms' magnitudes, plus what the residual
        and the suffix may move when the rendered colour is off by at most `catol` per
        channel (the colour tolerance; the suffix is a tail of the same composite): the
        oracle's sensitivity sums times `catol`, plus what moving the projected centre by
        `centre_atol` px (the float32 rounding of a tile-relative centre; it decides the
        sign of the centre terms at pixels that sit on the centre) moves them by; for b_mu
        these are pulled back through |J| like the score itself;
      * the statistics block: 10 * catol absolute per entry (logarithms of float32 sums
        of positive terms, and eigenvalue ratios <= 1).
    Returns {block: (max ratio of error to bound, argmax)}; a ratio <= 1 passes."""
    acc = o.acc()                                   # [n_sel, V, na]
    d, V = o.d, o.V
    na = acc.shape[2]
    sens = acc[:, :, na - NACC_SENS:]
    Q = eps + np.sum(eps + acc[:, :, 0], axis=1)    # [n_sel]
    sel = np.arange(o.G) if o._sel is None else o._sel
    r64 = o.records64()[:, sel]                     # [V, n_sel, 15]
    culled = o.records32()[:, sel, 0] != 0          # [V, n_sel]
    J = np.where(culled[:, :, None], 0.0, r64[:, :, 9:15]).reshape(V, -1, 2, 3)
    z = np.asarray(z, dtype=np.float64)
    zr = np.asarray(zr, dtype=np.float64)
    out = {}

    def report(name, err, bound):
        ratio = err / bound
        k = int(np.argmax(ratio)) if ratio.size else 0
        out[name] = (float(ratio.max()) if ratio.size else 0.0, k)

    # b_mu = (1/Q) sum_v J_v^T A_mu,v
    f_mu = (term_rtol * acc[:, :, 5:7] + catol * (sens[:, :, 1:3] + sens[:, :, 4:6])
            + centre_atol * sens[:, :, 7:9])                                              # [n_sel, V, 2]
    floor_mu = np.einsum("vgrj,gvr->gj", np.abs(J), f_mu) / Q[:, None]
    report("b_mu", np.linalg.norm(z[:, 0:3] - zr[:, 0:3], axis=1),
           TOKEN_RTOL * np.linalg.norm(zr[:, 0:3], axis=1) + np.linalg.norm(floor_mu, axis=1) + 1e-12)
    # s_alpha = (1/Q) sum_v A_alpha,v
    floor_a = (term_rtol * acc[:, :, 4] + catol * (sens[:, :, 0] + sens[:, :, 3])
               + centre_atol * sens[:, :, 6]).sum(axis=1) / Q
    report("s_alpha", np.abs(z[:, 3] - zr[:, 3]), TOKEN_RTOL * np.abs(zr[:, 3]) + floor_a + 1e-12)
    # s_SH = (1/Q) sum_v M^color B (x) U_c,v ; |B_k| <= 1 for degree <= 3
    k0 = NACC_FIXED
    abs_sh = acc[:, :, k0 + 3 * d: k0 + 6 * d].sum(axis=1)
    W = acc[:, :, 0].sum(axis=1)
    floor_sh = (term_rtol * abs_sh + catol * W[:, None]) / Q[:, None]
    sh = slice(4, 4 + 3 * d)
    report("s_sh", np.linalg.norm(z[:, sh] - zr[:, sh], axis=1),
           TOKEN_RTOL * np.linalg.norm(zr[:, sh], axis=1) + np.linalg.norm(floor_sh, axis=1) + 1e-12)
    report("s_sh_elementwise", np.abs(z[:, sh] - zr[:, sh]).ravel(),
           (TOKEN_RTOL * np.abs(zr[:, sh]) + floor_sh + 1e-12).ravel())
    # statistics block
    st = slice(4 + 3 * d, 9 + 3 * d)
    report("stats", np.linalg.norm(z[:, st] - zr[:, st], axis=1),
           TOKEN_RTOL * np.linalg.norm(zr[:, st], axis=1) + 1e-12)
    report("stats_elementwise", np.abs(z[:, st] - zr[:, st]).ravel(),
           np.full(z[:, st].size, 10.0 * catol))
    return out
