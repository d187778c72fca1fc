"""Seeded synthetic scenes, cameras and observation noise for the five workloads.

This module only draws inputs.  It holds none of the renderer's or the score
replay's arithmetic: it produces Gaussian parameters (activated scales and
opacities, unit quaternions, SH coefficients), pinhole cameras, a perturbed
copy of the means and per-pixel noise.  The observed image of a workload is
"the render of the scene with perturbed means, plus pixel noise"; whoever
consumes a scene renders the perturbed copy with its own renderer.

The 3D Gaussian primitive (centre, rotation, scale, opacity, SH colour) and the
two placements used below -- pixel-aligned back-projection of a depth per input
pixel, and anchors with K local offsets -- follow the ATSplat summary page
("前置知识: 3DGS", "Feed-forward 3DGS / pixel-aligned", "核心方法" anchor-plus-offset
placement).  The two-plane/three-layer occlusion toy follows the Block 0
diagnostic of the Renderer Score Tokens experiment plan.  Datasets named on the
pages (DL3DV, RealEstate10K) are not available here; these scenes stand in for
their shapes and sizes.

Conventions (shared by every consumer):
  * cameras are world->camera rigid transforms x_cam = R x_world + t, stored
    as float32 rows [R (9, row-major), t (3), fx, fy, cx, cy]; all views of a
    scene share one image size (W, H);
  * quaternions are (w, x, y, z);
  * scales and opacities are already activated (exp and sigmoid applied in
    float64, then rounded to float32);
  * SH coefficients are laid out [G, d, 3] with d = (degree + 1)^2.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Scene", "make_scene", "rotated_clip_scene", "CONFIG_NAMES", "c1_occlusion_toy", "c2_resplat_step",
           "c3_atsplat_compact", "c4_dense_pixel_aligned", "c5_multiview_layers", "view_sweep"]

SH_C0 = 0.28209479177387814  # 1 / (2 sqrt(pi)); used only to draw degree-0 colours


@dataclasses.dataclass
class Scene:
    name: str
    means: np.ndarray          # [G, 3] float32
    quats: np.ndarray          # [G, 4] float32, (w, x, y, z), unit up to rounding
    scales: np.ndarray         # [G, 3] float32, > 0
    opacities: np.ndarray      # [G] float32, in (0, 1)
    sh: np.ndarray             # [G, d, 3] float32
    sh_degree: int
    cams: np.ndarray           # [V, 16] float32
    width: int
    height: int
    background: np.ndarray     # [3] float32
    means_perturbed: np.ndarray  # [G, 3] float32 (means + N(0, 0.01^2))
    pixel_noise: np.ndarray    # [V, H, W, 3] float32, N(0, 0.01^2)
    notes: dict

    @property
    def n(self) -> int:
        return int(self.means.shape[0])

    @property
    def n_views(self) -> int:
        return int(self.cams.shape[0])

    @property
    def d(self) -> int:
        return (self.sh_degree + 1) ** 2

    def perturbed(self) -> "Scene":
        """Same scene with the perturbed means (used to render the observation)."""
        return dataclasses.replace(self, means=self.means_perturbed)


def _camera(center, f, W, H) -> np.ndarray:
    """Camera looking down +z with identity rotation and its centre at `center`."""
    row = np.zeros(16, dtype=np.float64)
    row[0] = row[4] = row[8] = 1.0
    row[9:12] = -np.asarray(center, dtype=np.float64)
    row[12] = row[13] = f
    row[14] = W / 2.0
    row[15] = H / 2.0
    return row


def _unit_quats(rng, n) -> np.ndarray:
    q = rng.standard_normal((n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    return q


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _finish(name, rng, means, quats, log_scales, logits, sh, sh_degree, cams, W, H, notes,
            background=(0.0, 0.0, 0.0)) -> Scene:
    """Draw the mean perturbation and pixel noise (in that order) and cast to float32."""
    G = means.shape[0]
    V = cams.shape[0]
    pert = rng.standard_normal((G, 3)) * 0.01
    noise = (rng.standard_normal((V, H, W, 3)) * 0.01).astype(np.float32)
    means32 = means.astype(np.float32)
    return Scene(
        name=name,
        means=means32,
        quats=quats.astype(np.float32),
        scales=np.exp(log_scales).astype(np.float32),
        opacities=_sigmoid(logits).astype(np.float32),
        sh=sh.astype(np.float32).reshape(G, (sh_degree + 1) ** 2, 3),
        sh_degree=sh_degree,
        cams=np.ascontiguousarray(cams, dtype=np.float32),
        width=int(W), height=int(H),
        background=np.asarray(background, dtype=np.float32),
        means_perturbed=(means + pert).astype(np.float32),
        pixel_noise=noise,
        notes=notes,
    )


def _pixel_aligned(rng, cams, W, H, f, depth_lo, depth_hi):
    """One Gaussian per pixel of each source camera: centre = camera centre +
    depth * K^-1 (u + 0.5, v + 0.5, 1) (identity rotations), view-major, row-major."""
    V = cams.shape[0]
    u = (np.arange(W) + 0.5 - W / 2.0) / f
    v = (np.arange(H) + 0.5 - H / 2.0) / f
    uu, vv = np.meshgrid(u, v)                      # [H, W]
    out = np.empty((V, H, W, 3), dtype=np.float64)
    for i in range(V):
        z = rng.uniform(depth_lo, depth_hi, size=(H, W))
        centre = -cams[i, 9:12]
        out[i, :, :, 0] = centre[0] + z * uu
        out[i, :, :, 1] = centre[1] + z * vv
        out[i, :, :, 2] = centre[2] + z
    return out.reshape(-1, 3)


def c1_occlusion_toy(seed=1, W=64, H=64, n=2000) -> Scene:
    """Two-plane/three-layer occlusion toy: one 64x64 view, Gaussians split
    equally over depth planes z = 2, 3, 4 with +-0.05 jitter, filling the frustum,
    log-scales N(-3, 0.3), opacity logits N(0, 1), SH degree 0 with colour U(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f = float(W)
    cams = np.stack([_camera((0, 0, 0), f, W, H)])
    counts = [n // 3 + (1 if i < n % 3 else 0) for i in range(3)]   # 667/667/666 for n = 2000
    planes = [2.0, 3.0, 4.0]
    pos = []
    for z0, c in zip(planes, counts):
        z = z0 + rng.uniform(-0.05, 0.05, size=c)
        x = rng.uniform(-0.5, 0.5, size=c) * z * (W / f)
        y = rng.uniform(-0.5, 0.5, size=c) * z * (H / f)
        pos.append(np.stack([x, y, z], axis=1))
    means = np.concatenate(pos, axis=0)
    quats = _unit_quats(rng, n)
    log_scales = rng.normal(-3.0, 0.3, size=(n, 3))
    logits = rng.normal(0.0, 1.0, size=n)
    u = rng.uniform(0.0, 1.0, size=(n, 1, 3))
    sh = (u - 0.5) / SH_C0
    return _finish("c1_occlusion_toy", rng, means, quats, log_scales, logits, sh, 0, cams, W, H,
                   {"planes": planes, "counts": counts})


def c2_resplat_step(seed=2, n_views=8, W=448, H=256) -> Scene:
    """ReSplat-like step: 8 views 256x448 (fx = fy = 448, centres 0.1 m apart on
    the x axis), one pixel-aligned Gaussian per pixel of every view (depth U(1, 10)),
    SH degree 3 with coefficients N(0, 0.2^2), opacity logits N(0, 1), log-scales
    N(-4.5, 0.5).  Every view renders all Gaussians."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f = float(W)
    cams = np.stack([_camera((0.1 * (i - (n_views - 1) / 2.0), 0, 0), f, W, H)
                     for i in range(n_views)])
    means = _pixel_aligned(rng, cams, W, H, f, 1.0, 10.0)
    n = means.shape[0]
    quats = _unit_quats(rng, n)
    log_scales = rng.normal(-4.5, 0.5, size=(n, 3))
    logits = rng.normal(0.0, 1.0, size=n)
    sh = rng.normal(0.0, 0.2, size=(n, 16, 3))
    return _finish("c2_resplat_step", rng, means, quats, log_scales, logits, sh, 3, cams, W, H,
                   {"placement": "pixel-aligned", "depth": [1, 10]})


def c3_atsplat_compact(seed=3, n_anchors=19456, K=16, W=960, H=512) -> Scene:
    """ATSplat-like compact scene: one 512x960 view (fx = fy = 960), anchors
    uniform in a 10 m box in front of the camera ([-5, 5]^2 x [10, 20]), K = 16
    offsets N(0, 0.05^2) per anchor (anchor-major), SH degree 3 N(0, 0.2^2),
    anisotropic log-scales N(-3.5, 0.7), opacity logits N(0.5, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f = float(W)
    cams = np.stack([_camera((0, 0, 0), f, W, H)])
    anchors = np.stack([rng.uniform(-5, 5, n_anchors), rng.uniform(-5, 5, n_anchors),
                        rng.uniform(10, 20, n_anchors)], axis=1)
    offsets = rng.normal(0.0, 0.05, size=(n_anchors, K, 3))
    means = (anchors[:, None, :] + offsets).reshape(-1, 3)
    n = means.shape[0]
    quats = _unit_quats(rng, n)
    log_scales = rng.normal(-3.5, 0.7, size=(n, 3))
    logits = rng.normal(0.5, 1.0, size=n)
    sh = rng.normal(0.0, 0.2, size=(n, 16, 3))
    return _finish("c3_atsplat_compact", rng, means, quats, log_scales, logits, sh, 3, cams, W, H,
                   {"anchors": n_anchors, "K": K})


def c4_dense_pixel_aligned(seed=4, n_sources=12, W=960, H=512) -> Scene:
    """Dense pixel-aligned high-res: 12 source cameras (0.1 m apart) x 512x960
    pixels back-projected at depth U(1, 20) (5,898,240 Gaussians, source-major,
    row-major) rendered into one target camera at the origin; SH degree 3
    N(0, 0.2^2); scale and opacity distributions of the ReSplat-like step."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f = float(W)
    sources = np.stack([_camera((0.1 * (j - (n_sources - 1) / 2.0), 0, 0), f, W, H)
                        for j in range(n_sources)])
    means = _pixel_aligned(rng, sources, W, H, f, 1.0, 20.0)
    n = means.shape[0]
    quats = _unit_quats(rng, n)
    log_scales = rng.normal(-4.5, 0.5, size=(n, 3))
    logits = rng.normal(0.0, 1.0, size=n)
    sh = rng.normal(0.0, 0.2, size=(n, 16, 3))
    cams = np.stack([_camera((0, 0, 0), f, W, H)])
    return _finish("c4_dense_pixel_aligned", rng, means, quats, log_scales, logits, sh, 3, cams, W, H,
                   {"sources": n_sources, "depth": [1, 20]})


def c5_multiview_layers(seed=5, n_views=8, W=448, H=256, n=500_000) -> Scene:
    """Multi-view score averaging: 8 views 256x448 (fx = fy = 448, centres 0.05 m
    apart) sharing one scene of three layers at z = 4, 3, 2 (+-0.05 jitter).  Each
    layer is a centred rectangle covering 100 % (widened to the union of the
    frusta) / 70 % / 40 % of the centre view's image area, with Gaussian counts in
    proportion to area (238,095 / 166,667 / 95,238), so about 40 % of the pixels
    see all three layers.  Log-scales N(-5, 0.3), opacity logits N(-2.5, 1),
    SH degree 3 N(0, 0.2^2)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f = float(W)
    offs = [0.05 * (i - (n_views - 1) / 2.0) for i in range(n_views)]
    cams = np.stack([_camera((o, 0, 0), f, W, H) for o in offs])
    fracs = [1.0, 0.7, 0.4]
    depths = [4.0, 3.0, 2.0]
    base = n / sum(fracs)
    counts = [int(round(base * fr)) for fr in fracs]
    counts[0] = n - counts[1] - counts[2]
    pos = []
    for z0, fr, c in zip(depths, fracs, counts):
        half_w = 0.5 * z0 * (W / f) * math.sqrt(fr)
        half_h = 0.5 * z0 * (H / f) * math.sqrt(fr)
        if fr == 1.0:
            half_w += max(abs(o) for o in offs)
        x = rng.uniform(-half_w, half_w, size=c)
        y = rng.uniform(-half_h, half_h, size=c)
        z = z0 + rng.uniform(-0.05, 0.05, size=c)
        pos.append(np.stack([x, y, z], axis=1))
    means = np.concatenate(pos, axis=0)
    quats = _unit_quats(rng, n)
    log_scales = rng.normal(-5.0, 0.3, size=(n, 3))
    logits = rng.normal(-2.5, 1.0, size=n)
    sh = rng.normal(0.0, 0.2, size=(n, 16, 3))
    return _finish("c5_multiview_layers", rng, means, quats, log_scales, logits, sh, 3, cams, W, H,
                   {"layer_counts": counts, "layer_depths": depths, "layer_area_fracs": fracs,
                    "three_layer_pixel_fraction": fracs[2]})


def view_sweep(n_views=8, W=448, H=256, n_sources=8, seed=6) -> Scene:
    """View/resolution scaling scene: the Gaussians of the ReSplat-like step
    (one pixel-aligned Gaussian per pixel of `n_sources` source views 0.1 m apart,
    depth U(1, 10), log-scales N(-4.5, 0.5), logits N(0, 1), SH degree 3 N(0, 0.2^2))
    rendered by `n_views` target cameras spread evenly over the same baseline, so
    the Gaussian set is fixed while the view count and resolution vary."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f = float(W)
    src = np.stack([_camera((0.1 * (i - (n_sources - 1) / 2.0), 0, 0), f, W, H) for i in range(n_sources)])
    half = 0.05 * (n_sources - 1)
    xs = np.linspace(-half, half, n_views) if n_views > 1 else np.zeros(1)
    cams = np.stack([_camera((float(x), 0, 0), f, W, H) for x in xs])
    means = _pixel_aligned(rng, src, W, H, f, 1.0, 10.0)
    n = means.shape[0]
    quats = _unit_quats(rng, n)
    log_scales = rng.normal(-4.5, 0.5, size=(n, 3))
    logits = rng.normal(0.0, 1.0, size=n)
    sh = rng.normal(0.0, 0.2, size=(n, 16, 3))
    return _finish("view_sweep", rng, means, quats, log_scales, logits, sh, 3, cams, W, H,
                   {"placement": "pixel-aligned", "depth": [1, 10], "sources": n_sources})


CONFIG_NAMES = {
    1: "c1_occlusion_toy",
    2: "c2_resplat_step",
    3: "c3_atsplat_compact",
    4: "c4_dense_pixel_aligned",
    5: "c5_multiview_layers",
}

_MAKERS = {1: c1_occlusion_toy, 2: c2_resplat_step, 3: c3_atsplat_compact,
           4: c4_dense_pixel_aligned, 5: c5_multiview_layers}


def _rot_xyz(ax, ay, az) -> np.ndarray:
    cx, sx, cy, sy, cz, sz = np.cos(ax), np.sin(ax), np.cos(ay), np.sin(ay), np.cos(az), np.sin(az)
    Rx = np.array([[1, 0, 0], [0, cx, -sx], [0, sx, cx]])
    Ry = np.array([[cy, 0, sy], [0, 1, 0], [-sy, 0, cy]])
    Rz = np.array([[cz, -sz, 0], [sz, cz, 0], [0, 0, 1]])
    return Rz @ Ry @ Rx


def rotated_clip_scene(seed=21, n=16, W=32, H=32, sh_degree=3,
                       angles=((0.04, -0.06, 0.03), (-0.03, 0.05, -0.02))) -> Scene:
    """tiny_scene seen by rotated cameras (same centres; one per entry of `angles`,
    rotations Rz Ry Rx), plus two large Gaussians whose centres lie beyond 1.3x
    the half field of view of view 0, one in x and one in y."""
    sc = tiny_scene(seed=seed, n=n, n_views=len(angles), W=W, H=H, sh_degree=sh_degree)
    cams = np.array(sc.cams, dtype=np.float64)
    for i, a in enumerate(angles):
        R = _rot_xyz(*a)
        centre = -cams[i, 9:12]               # identity-rotation camera: t = -centre
        cams[i, 0:9] = R.reshape(-1)
        cams[i, 9:12] = -R @ centre
    cams = cams.astype(np.float32)
    R0 = cams[0, 0:9].reshape(3, 3).astype(np.float64)
    t0 = cams[0, 9:12].astype(np.float64)
    extra = np.array([R0.T @ (np.array([tx * 3.0, ty * 3.0, 3.0]) - t0)
                      for tx, ty in [(0.8, 0.1), (-0.1, -0.78)]], dtype=np.float32)
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    d = sc.d
    sh_x = rng.normal(0, 0.3, size=(2, d, 3))
    sh_x[:, 0, :] = 0.3 / SH_C0
    q_x = _unit_quats(rng, 2)
    return dataclasses.replace(
        sc, name="rotated_clip", cams=cams,
        means=np.concatenate([sc.means, extra]),
        quats=np.concatenate([sc.quats, q_x.astype(np.float32)]),
        scales=np.concatenate([sc.scales, np.array([[0.6, 0.45, 0.5], [0.5, 0.6, 0.4]], np.float32)]),
        opacities=np.concatenate([sc.opacities, np.array([0.7, 0.6], np.float32)]),
        sh=np.concatenate([sc.sh, sh_x.astype(np.float32)]),
        means_perturbed=np.concatenate([sc.means_perturbed, extra]))


def make_scene(config: int, **overrides) -> Scene:
    """Build workload `config` (1..5) with seed = config unless overridden."""
    return _MAKERS[config](**overrides)


def tiny_scene(seed=11, n=12, n_views=2, W=32, H=32, sh_degree=2, depth=(2.5, 3.5), log_scale=(-2.3, 0.3),
               logit=(0.0, 1.0), background=(0.1, 0.2, 0.3), spread=0.45, baseline=0.15) -> Scene:
    """Small scene for finite-difference and closed-form checks: `n` Gaussians in a
    box in front of `n_views` cameras placed `baseline` apart on the x axis,
    SH coefficients N(0, 0.3^2) with the DC term set so colours sit near 0.5."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f = float(W)
    cams = np.stack([_camera((baseline * (i - (n_views - 1) / 2.0), 0, 0), f, W, H)
                     for i in range(n_views)])
    z = rng.uniform(depth[0], depth[1], size=n)
    x = rng.uniform(-spread, spread, size=n) * z * (W / f)
    y = rng.uniform(-spread, spread, size=n) * z * (H / f)
    means = np.stack([x, y, z], axis=1)
    quats = _unit_quats(rng, n)
    log_scales = rng.normal(log_scale[0], log_scale[1], size=(n, 3))
    logits = rng.normal(logit[0], logit[1], size=n)
    d = (sh_degree + 1) ** 2
    sh = rng.normal(0.0, 0.3, size=(n, d, 3))
    sh[:, 0, :] = rng.uniform(-0.3, 0.3, size=(n, 3)) / SH_C0
    return _finish("tiny", rng, means, quats, log_scales, logits, sh, sh_degree, cams, W, H,
                   {}, background=background)
