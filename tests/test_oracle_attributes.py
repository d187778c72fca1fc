"""Pins of the oracle's feature composite and attribution scatter -- CPU only.

  * a single isotropic Gaussian on the optical axis: the composite at a pixel is
    alpha f + (1 - alpha) bg with alpha from the closed-form 2D covariance;
  * per-Gaussian features equal to the (view-independent, SH degree 0) colour
    reproduce the colour render;
  * the scatter is the transpose of the composite: sum_p <m_p, F_p> equals
    sum_g <a_g, f_g> for any features f and map m (background 0);
  * the scatter of ones is the support the score replay accumulates (sum of
    T alpha per Gaussian over pixels and views), and sums to sum_p (1 - T_final);
  * top-K contributors: with K >= n_contrib the weights are all of a pixel's (they
    sum to 1 - T_final, their count is n_contrib), decreasing, and a smaller K
    keeps a prefix; two stacked Gaussians in closed form.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
import scenes


def _single_scene(opac, bg):
    z, s, f, W = 3.0, 0.0625, 64.0, 64
    cams = np.zeros((1, 16))
    cams[0, [0, 4, 8]] = 1.0
    cams[0, 12:16] = [f, f, W / 2.0, W / 2.0]
    sh = np.zeros((1, 1, 3))
    sh[0, 0, :] = (np.array([0.9, 0.5, 0.2]) - 0.5) / scenes.SH_C0
    sc = scenes.Scene(
        name="unit", means=np.array([[0.0, 0.0, z]], np.float32), quats=np.array([[1, 0, 0, 0]], np.float32),
        scales=np.full((1, 3), s, np.float32), opacities=np.array([opac], np.float32), sh=sh.astype(np.float32),
        sh_degree=0, cams=cams.astype(np.float32), width=W, height=W, background=np.asarray(bg, np.float32),
        means_perturbed=np.array([[0.0, 0.0, z]], np.float32), pixel_noise=np.zeros((1, W, W, 3), np.float32),
        notes={})
    var = (f * s / z) ** 2 + 0.3
    return sc, var


def test_single_gaussian_feature_closed_form():
    bg = np.array([0.25, -1.0], np.float32)
    feat = np.array([[2.0, 0.5]], np.float32)
    sc, var = _single_scene(0.8, (0, 0, 0))
    o = oracle.OracleScene(sc)
    F = o.render_features(feat, background=bg)
    for (x, y) in [(31, 31), (33, 30), (36, 32)]:
        dx, dy = x + 0.5 - 32.0, y + 0.5 - 32.0
        alpha = float(np.float32(0.8)) * math.exp(-0.5 * (dx * dx + dy * dy) / var)
        want = alpha * feat[0].astype(np.float64) + (1 - alpha) * bg.astype(np.float64)
        assert np.allclose(F[0, y, x], want, rtol=1e-12, atol=1e-14), (x, y, F[0, y, x], want)
    # far away: nothing contributes, the background alone
    assert np.allclose(F[0, 0, 0], bg.astype(np.float64), rtol=0, atol=0)


def test_colour_as_feature_reproduces_the_render():
    sc = scenes.tiny_scene(seed=13, n=50, n_views=2, W=48, H=40, sh_degree=0, background=(0.3, 0.6, 0.1))
    o = oracle.OracleScene(sc)
    color, _, _, _ = o.render()
    # degree 0: the colour is view-independent; the float32 clamp decision as in preprocess
    pre = (np.float32(0.28209479177387814) * sc.sh[:, 0, :]) + np.float32(0.5)
    col64 = np.where(pre >= 0, scenes.SH_C0 * sc.sh[:, 0, :].astype(np.float64) + 0.5, 0.0)
    F = o.render_features(col64.astype(np.float32), background=sc.background)
    # features rounded to float32: |dF| <= sum_k w_k |df_k| <= 2^-24 max|c|
    assert np.abs(F - color).max() <= 1e-7, np.abs(F - color).max()


def test_scatter_is_the_transpose_of_the_composite():
    sc = scenes.rotated_clip_scene()
    o = oracle.OracleScene(sc)
    rng = np.random.default_rng(9)
    C = 5
    f = rng.normal(size=(sc.n, C)).astype(np.float32)
    m = rng.normal(size=(sc.n_views, sc.height, sc.width, C)).astype(np.float32)
    F = o.render_features(f)
    a = o.attribute(m)
    lhs = float(np.sum(F * m.astype(np.float64)))
    rhs = float(np.sum(a * f.astype(np.float64)))
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs)), (lhs, rhs)
    # and channel by channel
    for c in range(C):
        l = float(np.sum(F[..., c] * m[..., c].astype(np.float64)))
        r = float(np.sum(a[:, c] * f[:, c].astype(np.float64)))
        assert abs(l - r) <= 1e-11 * max(1.0, abs(l))


def test_scatter_of_ones_is_the_replay_support():
    sc = scenes.tiny_scene(seed=21, n=60, n_views=2, W=40, H=24, sh_degree=2)
    o = oracle.OracleScene(sc)
    o.build_lists()
    o.select(None)
    obs = np.zeros((sc.n_views, sc.height, sc.width, 3), np.float32)
    _, _, _, T64 = o.render(obs=obs)
    W_support = o.acc()[:, :, 0].sum(axis=1)
    a = o.attribute(np.ones((sc.n_views, sc.height, sc.width, 1), np.float32))[:, 0]
    assert np.allclose(a, W_support, rtol=1e-13, atol=1e-15)
    assert abs(a.sum() - np.sum(1.0 - T64)) <= 1e-10 * a.sum()


def test_topk_weights_sum_and_counts():
    """With K at least the contributor count, the top-K weights of a pixel are all its
    weights: they sum to 1 - T_final and their number is n_contrib; weights decrease."""
    sc = scenes.tiny_scene(seed=21, n=60, n_views=2, W=40, H=24, sh_degree=2)
    o = oracle.OracleScene(sc)
    _, _, n, T64 = o.render()
    K = int(n.max())
    ids, w = o.topk(K)
    assert np.array_equal((ids >= 0).sum(axis=-1), n)
    assert np.allclose(w.sum(axis=-1), 1.0 - T64, rtol=0, atol=1e-13)
    assert np.all(np.diff(w, axis=-1) <= 0)
    # a smaller K keeps the largest ones
    ids3, w3 = o.topk(3)
    assert np.array_equal(ids3, ids[..., :3]) and np.array_equal(w3, w[..., :3])


def test_topk_two_gaussians_far_one_wins():
    """A faint near Gaussian in front of an opaque far one: at the centre pixel the far
    one has the larger weight (1 - a_near) * a_far and comes first."""
    z1, z2, f, W = 2.0, 4.0, 64.0, 64
    cams = np.zeros((1, 16))
    cams[0, [0, 4, 8]] = 1.0
    cams[0, 12:16] = [f, f, W / 2.0, W / 2.0]
    sh = np.zeros((2, 1, 3), np.float32)
    sc = scenes.Scene(
        name="two", means=np.array([[0, 0, z1], [0, 0, z2]], np.float32),
        quats=np.array([[1, 0, 0, 0]] * 2, np.float32), scales=np.full((2, 3), 0.05, np.float32),
        opacities=np.array([0.2, 0.95], np.float32), sh=sh, sh_degree=0, cams=cams.astype(np.float32),
        width=W, height=W, background=np.zeros(3, np.float32), means_perturbed=np.zeros((2, 3), np.float32),
        pixel_noise=np.zeros((1, W, W, 3), np.float32), notes={})
    o = oracle.OracleScene(sc)
    ids, w = o.topk(2)
    assert list(ids[0, 31, 31]) == [1, 0]
    # closed form at the pixel centre (31.5, 31.5), offset 0.5 px in x and y from the centre (32, 32)
    s32 = float(np.float32(0.05))
    a_near = float(np.float32(0.2)) * math.exp(-0.25 / ((f * s32 / z1) ** 2 + 0.3))
    a_far = float(np.float32(0.95)) * math.exp(-0.25 / ((f * s32 / z2) ** 2 + 0.3))
    assert abs(w[0, 31, 31, 1] - a_near) <= 1e-12
    assert abs(w[0, 31, 31, 0] - (1.0 - a_near) * a_far) <= 1e-12
