"""Pins of the oracle's renderer backward (vector-Jacobian product of the colour
image) -- CPU only.

The backward is written as an explicit chain rule (composite -> 2D Gaussian ->
EWA projection -> quaternion/scale covariance, and SH colour with the view
direction).  It is pinned here against things other than itself:
  * central finite differences of the oracle's own float64 forward render, with
    the float32 decisions frozen (so the image is a smooth function of every
    parameter), for every parameter of every covered Gaussian, on rotated
    cameras and with the field-of-view clamp active for some Gaussians;
  * the SH polynomial derivatives against finite differences of the basis;
  * the score replay's opacity-logit and SH scores, which are the same
    derivatives of 1/2 |C_hat - C|^2 reached through the suffix equation
    (epsilon -> 0, no suffix-denominator mask).
Every check runs in the plain and the antialiased (opacity-compensated) mode.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import scenes


@pytest.fixture(scope="module", params=[False, True], ids=["plain", "antialiased"])
def bw_setup(request):
    sc = scenes.rotated_clip_scene()
    gC = np.random.default_rng(2).uniform(-1, 1, size=(sc.n_views, sc.height, sc.width, 3)).astype(np.float32)
    o = oracle.OracleScene(sc, antialiased=request.param)
    o.build_lists()
    grads, g2d = o.backward(gC, with_image_sums=True)
    return sc, gC, o, grads, g2d


def _lin(o, gC):
    color, _, _, _ = o.render()
    return float(np.sum(color * gC.astype(np.float64)))


def test_fov_clamp_is_exercised(bw_setup):
    sc, gC, o, grads, g2d = bw_setup
    r64 = o.records64()
    # the two extra Gaussians are live in view 0 and their centres lie outside the clamp
    for g, axis in [(sc.n - 2, 0), (sc.n - 1, 1)]:
        mx, my = r64[0, g, 0], r64[0, g, 1]
        tan = ((mx - sc.width / 2) if axis == 0 else (my - sc.height / 2)) / float(sc.cams[0, 12])
        assert abs(tan) > 1.3 * 0.5
        assert np.abs(g2d[0, g]).sum() > 0


@pytest.mark.parametrize("group", ["mean", "quat", "scale", "opacity"])
def test_fd_every_parameter(bw_setup, group):
    sc, gC, o, grads, g2d = bw_setup
    sl = {"mean": range(0, 3), "quat": range(3, 7), "scale": range(7, 10), "opacity": range(10, 11)}[group]
    checked = 0
    for g in range(sc.n):
        if np.abs(g2d[:, g]).sum() == 0:
            continue
        p0 = o.params64(g)
        for i in sl:
            h = 1e-6 * max(1.0, abs(p0[i]))
            p = p0.copy()
            p[i] = p0[i] + h
            o.set_params64(g, p)
            lp = _lin(o, gC)
            p[i] = p0[i] - h
            o.set_params64(g, p)
            lm = _lin(o, gC)
            o.values_reset()
            fd = (lp - lm) / (2 * h)
            got = grads[g, i]
            assert abs(got - fd) <= 2e-6 * max(1.0, abs(fd)), (group, g, i, got, fd)
            checked += 1
    assert checked >= 12 * len(sl)


def test_fd_sh_coefficients(bw_setup):
    sc, gC, o, grads, g2d = bw_setup
    d = sc.d
    checked = 0
    for g in range(sc.n):
        if np.abs(g2d[:, g]).sum() == 0:
            continue
        for k in range(d):
            ch = (g + k) % 3
            x0 = float(sc.sh[g, k, ch])
            o.set_sh64(g, k, ch, x0 + 1e-4)
            lp = _lin(o, gC)
            o.set_sh64(g, k, ch, x0 - 1e-4)
            lm = _lin(o, gC)
            o.values_reset()
            fd = (lp - lm) / 2e-4
            got = grads[g, 11 + 3 * k + ch]
            assert abs(got - fd) <= 1e-7 * max(1.0, abs(fd)), (g, k, ch, got, fd)
            checked += 1
    assert checked >= 12 * d


def test_quaternion_gradient_is_tangent(bw_setup):
    """The image depends on q only through q / |q|: the gradient has no radial part."""
    sc, gC, o, grads, g2d = bw_setup
    for g in range(sc.n):
        q = sc.quats[g].astype(np.float64)
        gq = grads[g, 3:7]
        assert abs(np.dot(gq, q)) <= 1e-9 * max(1.0, np.linalg.norm(gq) * np.linalg.norm(q))


def test_uncovered_gaussians_have_zero_gradient(bw_setup):
    sc, gC, o, grads, g2d = bw_setup
    for g in range(sc.n):
        if np.abs(g2d[:, g]).sum() == 0:
            assert np.all(grads[g] == 0.0)


def test_sh_basis_derivative_matches_finite_difference():
    rng = np.random.default_rng(4)
    dirs = rng.normal(size=(20, 3))
    dirs /= np.linalg.norm(dirs, axis=1, keepdims=True)
    dB = oracle.sh_basis_grad64(dirs, 16)
    h = 1e-6
    for j in range(3):
        e = np.zeros(3)
        e[j] = h
        fd = (oracle.sh_basis64(dirs + e, 16) - oracle.sh_basis64(dirs - e, 16)) / (2 * h)
        assert np.allclose(dB[:, :, j], fd, rtol=1e-7, atol=1e-8)


@pytest.mark.parametrize("antialiased", [False, True])
def test_backward_of_squared_residual_equals_replay_scores(antialiased):
    """With dL/dC_hat = C_hat - C_obs the backward is the gradient of
    1/2 |C_hat - C_obs|^2; the replay reaches the same opacity-logit and SH scores
    (summed over views) through the suffix equation when epsilon -> 0 and the
    suffix-denominator mask is off."""
    sc = scenes.tiny_scene(seed=7, n=14, n_views=2, W=32, H=32, sh_degree=2)
    obs = np.random.default_rng(1).uniform(0, 1, size=(2, 32, 32, 3)).astype(np.float32)
    o = oracle.OracleScene(sc, antialiased=antialiased)
    o.build_lists()
    o.select(None)
    color, _, _, _ = o.render(obs=obs, eps=1e-30, den_min=0.0)
    acc = o.acc()
    resid = (color - obs.astype(np.float64)).astype(np.float32)
    # the float32 rounding of the residual bounds the agreement
    grads = o.backward(resid)
    op = sc.opacities.astype(np.float64)
    s_alpha = acc[:, :, 1].sum(axis=1)
    d = sc.d
    s_sh = acc[:, :, 8:8 + 3 * d].sum(axis=1)
    for g in range(sc.n):
        if acc[g, :, 0].sum() < 1e-3:
            continue
        logit_grad = grads[g, 10] * op[g] * (1 - op[g])
        assert abs(logit_grad - s_alpha[g]) <= 1e-5 * max(1.0, abs(s_alpha[g])), (g, logit_grad, s_alpha[g])
        assert np.allclose(grads[g, 11:], s_sh[g], rtol=1e-5, atol=1e-6)
