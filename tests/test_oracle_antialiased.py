"""Pins of the oracle's antialiased (opacity-compensated) mode -- CPU only.

Reading: with the 0.3 px^2 dilation of the 2D covariance kept, the opacity is
scaled by comp = sqrt(det S / det(S + 0.3 I)) (S the undilated projected
covariance), so the footprint's integrated weight is that of the undilated
Gaussian; comp depends on depth through S.
  * isotropic Gaussian on the optical axis: comp = var / (var + 0.3) in closed
    form (float64 values, float32 record within rounding), and the rendered
    alpha at a pixel is comp times the plain mode's;
  * the integrated weight: the sum of alpha over the image equals
    o 2 pi sqrt(det S) (the undilated Gaussian's integral), within the
    alpha-cut and pixel-sampling error, while the plain mode's exceeds it by
    (var + 0.3) / var;
  * decisions: a Gaussian whose compensated opacity falls below 1/255 never
    contributes.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
import scenes


def _iso(s, z, opac, f=64.0, W=64):
    cams = np.zeros((1, 16))
    cams[0, [0, 4, 8]] = 1.0
    cams[0, 12:16] = [f, f, W / 2.0, W / 2.0]
    sh = np.zeros((1, 1, 3), np.float32)
    sh[0, 0, :] = 0.5 / scenes.SH_C0          # colour 1.0 in every channel
    sc = scenes.Scene(
        name="iso", means=np.array([[0.0, 0.0, z]], np.float32), quats=np.array([[1, 0, 0, 0]], np.float32),
        scales=np.full((1, 3), s, np.float32), opacities=np.array([opac], np.float32), sh=sh, sh_degree=0,
        cams=cams.astype(np.float32), width=W, height=W, background=np.zeros(3, np.float32),
        means_perturbed=np.array([[0.0, 0.0, z]], np.float32), pixel_noise=np.zeros((1, W, W, 3), np.float32),
        notes={})
    var = (f * float(np.float32(s)) / z) ** 2
    return sc, var


def test_isotropic_compensation_closed_form():
    sc, var = _iso(0.0625, 3.0, 0.8)
    comp = var / (var + 0.3)
    plain = oracle.OracleScene(sc)
    aa = oracle.OracleScene(sc, antialiased=True)
    r_plain, r_aa = plain.records64()[0, 0], aa.records64()[0, 0]
    assert abs(r_aa[5] - float(np.float32(0.8)) * comp) <= 1e-15
    assert abs(r_plain[5] - float(np.float32(0.8))) == 0.0
    assert abs(aa.records32()[0, 0, 9] - np.float32(0.8) * comp) <= 2e-7
    # the conic is the same in both modes (the dilation is kept)
    assert np.array_equal(r_plain[2:5], r_aa[2:5])
    c_plain, _, _, _ = plain.render()
    c_aa, _, _, _ = aa.render()
    for (x, y) in [(31, 31), (33, 30), (29, 34)]:
        assert abs(c_aa[0, y, x, 0] - comp * c_plain[0, y, x, 0]) <= 1e-14


def test_integrated_weight_is_the_undilated_gaussians():
    sc, var = _iso(0.125, 3.0, 0.9)       # var = 7.1 px^2
    total = {}
    for aa in (False, True):
        o = oracle.OracleScene(sc, antialiased=aa)
        c, _, _, _ = o.render()
        total[aa] = float(c[0, :, :, 0].sum())
    undilated = float(np.float32(0.9)) * 2 * math.pi * var
    assert abs(total[True] / undilated - 1.0) < 0.01, total[True] / undilated
    assert abs(total[False] / undilated - (var + 0.3) / var) < 0.01


def test_compensated_opacity_below_the_cut_never_contributes():
    # a tiny Gaussian: var << 0.3, so comp ~ var / 0.3 pushes o comp below 1/255
    sc, var = _iso(0.001, 3.0, 0.9)
    assert 0.9 * var / (var + 0.3) < 1.0 / 255
    o = oracle.OracleScene(sc, antialiased=True)
    _, T, n, _ = o.render()
    assert n.max() == 0 and np.all(T == 1.0)
    o2 = oracle.OracleScene(sc)
    _, _, n2, _ = o2.render()
    assert n2.max() > 0
