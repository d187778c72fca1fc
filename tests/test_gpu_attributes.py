"""Parity of the HIP feature composite (gs_render_features) and attribution
scatter (gs_attribute), through the C ABI, with the oracle.

Bars:
  * composite: per pixel and channel, |F - F_ref| <= FEAT_ATOL * (1 + max |f|)
    (float32 accumulation of up to ~100 weighted terms; the colour bar 1e-5
    scaled by the feature range), the background included;
  * scatter: per channel, relative L2 over all Gaussians <= ATTR_RTOL, and per
    Gaussian and channel |a - a_ref| <= ATTR_TERM_RTOL * sum_p w |m| (the sum of
    the terms' magnitudes, computed exactly by the oracle as the scatter of |m|:
    with a random-sign map a Gaussian's sum can cancel to far below its terms);
    1e-4: each alpha is evaluated at the float32 centre, which sits up to half an
    ulp of the pixel coordinate (3.8e-6 px at x ~ 100) from the oracle's; for the
    sub-pixel footprints of the pixel-aligned scenes (sigma ~ 0.6 px, offsets up
    to 2 px) that moves alpha by up to ~2e-5 relative (measured 2.1e-5);
  * the transpose identity sum_p <m, F> = sum_g <a, f> at full size (C2);
  * Gaussians no pixel reached get exactly zero.
The needle-like stress scene (condition numbers up to ~7e4) is held to the
same bars: preprocess keeps the exponent as a Cholesky factor formed in float64
and the centre as a float32 pair, so the per-pixel float32 evaluation keeps its
precision for elongated footprints.
"""
import zlib

import numpy as np
import pytest

import oracle
import scenes

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

FEAT_ATOL = 1e-5
ATTR_RTOL = 1e-5
ATTR_TERM_RTOL = 1e-4


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _scenes():
    return {
        "c1_toy": lambda: scenes.make_scene(1),
        "tiny_bg_deg1": lambda: scenes.tiny_scene(seed=5, n=30, n_views=3, W=33, H=17, sh_degree=1,
                                                  background=(0.3, 0.6, 0.1)),
        "rotated_clip": lambda: scenes.rotated_clip_scene(),
        "c2_small": lambda: scenes.c2_resplat_step(n_views=2, W=112, H=64),
        "c5_small": lambda: scenes.c5_multiview_layers(n_views=3, W=100, H=56, n=12000),
        "elongated": lambda: scenes.tiny_scene(seed=8, n=400, n_views=2, W=96, H=80, sh_degree=3,
                                               log_scale=(-3.0, 1.6), spread=0.6),
    }


CHANNELS = [1, 3, 9, 17]
_CACHE = {}


def _case(name, C):
    key = (name, C)
    if key not in _CACHE:
        _need_gpu()
        from gaussian_splatting_rasterizer_amd import binding
        sc = _scenes()[name]()
        rng = np.random.default_rng(zlib.crc32(f"{name}/{C}".encode()))
        f = rng.normal(size=(sc.n, C)).astype(np.float32)
        bg = rng.uniform(-1, 1, size=C).astype(np.float32)
        m = rng.normal(size=(sc.n_views, sc.height, sc.width, C)).astype(np.float32)
        o = oracle.OracleScene(sc)
        o.build_lists()
        F_ref = o.render_features(f, background=bg)
        a_ref = o.attribute(m)
        a_abs = o.attribute(np.abs(m))
        o.close()
        r = binding.rasterizer_for_scene(sc)
        r.project_and_bin()
        r.render()
        F = r.render_features(torch.from_numpy(f).cuda(), background=bg)
        a = r.attribute(torch.from_numpy(m).cuda())
        torch.cuda.synchronize()
        _CACHE[key] = (sc, f, bg, m, F_ref, (a_ref, a_abs), F.cpu().numpy(), a.cpu().numpy())
        r.close()
    return _CACHE[key]


NAMES = list(_scenes().keys())


@pytest.mark.parametrize("C", CHANNELS)
@pytest.mark.parametrize("name", NAMES)
def test_feature_composite_parity(name, C):
    sc, f, bg, m, F_ref, _, F, a = _case(name, C)
    atol = FEAT_ATOL
    bound = atol * (1.0 + float(np.abs(f).max()))
    err = np.abs(F.astype(np.float64) - F_ref).max()
    print(f"{name} C={C}: max feature error {err:.2e} (bound {bound:.1e})")
    assert np.all(np.isfinite(F))
    assert err <= bound, err


@pytest.mark.parametrize("C", CHANNELS)
@pytest.mark.parametrize("name", NAMES)
def test_attribution_parity(name, C):
    sc, f, bg, m, F_ref, (a_ref, a_abs), F, a = _case(name, C)
    rtol = ATTR_RTOL
    term_rtol = ATTR_TERM_RTOL
    a64 = a.astype(np.float64)
    rel = np.linalg.norm(a64 - a_ref, axis=0) / np.maximum(np.linalg.norm(a_ref, axis=0), 1e-30)
    per = np.abs(a64 - a_ref) / np.maximum(a_abs, 1e-30)
    print(f"{name} C={C}: attribution rel L2 max over channels {rel.max():.2e}, "
          f"worst per-Gaussian error / sum of |terms| {per.max():.2e}")
    assert rel.max() <= rtol, rel
    assert per.max() <= term_rtol, per.max()
    # never-reached Gaussians: exactly zero on both sides
    zero = np.all(a_ref == 0.0, axis=1)
    assert np.all(a[zero] == 0.0)


def test_fullsize_transpose_identity_and_sampled_parity():
    """C2 at full size (8 views 256x448, 917,504 Gaussians), 9 feature channels and a
    2-channel map (error, coverage): the transpose identity over the whole frame, the
    composite against the oracle on sampled tiles, and the scatter of sampled Gaussians."""
    _need_gpu()
    from gaussian_splatting_rasterizer_amd import binding
    sc = scenes.make_scene(2)
    rng = np.random.default_rng(77)
    f = rng.normal(size=(sc.n, 9)).astype(np.float32)
    m = np.stack([rng.uniform(0, 1, size=(sc.n_views, sc.height, sc.width)),
                  np.ones((sc.n_views, sc.height, sc.width))], axis=-1).astype(np.float32)
    r = binding.rasterizer_for_scene(sc)
    r.project_and_bin()
    r.render()
    F = r.render_features(torch.from_numpy(f).cuda()).cpu().numpy().astype(np.float64)
    a = r.attribute(torch.from_numpy(m).cuda()).cpu().numpy().astype(np.float64)
    # transpose identity on the first two feature channels against the two map channels
    f2 = np.zeros((sc.n, 2), np.float32)
    f2[:] = f[:, :2]
    F2 = r.render_features(torch.from_numpy(f2).cuda()).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    r.close()
    lhs = np.sum(F2 * m.astype(np.float64))
    rhs = np.sum(a * f2.astype(np.float64))
    print(f"transpose identity: {lhs:.9e} vs {rhs:.9e}")
    assert abs(lhs - rhs) <= 1e-5 * np.sum(np.abs(a) * np.abs(f2.astype(np.float64))), (lhs, rhs)
    assert np.allclose(F2, F[..., :2], rtol=0, atol=0)  # slices are independent of the channel count

    o = oracle.OracleScene(sc)
    o.build_lists()
    tiles = np.sort(rng.choice(o.V * o.T, size=24, replace=False))
    F_ref = o.render_features(f)
    a_ref = o.attribute(m)
    o.close()
    sel = np.zeros((o.V, o.H, o.W), dtype=bool)
    for tile in tiles:
        v, t = divmod(int(tile), o.T)
        ty, tx = divmod(t, o.TX)
        sel[v, ty * 16:(ty + 1) * 16, tx * 16:(tx + 1) * 16] = True
    err = np.abs(F[sel] - F_ref[sel]).max()
    print(f"full-size composite: max error {err:.2e} over {sel.sum()} pixels")
    assert err <= FEAT_ATOL * (1 + np.abs(f).max())
    rel = np.linalg.norm(a - a_ref, axis=0) / np.linalg.norm(a_ref, axis=0)
    print(f"full-size scatter: rel L2 {rel}")
    assert rel.max() <= ATTR_RTOL


TOPK_W_ATOL = 1e-5


@pytest.mark.parametrize("k", [1, 4, 9, 16])
@pytest.mark.parametrize("name", ["c1_toy", "tiny_bg_deg1", "c2_small", "c5_small"])
def test_topk_parity(name, k):
    """Per pixel: the number of filled entries is min(k, n_contrib) (exact), the weights
    match the oracle's sorted weights position by position, and every id whose weight
    is separated from its neighbours (> 2 TOPK_W_ATOL) is the oracle's id."""
    _need_gpu()
    from gaussian_splatting_rasterizer_amd import binding
    sc = _scenes()[name]()
    o = oracle.OracleScene(sc)
    _, _, n_ref, _ = o.render()
    ids_ref, w_ref = o.topk(k + 1)
    o.close()
    r = binding.rasterizer_for_scene(sc)
    r.project_and_bin()
    r.render()
    ids, w = r.topk(k)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy().astype(np.float64)
    r.close()
    assert np.array_equal((ids >= 0).sum(axis=-1), np.minimum(n_ref, k))
    assert np.all(w[ids < 0] == 0.0)
    assert np.abs(w - w_ref[..., :k]).max() <= TOPK_W_ATOL
    # uniqueness of each oracle position among its neighbours (the (k+1)-th included)
    wr = w_ref
    gap_prev = np.concatenate([np.full(wr.shape[:-1] + (1,), np.inf), wr[..., :-1] - wr[..., 1:]], axis=-1)
    gap_next = np.concatenate([wr[..., :-1] - wr[..., 1:], np.full(wr.shape[:-1] + (1,), np.inf)], axis=-1)
    unique = (np.minimum(gap_prev, gap_next) > 2 * TOPK_W_ATOL)[..., :k] & (ids_ref[..., :k] >= 0)
    assert np.array_equal(ids[unique], ids_ref[..., :k][unique])
    print(f"{name} k={k}: {unique.sum()} unique positions of {(ids >= 0).sum()} filled")
