"""Pins of the CPU oracle against facts that the pages and the mathematics fix.

None of these tests compares the oracle with itself: each checks a closed form,
an invariant, a textbook/library routine, a brute-force enumeration, or a
central finite difference of the rendered squared-residual loss.  The score
operators are the ones of the page "Research Proposal: Renderer Score Tokens
for Recurrent Gaussian Splatting" (Exact Score Operators): each block is stated
there to be the support-normalised local (partial) VJP of the RGB squared loss
under fixed contributor order/visibility and clamp masks, which is what the
finite-difference tests check.
"""
import math

import numpy as np
import pytest

import oracle
import scenes


# --------------------------------------------------------------------------
# the float32 decision exponential
# --------------------------------------------------------------------------
def test_exp2_spec_accuracy_and_exact_powers():
    x = np.linspace(-8.0, 0.5, 2_000_001, dtype=np.float32)
    got = oracle.exp2f(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    err = np.abs(got - ref) / ulp
    assert err.max() <= 2.0, err.max()
    ks = np.arange(-8, 1, dtype=np.float32)
    assert np.array_equal(oracle.exp2f(ks), np.exp2(ks.astype(np.float64)).astype(np.float32))


def test_exp2_coefficients_are_taylor_of_2_pow_f():
    c = oracle.constants()["exp2_coef"]
    want = np.array([math.log(2.0) ** j / math.factorial(j) for j in range(8)])
    assert np.allclose(c.astype(np.float64), want, rtol=6e-8, atol=0)
    assert c[0] == 1.0


# --------------------------------------------------------------------------
# SH basis: orthonormal on the sphere (textbook identity), degree-0 closed form
# --------------------------------------------------------------------------
def test_sh_basis_orthonormal():
    n_t, n_p = 24, 48
    xg, wg = np.polynomial.legendre.leggauss(n_t)        # exact for the degree <= 6 products
    phi = (np.arange(n_p) + 0.5) * 2 * np.pi / n_p
    ct, ph = np.meshgrid(xg, phi, indexing="ij")
    st = np.sqrt(1 - ct ** 2)
    dirs = np.stack([st * np.cos(ph), st * np.sin(ph), ct], axis=-1).reshape(-1, 3)
    w = (wg[:, None] * np.full(n_p, 2 * np.pi / n_p)[None, :]).reshape(-1)
    B = oracle.sh_basis64(dirs, 16)
    gram = (B * w[:, None]).T @ B
    assert np.allclose(gram, np.eye(16), atol=1e-12)


def test_sh_basis_degree_one_is_linear_in_direction():
    d = np.array([[0.0, 0.0, 1.0], [1.0, 0.0, 0.0], [0.0, 1.0, 0.0]])
    B = oracle.sh_basis64(d, 4)
    c1 = math.sqrt(3.0 / (4.0 * math.pi))
    assert np.allclose(B[:, 0], 0.5 / math.sqrt(math.pi))
    assert np.allclose(np.abs(B[:, 1:]), c1 * np.abs(np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]])), atol=1e-15)


# --------------------------------------------------------------------------
# preprocess: EWA closed forms
# --------------------------------------------------------------------------
def _single(means, quats, scales, opac=0.8, W=64, H=64, f=64.0, sh=None, bg=(0, 0, 0), cams=None):
    means = np.atleast_2d(np.asarray(means, dtype=np.float64))
    G = means.shape[0]
    if cams is None:
        cams = np.zeros((1, 16))
        cams[0, [0, 4, 8]] = 1.0
        cams[0, 12:16] = [f, f, W / 2.0, H / 2.0]
    if sh is None:
        sh = np.zeros((G, 1, 3))
        sh[:, 0, :] = (np.array([0.9, 0.5, 0.2]) - 0.5) / scenes.SH_C0
    sh = np.asarray(sh, dtype=np.float64)
    V = cams.shape[0]
    return scenes.Scene(
        name="unit", means=means.astype(np.float32),
        quats=np.broadcast_to(np.asarray(quats, np.float64), (G, 4)).astype(np.float32),
        scales=np.broadcast_to(np.asarray(scales, np.float64), (G, 3)).astype(np.float32),
        opacities=np.broadcast_to(np.asarray(opac, np.float64), (G,)).astype(np.float32),
        sh=sh.astype(np.float32), sh_degree=int(round(math.sqrt(sh.shape[1]))) - 1,
        cams=np.asarray(cams, dtype=np.float32), width=W, height=H,
        background=np.asarray(bg, dtype=np.float32), means_perturbed=means.astype(np.float32),
        pixel_noise=np.zeros((V, H, W, 3), np.float32), notes={})


def test_isotropic_on_axis_closed_form():
    z, s, f = 3.0, 0.0625, 64.0   # exact binary values
    sc = _single([0.0, 0.0, z], [1, 0, 0, 0], [s, s, s], f=f)
    o = oracle.OracleScene(sc)
    r64 = o.records64()[0, 0]
    var = (f * s / z) ** 2 + 0.3
    assert np.allclose(r64[[2, 3, 4]], [1 / var, 0.0, 1 / var], rtol=1e-14, atol=1e-15)
    assert np.allclose(r64[[0, 1]], [32.0, 32.0], rtol=0, atol=1e-12)
    r32 = o.records32()[0, 0]
    assert r32[0] == 0
    # exponent factors: k Sigma2^-1 = L L^T with L = [[s1, 0], [s2, s3]], k = log2(e) / 2
    k = math.log2(math.e) / 2
    assert np.allclose(r32[[5, 6, 7]], [math.sqrt(k / var), 0.0, math.sqrt(k / var)], rtol=3e-7, atol=1e-7)
    assert r32[1] == 32.0 and r32[2] == 32.0 and r32[3] == 0.0 and r32[4] == 0.0
    lam = var + math.sqrt(0.1)             # disc = 0 -> floor 0.1
    assert r32[14] == math.ceil(3 * math.sqrt(lam))
    assert r32[13] == np.float32(z)
    # the quaternion is irrelevant for an isotropic Gaussian
    rng = np.random.default_rng(0)
    for _ in range(5):
        q = rng.normal(size=4)
        o2 = oracle.OracleScene(_single([0.0, 0.0, z], q / np.linalg.norm(q), [s, s, s], f=f))
        assert np.allclose(o2.records64()[0, 0, 2:5], r64[2:5], rtol=1e-12, atol=1e-14)


def test_off_axis_isotropic_covariance_closed_form():
    f, s = 64.0, 0.05
    p = np.array([0.3, -0.2, 2.5])
    o = oracle.OracleScene(_single(p, [1, 0, 0, 0], [s, s, s], f=f))
    r64 = o.records64()[0, 0]
    x, y, z = p.astype(np.float32).astype(np.float64)
    Jc = np.array([[f / z, 0, -f * x / z ** 2], [0, f / z, -f * y / z ** 2]])
    S2 = float(np.float32(s)) ** 2 * Jc @ Jc.T + 0.3 * np.eye(2)
    conic = np.linalg.inv(S2)
    assert np.allclose(r64[[2, 3, 4]], [conic[0, 0], conic[0, 1], conic[1, 1]], rtol=1e-12)
    assert np.allclose(r64[[0, 1]], [f * x / z + 32, f * y / z + 32], rtol=1e-14)


def test_roll_by_90_degrees_swaps_axes():
    f, z = 64.0, 3.0
    a, b, c = 0.1, 0.03, 0.05
    o1 = oracle.OracleScene(_single([0, 0, z], [1, 0, 0, 0], [a, b, c], f=f))
    h = math.sqrt(0.5)
    o2 = oracle.OracleScene(_single([0, 0, z], [h, 0, 0, h], [a, b, c], f=f))
    c1 = o1.records64()[0, 0, 2:5]
    c2 = o2.records64()[0, 0, 2:5]
    assert np.allclose([c1[0], c1[2]], [c2[2], c2[0]], rtol=1e-12)
    assert abs(c2[1]) < 1e-12 and abs(c1[1]) < 1e-12


def test_projection_jacobian_matches_finite_difference():
    sc = scenes.tiny_scene(seed=3, n=6, n_views=2)
    o = oracle.OracleScene(sc)
    r64 = o.records64()
    for v in range(sc.n_views):
        cam = sc.cams[v].astype(np.float64)
        R = cam[:9].reshape(3, 3)
        t = cam[9:12]

        def proj(m):
            pc = R @ m + t
            return np.array([cam[12] * pc[0] / pc[2] + cam[14], cam[13] * pc[1] / pc[2] + cam[15]])

        for g in range(sc.n):
            mu = sc.means[g].astype(np.float64)
            J = np.zeros((2, 3))
            for j in range(3):
                e = np.zeros(3)
                e[j] = 1e-6
                J[:, j] = (proj(mu + e) - proj(mu - e)) / 2e-6
            assert np.allclose(r64[v, g, 9:15].reshape(2, 3), J, rtol=1e-6, atol=1e-6)
            assert np.allclose(r64[v, g, 0:2], proj(mu), rtol=1e-12)


def test_exponent_factors_and_split_centre_reproduce_the_float64_projection():
    """The decision record keeps the exponent as -((s1 dx + s2 dy)^2 + (s3 dy)^2): the factors
    must satisfy L L^T = k conic (k = log2(e) / 2) for the float64 conic, and the centre is
    kept as a float32 pair whose sum is the float64 centre."""
    sc = scenes.tiny_scene(seed=8, n=400, n_views=2, W=96, H=80, sh_degree=1, log_scale=(-3.0, 1.6), spread=0.6)
    o = oracle.OracleScene(sc)
    r32, r64 = o.records32(), o.records64()
    live = r32[:, :, 0] == 0
    s1, s2, s3 = (r32[:, :, i].astype(np.float64) for i in (5, 6, 7))
    k = math.log2(math.e) / 2
    ca, cb, cc = (r64[:, :, i][live] for i in (2, 3, 4))
    cond = (ca + cc) ** 2 / (ca * cc - cb * cb)          # >= the conic's condition number
    assert cond.max() > 1e3                             # needle-like footprints are in the sample
    # each factor within a few float32 rounding units of the float64 conic's Cholesky factor
    L11, L21 = np.sqrt(k * ca), k * cb / np.sqrt(k * ca)
    L22 = np.sqrt(k * (ca * cc - cb * cb) / ca)
    for got, want in ((s1[live], L11), (s2[live], L21), (s3[live], L22)):
        assert np.all(np.abs(got - want) <= 1e-6 * np.abs(want)), np.max(np.abs(got - want) / np.abs(want))
    hi = r32[:, :, 1:3].astype(np.float64)
    lo = r32[:, :, 3:5].astype(np.float64)
    assert np.all(np.abs(hi + lo - r64[:, :, 0:2])[live] <= 1e-12 * np.abs(r64[:, :, 0:2])[live] + 1e-12)
    assert np.all(np.abs(lo)[live] <= np.spacing(np.abs(hi).astype(np.float32))[live])


def test_fov_clamp_state_matches_its_definition():
    """The clamp of the Jacobian's lateral offset is active where |t_x / t_z| > 1.3 (W/2) / f_x
    (likewise y); Gaussians are placed on both sides of the boundary."""
    f, W, H = 64.0, 64, 48
    lim_x, lim_y = 1.3 * (W / 2) / f, 1.3 * (H / 2) / f
    z = 3.0
    xs = np.array([0.0, 0.9, 0.99, 1.01, 1.2]) * lim_x * z
    ys = np.array([0.0, 0.95, 1.05, -1.05, -0.5]) * lim_y * z
    means = np.stack([xs, ys, np.full(5, z)], axis=1)
    sc = _single(means, [1, 0, 0, 0], [0.8, 0.8, 0.8], W=W, H=H, f=f)
    o = oracle.OracleScene(sc)
    r32 = o.records32()[0]
    m = sc.means.astype(np.float64)
    want = (np.abs(m[:, 0] / m[:, 2]) > 1.3 * ((0.5 * W) / f)).astype(int) | \
           ((np.abs(m[:, 1] / m[:, 2]) > 1.3 * ((0.5 * H) / f)).astype(int) << 1)
    live = r32[:, 0] == 0
    assert live.sum() >= 4
    assert np.array_equal(r32[live, 8].astype(int), want[live])


def test_behind_camera_is_culled():
    o = oracle.OracleScene(_single([[0, 0, -1.0], [0, 0, 0.001], [0, 0, 2.0]], [1, 0, 0, 0], [0.1] * 3))
    r = o.records32()[0]
    assert list(r[:, 0]) == [1.0, 1.0, 0.0]


# --------------------------------------------------------------------------
# tile lists: brute force
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", ["c1", "tiny_ragged"])
def test_tile_lists_equal_brute_force_scan(cfg):
    sc = scenes.make_scene(1) if cfg == "c1" else scenes.tiny_scene(seed=5, n=40, W=40, H=24)
    o = oracle.OracleScene(sc)
    starts, ids = o.lists()
    rec = o.records32()
    for tile in range(o.V * o.T):
        got = ids[starts[tile]:starts[tile + 1]]
        assert np.array_equal(got, o.tile_list_scan(tile))
        # membership = rectangle containment, order = (depth bits, id): checked in numpy
        v, t = divmod(tile, o.T)
        ty, tx = divmod(t, o.TX)
        r = rec[v]
        inside = ((r[:, 0] == 0) & (r[:, 15] <= tx) & (tx < r[:, 17]) & (r[:, 16] <= ty) & (ty < r[:, 18]))
        cand = np.nonzero(inside)[0]
        keys = r[cand, 13].view(np.uint32).astype(np.uint64) << np.uint64(32) | cand.astype(np.uint64)
        assert np.array_equal(got, cand[np.argsort(keys, kind="stable")])


# --------------------------------------------------------------------------
# composite: closed forms and invariants
# --------------------------------------------------------------------------
def test_single_gaussian_composite_closed_form():
    bg = np.array([0.2, 0.1, 0.05])
    sc = _single([0.0, 0.0, 2.0], [1, 0, 0, 0], [0.08, 0.08, 0.08], opac=0.7, bg=bg)
    o = oracle.OracleScene(sc)
    color, T, n, T64 = o.render()
    r64 = o.records64()[0, 0]
    ys, xs = np.mgrid[0:64, 0:64]
    dx, dy = xs + 0.5 - r64[0], ys + 0.5 - r64[1]
    alpha = 0.7 * np.exp(-0.5 * (r64[2] * dx * dx + 2 * r64[3] * dx * dy + r64[4] * dy * dy))
    col = np.array([0.9, 0.5, 0.2])
    live = n[0] == 1
    assert live.sum() > 50 and np.all(n[0][~live] == 0)
    a = alpha[live][:, None]
    want = a * col + (1 - a) * bg
    assert np.allclose(color[0][live], want, rtol=0, atol=1e-7)   # float32 inputs -> 1e-7
    assert np.allclose(T64[0][live], 1 - alpha[live], atol=1e-7)
    assert np.all(color[0][~live] == bg.astype(np.float32).astype(np.float64))
    # the skipped pixels are exactly those with alpha < 1/255 (up to float32 rounding ties)
    assert np.all(alpha[~live] < 1 / 255 + 1e-6) and np.all(alpha[live] > 1 / 255 - 1e-6)


def test_partition_of_unity_same_colour_everywhere():
    sc = scenes.make_scene(1)
    c = np.array([0.3, 0.6, 0.9], dtype=np.float32)
    sc.sh[:, 0, :] = (c - 0.5) / np.float32(scenes.SH_C0)
    sc.background = c.copy()
    o = oracle.OracleScene(sc)
    color, T, n, T64 = o.render()
    pre = o.records32()[0, :, 10:13]
    assert np.allclose(pre[o.records32()[0, :, 0] == 0], c, atol=1e-6)
    assert np.allclose(color[0], c.astype(np.float64), atol=2e-6)


def test_count_and_transmittance_by_per_pixel_brute_force():
    """Every Gaussian tested at every pixel, sorted by depth, decisions in float64:
    agrees with the list-based float32-decision composite except at rounding ties."""
    sc = scenes.make_scene(1)
    o = oracle.OracleScene(sc)
    color, T, n, T64 = o.render()
    r32 = o.records32()[0]
    r64 = o.records64()[0]
    ok = np.nonzero(r32[:, 0] == 0)[0]
    order = ok[np.lexsort((ok, r32[ok, 13].view(np.uint32)))]
    mism = 0
    for y in range(0, 64, 3):
        for x in range(0, 64, 3):
            px, py = x + 0.5, y + 0.5
            Tb, nb = 1.0, 0
            for g in order:
                rect = r32[g, 15:19]
                if not (rect[0] <= x // 16 < rect[2] and rect[1] <= y // 16 < rect[3]):
                    continue
                dx, dy = px - r64[g, 0], py - r64[g, 1]
                sig = 0.5 * (r64[g, 2] * dx * dx + 2 * r64[g, 3] * dx * dy + r64[g, 4] * dy * dy)
                a = min(0.99, r64[g, 5] * math.exp(-sig))
                if a < 1 / 255:
                    continue
                if Tb * (1 - a) < 1e-4:
                    break
                Tb *= 1 - a
                nb += 1
            if nb != n[0, y, x]:
                mism += 1
            else:
                assert abs(Tb - T64[0, y, x]) < 1e-5
    assert mism <= 2, mism


# --------------------------------------------------------------------------
# scores: central finite differences of L = 1/2 sum_p |C_hat - C|^2
# (decisions frozen; eps -> 0; no suffix-denominator mask)
# --------------------------------------------------------------------------
EPS0 = 1e-30


def _loss(o, obs):
    color, _, _, _ = o.render()
    return 0.5 * float(np.sum((color - obs.astype(np.float64)) ** 2))


@pytest.fixture(scope="module")
def fd_setup():
    sc = scenes.tiny_scene(seed=7, n=14, n_views=2, W=32, H=32, sh_degree=2)
    obs = (np.random.default_rng(1).uniform(0, 1, size=(2, 32, 32, 3))).astype(np.float32)
    o = oracle.OracleScene(sc)
    o.build_lists()
    o.select(None)
    o.render(obs=obs, eps=EPS0, den_min=0.0)
    acc = o.acc()
    tok = o.tokens(eps=EPS0, lam=1.0)
    return sc, obs, o, acc, tok


def _fd(o, obs, setter, x0, h):
    setter(x0 + h)
    lp = _loss(o, obs)
    setter(x0 - h)
    lm = _loss(o, obs)
    o.values_reset()
    return (lp - lm) / (2 * h)


def test_fd_opacity_logit(fd_setup):
    sc, obs, o, acc, tok = fd_setup
    checked = 0
    for g in range(sc.n):
        if acc[g, :, 0].sum() < 1e-3:
            continue
        op = float(sc.opacities[g])
        a0 = math.log(op / (1 - op))
        fd = _fd(o, obs, lambda a: o.set_opacity64(g, 1 / (1 + math.exp(-a))), a0, 1e-5)
        got = acc[g, :, 1].sum()
        assert abs(got - fd) <= 1e-6 * max(1.0, abs(fd)), (g, got, fd)
        Q = acc[g, :, 0].sum()
        assert abs(Q * tok[g, 3] - fd) <= 1e-6 * max(1.0, abs(fd))
        checked += 1
    assert checked >= 8


def test_fd_sh_coefficients(fd_setup):
    sc, obs, o, acc, tok = fd_setup
    d = sc.d
    rng = np.random.default_rng(3)
    checked = 0
    for g in range(sc.n):
        if acc[g, :, 0].sum() < 1e-3:
            continue
        for k, ch in [(0, 0), (int(rng.integers(1, d)), int(rng.integers(0, 3))), (d - 1, 2)]:
            x0 = float(sc.sh[g, k, ch])
            fd = _fd(o, obs, lambda x: o.set_sh64(g, k, ch, x), x0, 1e-4)
            got = acc[g, :, 8 + 3 * k + ch].sum()
            assert abs(got - fd) <= 1e-7 * max(1.0, abs(fd)), (g, k, ch, got, fd)
            Q = acc[g, :, 0].sum()
            assert abs(Q * tok[g, 4 + 3 * k + ch] - fd) <= 1e-7 * max(1.0, abs(fd))
            checked += 1
    assert checked >= 20


def test_fd_projected_centre(fd_setup):
    sc, obs, o, acc, tok = fd_setup
    r64 = o.records64()
    checked = 0
    for g in range(sc.n):
        for v in range(sc.n_views):
            if acc[g, v, 0] < 1e-3:
                continue
            mx, my = r64[v, g, 0], r64[v, g, 1]
            fdx = _fd(o, obs, lambda x: o.set_mean2d64(g, v, x, my), mx, 1e-5)
            fdy = _fd(o, obs, lambda y: o.set_mean2d64(g, v, mx, y), my, 1e-5)
            assert abs(acc[g, v, 2] - fdx) <= 1e-6 * max(1.0, abs(fdx)), (g, v, acc[g, v, 2], fdx)
            assert abs(acc[g, v, 3] - fdy) <= 1e-6 * max(1.0, abs(fdy)), (g, v, acc[g, v, 3], fdy)
            checked += 1
    assert checked >= 10


def test_fd_mean_pullback_multiview(fd_setup):
    """Q b^mu equals dL/dmu (all views, covariance and colour frozen): the
    gamma-weighted pullback of the per-view projected-centre scores."""
    sc, obs, o, acc, tok = fd_setup
    checked = 0
    for g in range(sc.n):
        Q = acc[g, :, 0].sum()
        if Q < 1e-3:
            continue
        mu = sc.means[g].astype(np.float64)
        for j in range(3):
            def setter(x, j=j):
                m = mu.copy()
                m[j] = x
                o.set_mean3d64(g, m)
            fd = _fd(o, obs, setter, mu[j], 1e-6)
            assert abs(Q * tok[g, j] - fd) <= 1e-5 * max(1.0, abs(fd)), (g, j, Q * tok[g, j], fd)
        checked += 1
    assert checked >= 8


def test_single_gaussian_opacity_score_closed_form():
    """bg = 0 and one Gaussian: the suffix is empty, so rho = <r, c> and
    s_alpha q = sum_p alpha (1 - o) <r, c>."""
    sc = _single([0.0, 0.0, 2.0], [1, 0, 0, 0], [0.08, 0.08, 0.08], opac=0.6)
    obs = np.random.default_rng(2).uniform(0, 1, size=(1, 64, 64, 3)).astype(np.float32)
    o = oracle.OracleScene(sc)
    o.select(None)
    color, _, n, _ = o.render(obs=obs, eps=EPS0, den_min=0.0)
    r64 = o.records64()[0, 0]
    live = n[0] == 1
    ys, xs = np.mgrid[0:64, 0:64]
    dx, dy = xs + 0.5 - r64[0], ys + 0.5 - r64[1]
    op = float(np.float32(0.6))
    alpha = op * np.exp(-0.5 * (r64[2] * dx * dx + 2 * r64[3] * dx * dy + r64[4] * dy * dy))
    c = r64[6:9]
    r = color[0] - obs[0]
    want = np.sum((alpha * (1 - op) * (r @ c))[live])
    assert abs(o.acc()[0, 0, 1] - want) <= 1e-9 * max(1, abs(want))
    want_w = alpha[live].sum()
    assert abs(o.acc()[0, 0, 0] - want_w) <= 1e-9 * want_w


@pytest.mark.parametrize("op,den_min", [(0.8, 0.204), (0.995, 1e-3)])
def test_single_gaussian_masks_closed_form(op, den_min):
    """Exact Score Operators: the opacity and centre scores carry M^alpha (alpha clamp not
    saturated, suffix denominator T(1 - alpha) not below the threshold), the support q and
    the SH score do not; the SH score carries the per-channel colour clamp instead.  One
    broad isotropic Gaussian centred on a pixel corner (var = 150 px^2), bg = 0, so T = 1,
    C+ = 0 and rho = <r, c>.  The four pixels nearest the centre have d^2 = 0.5 and the
    next ring d^2 = 2.5: with o = 0.8 the threshold 0.204 lies between their 1 - alpha
    (0.2013 and 0.2066), with o = 0.995 the alpha clamp o G >= 0.99 holds for d^2 <= 1.51
    only.  Channel 2's colour is negative before the clamp."""
    f, z = 64.0, 3.0
    var = 150.0
    s = math.sqrt(var - 0.3) * z / f
    sh = np.zeros((1, 1, 3))
    sh[0, 0, :] = (np.array([0.9, 0.5, -0.2]) - 0.5) / scenes.SH_C0
    sc = _single([0.0, 0.0, z], [1, 0, 0, 0], [s, s, s], opac=op, f=f, sh=sh)
    obs = np.random.default_rng(8).uniform(0, 1, size=(1, 64, 64, 3)).astype(np.float32)
    o = oracle.OracleScene(sc)
    o.select(None)
    color, _, n, _ = o.render(obs=obs, eps=EPS0, den_min=den_min)
    acc = o.acc()[0, 0]
    r64 = o.records64()[0, 0]
    assert np.allclose(r64[[2, 3, 4]], [1 / var, 0, 1 / var], rtol=1e-6, atol=1e-12)
    ys, xs = np.mgrid[0:64, 0:64]
    dx, dy = xs + 0.5 - r64[0], ys + 0.5 - r64[1]
    o32 = float(np.float32(op))
    ca, cb, cc = r64[2], r64[3], r64[4]            # 1/var up to the float32 rounding of the scale
    G = np.exp(-0.5 * (ca * dx * dx + 2 * cb * dx * dy + cc * dy * dy))
    clamped = o32 * G >= 0.99
    alpha = np.where(clamped, 0.99, o32 * G)
    live = n[0] == 1
    # every decision is far from its threshold (no float32 tie to resolve)
    assert np.all(np.abs(o32 * G - 0.99) > 1e-4)
    assert np.all(np.abs((1 - alpha) - den_min) > 1e-3)
    c = np.maximum(r64[6:9], 0.0)
    assert c[2] == 0.0
    r = color[0] - obs[0]
    rho = r @ c
    M = live & ~clamped & ((1 - alpha) >= den_min)
    assert 0 < (live & ~M).sum() <= 8          # the masked pixels are the centre ones
    assert abs(acc[0] - alpha[live].sum()) <= 1e-9 * alpha[live].sum()
    want_a = np.sum((alpha * (1 - o32) * rho)[M])
    want_mx = np.sum((o32 * G * (ca * dx + cb * dy) * rho)[M])
    want_my = np.sum((o32 * G * (cb * dx + cc * dy) * rho)[M])
    scale = np.sum(np.abs(alpha * rho)[live])
    assert abs(acc[1] - want_a) <= 1e-9 * scale, (acc[1], want_a)
    assert abs(acc[2] - want_mx) <= 1e-9 * scale, (acc[2], want_mx)
    assert abs(acc[3] - want_my) <= 1e-9 * scale, (acc[3], want_my)
    B0 = scenes.SH_C0
    for ch in range(3):
        want = 0.0 if ch == 2 else np.sum((alpha * B0 * r[..., ch])[live])
        assert abs(acc[oracle.NACC_FIXED + ch] - want) <= 1e-9 * scale, (ch, acc[oracle.NACC_FIXED + ch], want)


def test_all_masked_replay_keeps_support_and_sh():
    """With the suffix-denominator threshold at 1 every contribution is masked
    (T(1 - alpha) <= 1 - 1/255): the opacity and centre sums vanish exactly while the
    support and the SH sums equal those of the unmasked replay."""
    sc = scenes.tiny_scene(seed=12, n=20, n_views=2, sh_degree=1)
    obs = np.random.default_rng(9).uniform(0, 1, size=(2, 32, 32, 3)).astype(np.float32)
    res = []
    for den in (0.0, 1.0):
        o = oracle.OracleScene(sc)
        o.select(None)
        o.render(obs=obs, eps=1e-6, den_min=den)
        res.append(o.acc())
    a0, a1 = res
    assert a0[:, :, 0].sum() > 1.0 and np.abs(a0[:, :, 1:4]).sum() > 0
    assert np.all(a1[:, :, 1:4] == 0.0)
    # (the oracle's per-pixel sums run in a thread-dependent order: equal up to rounding)
    assert np.allclose(a1[:, :, 0], a0[:, :, 0], rtol=1e-12, atol=1e-12)
    k = oracle.NACC_FIXED
    assert np.allclose(a1[:, :, k:k + 3 * sc.d], a0[:, :, k:k + 3 * sc.d], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# token statistics: eigenvalues, single-view null direction, zero support
# --------------------------------------------------------------------------
def test_jacobi_eigenvalues_match_lapack():
    rng = np.random.default_rng(0)
    for _ in range(200):
        M = rng.normal(size=(3, 3)) * 10 ** rng.uniform(-3, 6)
        A = M @ M.T + np.eye(3) * rng.uniform(0, 2)
        ev = oracle.eig3(A)
        want = np.linalg.eigvalsh(A)[::-1]
        assert np.allclose(ev, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    assert np.allclose(oracle.eig3(np.diag([1.0, 3.0, 2.0])), [3, 2, 1])


def test_single_view_conditioning_has_lambda_along_the_ray():
    sc = scenes.tiny_scene(seed=9, n=10, n_views=1)
    obs = np.random.default_rng(4).uniform(0, 1, size=(1, 32, 32, 3)).astype(np.float32)
    o = oracle.OracleScene(sc)
    o.select(None)
    o.render(obs=obs)
    lam = 1.0
    tok, A, q = o.tokens(eps=1e-6, lam=lam, with_A=True)
    d = sc.d
    for g in range(sc.n):
        ev = np.linalg.eigvalsh(A[g])
        assert abs(ev[0] - lam) <= 1e-9 * ev[-1]
        tr = np.trace(A[g])
        assert np.allclose(tok[g, 5 + 3 * d: 8 + 3 * d] * (tr + 1e-6), ev[::-1], rtol=1e-10)
        assert abs(tok[g, 8 + 3 * d] - math.log(tr + 1e-6)) < 1e-12
        # the camera ray through the mean is in the null space of J^T J
        ray = sc.means[g].astype(np.float64) - (-sc.cams[0, 9:12].astype(np.float64))
        ray /= np.linalg.norm(ray)
        assert abs(ray @ A[g] @ ray - lam) <= 1e-6 * ev[-1]


def _isotropic_support(o, v, n, op, var, cx, cy, W, H):
    """W_gv = sum of alpha over the pixels where the single Gaussian contributes (n == 1),
    alpha = o exp(-|p - centre|^2 / (2 var)) for an isotropic footprint centred at (cx, cy)."""
    ys, xs = np.mgrid[0:H, 0:W]
    d2 = (xs + 0.5 - cx) ** 2 + (ys + 0.5 - cy) ** 2
    alpha = op * np.exp(-0.5 * d2 / var)
    return float(alpha[n[v] == 1].sum())


def _token_stats_closed_form(tok, d, lam, eps, ev):
    """The statistics block of the token: e~ = eig(A)/(tr A + eps) (descending) and log(tr A + eps)."""
    ev = np.sort(np.asarray(ev, dtype=np.float64))[::-1]
    tr = ev.sum()
    assert np.allclose(tok[5 + 3 * d: 8 + 3 * d], ev / (tr + eps), rtol=2e-6, atol=0), \
        (tok[5 + 3 * d: 8 + 3 * d], ev / (tr + eps))
    assert abs(tok[8 + 3 * d] - math.log(tr + eps)) <= 2e-6, (tok[8 + 3 * d], math.log(tr + eps))


@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_single_view_on_axis_conditioning_closed_form(eps):
    """One isotropic Gaussian on the optical axis of one camera (Exact Score Operators:
    q = eps + sum_p w, gamma = q / Q with Q = eps + sum_v q_v, A = lambda I + sum_v gamma J^T J).
    There J^T J = (f/z)^2 diag(1, 1, 0), so A = diag(lam + gamma k, lam + gamma k, lam) with
    k = (f/z)^2; the support W is summed from the closed-form footprint.  The large eps makes
    gamma = q / (eps + q) far from 1, so dropping gamma, or weighting by q, fails."""
    z, s, f, op, lam = 3.0, 0.0625, 64.0, 0.8, 1.0
    sc = _single([0.0, 0.0, z], [1, 0, 0, 0], [s, s, s], opac=op, f=f)
    obs = np.random.default_rng(5).uniform(0, 1, size=(1, 64, 64, 3)).astype(np.float32)
    o = oracle.OracleScene(sc)
    o.select(None)
    _, _, n, _ = o.render(obs=obs)
    var = (f * s / z) ** 2 + 0.3
    Wsum = _isotropic_support(o, 0, n, float(np.float32(op)), var, 32.0, 32.0, 64, 64)
    assert Wsum > 1.0
    tok, A, q = o.tokens(eps=eps, lam=lam, with_A=True)
    q_want = eps + Wsum
    assert abs(q[0, 0] - q_want) <= 1e-9 * q_want
    gamma = q_want / (eps + q_want)
    k = (f / z) ** 2
    A_want = np.diag([lam + gamma * k, lam + gamma * k, lam])
    assert np.allclose(A[0], A_want, rtol=1e-9, atol=1e-9), (A[0], A_want)
    _token_stats_closed_form(tok[0], sc.d, lam, eps, np.diag(A_want))
    assert abs(tok[0, 4 + 3 * sc.d] - math.log(eps + q_want)) <= 1e-9


def _look_at_camera(centre, direction, f, W, H):
    """Camera at `centre` whose optical axis is the unit vector `direction` in the x-z plane."""
    dx, _, dz = direction
    R = np.array([[dz, 0.0, -dx], [0.0, 1.0, 0.0], [dx, 0.0, dz]])  # rows: camera x, y, z axes
    row = np.zeros(16)
    row[0:9] = R.reshape(-1)
    row[9:12] = -R @ np.asarray(centre, dtype=np.float64)
    row[12:16] = [f, f, W / 2.0, H / 2.0]
    return row


@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_two_view_conditioning_gamma_weighting_closed_form(eps):
    """One isotropic Gaussian on the optical axes of two cameras at distances z1 = 3 and
    z2 = 4.5, the second axis tilted by 30 degrees.  For a camera looking straight at the
    Gaussian, J = (f/z) (rows 1, 2 of R), so J^T J = (f/z)^2 (I - d d^T) with d the viewing
    direction, and A = lam I + a1 (I - d1 d1^T) + a2 (I - d2 d2^T), a_v = gamma_v (f/z_v)^2,
    gamma_v = q_v / (eps + q1 + q2).  Its eigenvalues are lam + a1 + a2 (along y) and
    lam + a1 + a2 - m for m the eigenvalues of a1 d1 d1^T + a2 d2 d2^T (trace a1 + a2,
    determinant a1 a2 sin^2 30deg).  The supports differ (q1 != q2), so replacing gamma by 1
    or by q fails."""
    mu = np.array([0.0, 0.0, 3.0])
    s, f, op, lam, W = 0.0625, 64.0, 0.8, 1.0, 64
    th = math.radians(30.0)
    d2 = np.array([math.sin(th), 0.0, math.cos(th)])
    z = [3.0, 4.5]
    cams = np.stack([_look_at_camera([0, 0, 0], [0.0, 0.0, 1.0], f, W, W),
                     _look_at_camera(mu - z[1] * d2, d2, f, W, W)])
    sc = _single(mu, [1, 0, 0, 0], [s, s, s], opac=op, W=W, H=W, f=f, cams=cams)
    obs = np.random.default_rng(6).uniform(0, 1, size=(2, W, W, 3)).astype(np.float32)
    o = oracle.OracleScene(sc)
    o.select(None)
    _, _, n, _ = o.render(obs=obs)
    r64 = o.records64()
    Ws = []
    for v in range(2):
        var = (f * s / z[v]) ** 2 + 0.3
        assert np.allclose(r64[v, 0, 0:2], [32.0, 32.0], atol=2e-4)
        Ws.append(_isotropic_support(o, v, n, float(np.float32(op)), var, r64[v, 0, 0], r64[v, 0, 1], W, W))
    q_want = np.array([eps + Ws[0], eps + Ws[1]])
    assert abs(q_want[0] - q_want[1]) > 0.2 * q_want.max()      # unequal supports
    tok, A, q = o.tokens(eps=eps, lam=lam, with_A=True)
    assert np.allclose(q[0], q_want, rtol=1e-6)
    Q = eps + q_want.sum()
    a = q_want / Q * (f / np.array(z)) ** 2
    dirs = [np.array([0.0, 0.0, 1.0]), d2]
    A_want = lam * np.eye(3) + sum(a[v] * (np.eye(3) - np.outer(dirs[v], dirs[v])) for v in range(2))
    assert np.allclose(A[0], A_want, rtol=2e-6, atol=2e-6 * np.abs(A_want).max()), (A[0], A_want)
    tr_m, det_m = a.sum(), a[0] * a[1] * math.sin(th) ** 2
    disc = math.sqrt(tr_m ** 2 - 4 * det_m)
    m = [(tr_m + disc) / 2, (tr_m - disc) / 2]
    base = lam + a.sum()
    _token_stats_closed_form(tok[0], sc.d, lam, eps, [base, base - m[1], base - m[0]])
    assert abs(tok[0, 4 + 3 * sc.d] - math.log(Q)) <= 1e-6


def test_zero_support_token_closed_form():
    V = 3
    cams = np.zeros((V, 16))
    for v in range(V):
        cams[v, [0, 4, 8]] = 1.0
        cams[v, 9] = -0.1 * v
        cams[v, 12:16] = [32, 32, 16, 16]
    sc = _single([[0.0, 0.0, -2.0], [0.0, 0.0, 2.0]], [1, 0, 0, 0], [0.05] * 3, W=32, H=32, f=32, cams=cams)
    obs = np.full((V, 32, 32, 3), 0.5, np.float32)
    o = oracle.OracleScene(sc)
    o.select(None)
    o.render(obs=obs)
    eps, lam = 1e-6, 1.0
    tok = o.tokens(eps=eps, lam=lam)
    z = tok[0]
    d = 1
    want = np.zeros(9 + 3 * d)
    want[4 + 3 * d] = math.log((V + 1) * eps)
    want[5 + 3 * d: 8 + 3 * d] = lam / (3 * lam + eps)
    want[8 + 3 * d] = math.log(3 * lam + eps)
    assert np.allclose(z, want, rtol=1e-14, atol=1e-300)


def test_support_sum_equals_rendered_coverage():
    """sum_g sum_v (q_gv - eps) = sum_p (1 - T_final(p)) (telescoping of w = T alpha)."""
    sc = scenes.tiny_scene(seed=12, n=20, n_views=2)
    obs = np.zeros((2, 32, 32, 3), np.float32)
    o = oracle.OracleScene(sc)
    o.select(None)
    _, _, _, T64 = o.render(obs=obs)
    acc = o.acc()
    assert abs(acc[:, :, 0].sum() - np.sum(1 - T64)) <= 1e-10 * acc[:, :, 0].sum()


# --------------------------------------------------------------------------
# the occlusion toy: the method's own diagnostic (sign accuracy on high support)
# --------------------------------------------------------------------------
def test_occlusion_toy_mean_score_sign_accuracy():
    """Method diagnostic of the Block 0 occlusion toy (not a parity pin): on the
    top-quartile-support Gaussians, for axes perturbed by more than one standard
    deviation, the descent direction -b^mu points toward the perturbed position
    (measured 0.80 here; the plan's >80 % target is an untested hypothesis)."""
    sc = scenes.make_scene(1)
    obs = oracle.render_observation(sc)
    ref = oracle.full_reference(sc, obs)
    tok = ref["tokens"]
    logq = tok[:, 4 + 3 * sc.d]
    delta = (sc.means_perturbed - sc.means).astype(np.float64)
    high = logq > np.quantile(logq, 0.75)
    agree = np.sign(-tok[high, 0:2]) == np.sign(delta[high, 0:2])
    big = np.abs(delta[high, 0:2]) > 0.01
    assert agree[big].mean() > 0.7, agree[big].mean()
    assert agree.mean() > 0.6, agree.mean()
    # Gaussians behind two saturated layers receive (almost) no support
    back = sc.means[:, 2] > 3.5
    assert np.median(logq[back]) < np.median(logq[~back])


# --------------------------------------------------------------------------
# degenerate inputs: non-finite parameters, nothing visible, no Gaussians
# (boundary reading: non-finite values are not an error; the affected
# (Gaussian, view) pairs are culled or masked -- Proposal, Stage 2: explicit
# masks for numerically unstable contributions)
# --------------------------------------------------------------------------
NONFINITE_CULLED = [("means", (0, 0), np.nan), ("means", (1, 2), np.inf), ("means", (2, 0), -np.inf),
                    ("quats", (3, 1), np.nan), ("quats", (4, 0), np.inf), ("quats", (5, slice(None)), 0.0),
                    ("scales", (6, 0), np.nan), ("scales", (7, 1), np.inf), ("opacities", (8,), np.nan),
                    ("opacities", (9,), 1.5)]
NONFINITE_SH = [((10, 0, 1), np.nan), ((11, 0, 2), np.inf), ((12, 1, 0), -np.inf)]


def nonfinite_scene(base=None):
    """A small scene whose Gaussians 0..9 carry a non-finite (or out-of-range) mean,
    quaternion, scale or opacity and 10..12 a non-finite SH coefficient."""
    import dataclasses
    sc = base if base is not None else scenes.tiny_scene(seed=21, n=30, n_views=2, W=40, H=24, sh_degree=1)
    arrs = {k: getattr(sc, k).copy() for k in ("means", "quats", "scales", "opacities", "sh")}
    for field, idx, val in NONFINITE_CULLED:
        arrs[field][idx] = val
    for idx, val in NONFINITE_SH:
        arrs["sh"][idx] = val
    return dataclasses.replace(sc, means_perturbed=arrs["means"], **arrs)


def _drop(sc, keep):
    import dataclasses
    return dataclasses.replace(sc, means=sc.means[keep], quats=sc.quats[keep], scales=sc.scales[keep],
                               opacities=sc.opacities[keep], sh=sc.sh[keep], means_perturbed=sc.means_perturbed[keep])


def test_nonfinite_parameters_are_culled_like_absent_gaussians():
    sc = nonfinite_scene()
    obs = np.random.default_rng(1).uniform(0, 1, size=(2, 24, 40, 3)).astype(np.float32)
    full = oracle.full_reference(sc, obs)
    r32 = full["oracle"].records32()
    assert np.all(r32[:, :10, 0] == 1) and np.all(r32[:, 10:, 0] == 0)
    keep = np.arange(10, sc.n)
    part = oracle.full_reference(_drop(sc, keep), obs)
    assert np.array_equal(full["n"], part["n"]) and np.array_equal(full["T"], part["T"])
    assert np.allclose(full["color"], part["color"], rtol=0, atol=1e-14)
    assert np.allclose(full["tokens"][10:], part["tokens"], rtol=1e-12, atol=1e-14)
    # culled in every view: the zero-support token
    d, V, eps, lam = sc.d, sc.n_views, 1e-6, 1.0
    want = np.zeros(9 + 3 * d)
    want[4 + 3 * d] = math.log((V + 1) * eps)
    want[5 + 3 * d: 8 + 3 * d] = lam / (3 * lam + eps)
    want[8 + 3 * d] = math.log(3 * lam + eps)
    assert np.allclose(full["tokens"][:10], want[None, :], rtol=1e-14, atol=0)
    assert np.all(np.isfinite(full["tokens"]))


def test_nonfinite_sh_is_clamped_and_masked_like_a_negative_colour():
    """A non-finite SH coefficient makes its channel's pre-clamp colour non-finite: the colour
    clamp sends it to 0 and clears the clamp bit, exactly as a large negative coefficient does."""
    sc = nonfinite_scene()
    neg = nonfinite_scene()
    for idx, _ in NONFINITE_SH:
        neg.sh[idx] = -1e3
    obs = np.random.default_rng(2).uniform(0, 1, size=(2, 24, 40, 3)).astype(np.float32)
    a = oracle.full_reference(sc, obs)
    b = oracle.full_reference(neg, obs)
    r32 = a["oracle"].records32()
    for (g, k, ch), _ in NONFINITE_SH:
        assert np.all((r32[:, g, 19].astype(int) >> ch) & 1 == 0)
    assert np.array_equal(r32[:, :, 19], b["oracle"].records32()[:, :, 19])
    assert np.array_equal(a["n"], b["n"]) and np.array_equal(a["T"], b["T"])
    assert np.allclose(a["color"], b["color"], rtol=0, atol=1e-14)
    assert np.allclose(a["tokens"], b["tokens"], rtol=1e-12, atol=1e-14)
    for (g, k, ch), _ in NONFINITE_SH:
        assert np.all(a["tokens"][g, 4 + ch: 4 + 3 * sc.d: 3] == 0.0)    # the clamped channel's SH score
    # the renderer backward: a clamped channel passes no gradient, finite or not
    gC = np.random.default_rng(5).uniform(-1, 1, size=obs.shape).astype(np.float32)
    ga, gb = a["oracle"].backward(gC), b["oracle"].backward(gC)
    assert np.all(np.isfinite(ga))
    assert np.allclose(ga, gb, rtol=1e-12, atol=1e-14)


def test_all_culled_scene_renders_background():
    """Every Gaussian behind the cameras: no pair, every pixel the background with T = 1 and
    no contributor, every token the zero-support closed form."""
    import dataclasses
    sc = scenes.tiny_scene(seed=21, n=30, n_views=2, W=40, H=24, sh_degree=1, background=(0.3, 0.6, 0.1))
    m = sc.means.copy()
    m[:, 2] = -m[:, 2]
    sc = dataclasses.replace(sc, means=m, means_perturbed=m)
    obs = np.random.default_rng(3).uniform(0, 1, size=(2, 24, 40, 3)).astype(np.float32)
    ref = oracle.full_reference(sc, obs)
    assert ref["oracle"].n_pairs == 0
    assert np.all(ref["n"] == 0) and np.all(ref["T"] == 1.0)
    assert np.array_equal(ref["color"], np.broadcast_to(sc.background.astype(np.float64), ref["color"].shape))
    d, V, eps, lam = sc.d, sc.n_views, 1e-6, 1.0
    assert np.allclose(ref["tokens"][:, 4 + 3 * d], math.log((V + 1) * eps), rtol=1e-14)
    assert np.all(ref["tokens"][:, :4 + 3 * d] == 0.0)


def test_no_gaussians_renders_background():
    import dataclasses
    sc = scenes.tiny_scene(seed=21, n=30, n_views=2, W=40, H=24, sh_degree=2, background=(0.3, 0.6, 0.1))
    sc = _drop(sc, np.zeros(0, dtype=np.int64))
    assert sc.n == 0
    obs = np.random.default_rng(3).uniform(0, 1, size=(2, 24, 40, 3)).astype(np.float32)
    ref = oracle.full_reference(sc, obs)
    assert ref["oracle"].n_pairs == 0 and ref["tokens"].shape == (0, 9 + 3 * sc.d)
    assert np.all(ref["n"] == 0) and np.all(ref["T"] == 1.0)
    assert np.array_equal(ref["color"], np.broadcast_to(sc.background.astype(np.float64), ref["color"].shape))
