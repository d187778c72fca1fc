"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars (from the benchmark spec and the plan's Block 0 gate):
  * preprocess records, tile lists and ranges: bit-exact;
  * contributor counts and final transmittance: bit-exact;
  * rendered colour: within 1e-5 absolute;
  * tokens: relative L2 error per Gaussian within 1e-3 (the validation
    threshold of the Renderer Score Tokens experiment plan, Block 0).
Small configurations are compared element by element; the full-size
configurations on sampled tiles and sampled Gaussians the oracle computes
one by one.
"""
import math

import numpy as np
import pytest

import oracle
import scenes

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOKEN_RTOL = 1e-3
COLOR_ATOL = 1e-5


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _binding():
    from gaussian_splatting_rasterizer_amd import binding
    binding.load_library()
    return binding


def _run_gpu(sc, obs, antialiased=False):
    b = _binding()
    r = b.rasterizer_for_scene(sc, antialiased=antialiased)
    r.project_and_bin()
    rec = r.export(b.GS_EXPORT_RECORDS).cpu().numpy()
    keys = r.export(b.GS_EXPORT_DEPTH_KEYS).cpu().numpy().view(np.uint32)
    ids = r.export(b.GS_EXPORT_SORTED_IDS).cpu().numpy()[: r.n_pairs]
    ranges = r.export(b.GS_EXPORT_RANGES).cpu().numpy()
    color, T, n = r.render()
    tok = r.score_replay(torch.from_numpy(obs).cuda())
    work = r.export(b.GS_EXPORT_PIXEL_STATS).cpu().numpy().view(np.uint32)
    torch.cuda.synchronize()
    out = dict(rec=rec, keys=keys, ids=ids, ranges=ranges, n_pairs=r.n_pairs, color=color.cpu().numpy(),
               T=T.cpu().numpy(), n=n.cpu().numpy(), tokens=tok.cpu().numpy(), work=work)
    r.close()
    return out


def _small_scenes():
    return {
        "c1_toy": lambda: scenes.make_scene(1),
        "tiny_ragged_2view": lambda: scenes.tiny_scene(seed=21, n=60, n_views=2, W=40, H=24, sh_degree=2),
        "c2_small": lambda: scenes.c2_resplat_step(n_views=2, W=112, H=64),
        "c3_small": lambda: scenes.c3_atsplat_compact(n_anchors=600, W=200, H=120),
        "c4_small": lambda: scenes.c4_dense_pixel_aligned(n_sources=3, W=120, H=72),
        "c5_small": lambda: scenes.c5_multiview_layers(n_views=3, W=100, H=56, n=12000),
        "tiny_bg_deg1": lambda: scenes.tiny_scene(seed=5, n=30, n_views=3, W=33, H=17, sh_degree=1,
                                                  background=(0.3, 0.6, 0.1)),
        # very anisotropic Gaussians (log-scales N(-3, 1.6)): needle-like footprints across many tiles
        "elongated": lambda: scenes.tiny_scene(seed=8, n=400, n_views=2, W=96, H=80, sh_degree=3,
                                               log_scale=(-3.0, 1.6), spread=0.6),
        # a tile grid wider than 256 tiles (4200 px): the depth sort gathers rectangles instead of carrying them
        "wide_grid": lambda: scenes.tiny_scene(seed=31, n=3000, n_views=1, W=4200, H=48, sh_degree=1,
                                               log_scale=(-5.5, 0.5)),
        # antialiased (opacity-compensated) mode
        "c2_small_aa": lambda: scenes.c2_resplat_step(n_views=2, W=112, H=64),
        "tiny_ragged_aa": lambda: scenes.tiny_scene(seed=21, n=60, n_views=2, W=40, H=24, sh_degree=2),
        "c5_small_aa": lambda: scenes.c5_multiview_layers(n_views=3, W=100, H=56, n=12000),
    }


def _aa(name):
    return name.endswith("_aa")


_CACHE = {}


def _case(name):
    if name not in _CACHE:
        _need_gpu()
        sc = _small_scenes()[name]()
        obs = oracle.render_observation(sc, antialiased=_aa(name))
        ref = oracle.full_reference(sc, obs, antialiased=_aa(name))
        o = ref["oracle"]
        starts, ids = o.lists()
        ref["starts"], ref["ids"] = starts, ids
        ref["rec32"] = o.records32()
        ref["work"] = o.pixel_work()
        gpu = _run_gpu(sc, obs, antialiased=_aa(name))
        _CACHE[name] = (sc, obs, ref, gpu)
    return _CACHE[name]


SMALL = list(_small_scenes().keys())


@pytest.mark.parametrize("name", SMALL)
def test_records_bit_exact(name):
    sc, obs, ref, gpu = _case(name)
    r32 = ref["rec32"].reshape(-1, 20)
    rec = gpu["rec"]                       # [3, VG, 4]
    live = r32[:, 0] == 0
    keys = gpu["keys"]
    assert np.array_equal(keys == 0xFFFFFFFF, ~live)
    assert np.array_equal(keys[live], r32[live, 13].view(np.uint32))
    got = np.stack([rec[0, :, 0], rec[0, :, 1], rec[0, :, 2], rec[0, :, 3], rec[1, :, 0], rec[1, :, 1],
                    rec[1, :, 2], rec[1, :, 3], rec[2, :, 0]], axis=1)[live]
    want = r32[live][:, [1, 2, 6, 7, 8, 9, 10, 11, 12]]
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), np.argwhere(got != want)[:5]
    lo = rec[2, live, 2].view(np.uint32)
    hi = rec[2, live, 3].view(np.uint32)
    rect = np.stack([lo & 0xFFFF, lo >> 16, hi & 0xFFFF, hi >> 16], axis=1)
    assert np.array_equal(rect, r32[live][:, 15:19].astype(np.uint32))


def _box_f64(a, b, c, opac, mx, my):
    """Reference half-widths of the region where an entry can pass the alpha test:
    Q(d) = a dx^2 + 2 b dx dy + c dy^2 <= t_eff with t_eff = (min(8, log2 255 o) + 1e-5) /
    (1 - 8u (cond + 1)), u = 2^-24, widened by 0.01 px + 1e-6 (|centre| + half-width);
    float64 from the float32 coefficients.  Returns (wx, wy, kind) with kind 0 finite,
    1 unbounded (never skipped), -1 empty."""
    with np.errstate(divide="ignore", invalid="ignore"):
        tt = np.log2(255.0 * opac)
        det = a * c - b * b
        t = np.minimum(tt, 8.0) + 1e-5
        mid, hd = 0.5 * (a + c), np.sqrt(0.25 * (a - c) ** 2 + b * b)
        lmax = mid + hd
        lmin = det / lmax
        grow = 8.0 * 2.0 ** -24 * (lmax / lmin + 1.0)
        te = t / (1.0 - grow)
        ex, ey = np.sqrt(te * c / det), np.sqrt(te * a / det)
    kind = np.where(~(tt > -1e-5), -1, np.where(~(det > 0) | ~(a > 0) | ~(c > 0) | ~(grow < 0.5), 1, 0))
    wx = ex + 0.01 + 1e-6 * (np.abs(mx) + ex)
    wy = ey + 0.01 + 1e-6 * (np.abs(my) + ey)
    return wx, wy, kind


@pytest.mark.parametrize("name", SMALL)
def test_entry_boxes_conservative(name):
    """Every live record's packed entry box (two binary16 half-widths, rounded up) holds
    the float64 box computed from the record's own float32 coefficients: the render may
    skip an entry only where it provably cannot pass the alpha test."""
    sc, obs, ref, gpu = _case(name)
    rec = gpu["rec"]
    live = gpu["keys"] != 0xFFFFFFFF
    r0, r1, r2 = rec[0, live].astype(np.float64), rec[1, live].astype(np.float64), rec[2, live]
    a, b, c = -r0[:, 2], -0.5 * r0[:, 3], -r1[:, 0]
    wx, wy, kind = _box_f64(a, b, c, r1[:, 1], r0[:, 0], r0[:, 1])
    bits = r2[:, 1].view(np.uint32)
    hx = (bits & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    hy = (bits >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    fin = kind == 0
    assert np.all(hx[fin] >= wx[fin]) and np.all(hy[fin] >= wy[fin]), \
        (np.min(hx[fin] / wx[fin]), np.min(hy[fin] / wy[fin]))
    assert np.all(np.isinf(hx[kind == 1]) & (hx[kind == 1] > 0)) and np.all(np.isinf(hy[kind == 1]))
    # an empty box only where the opacity alone keeps alpha below 1/255
    empty = np.isinf(hx) & (hx < 0)
    assert np.all(r1[empty, 1] * 255.0 < 1.0)
    print(f"{name}: {fin.sum()} finite boxes, min ratio to the float64 box "
          f"{min(np.min(hx[fin] / wx[fin]), np.min(hy[fin] / wy[fin])) if fin.any() else float('nan'):.6f}, "
          f"{(kind == 1).sum()} unbounded, {empty.sum()} empty")


@pytest.mark.parametrize("name", SMALL)
def test_tile_lists_bit_exact(name):
    sc, obs, ref, gpu = _case(name)
    assert gpu["n_pairs"] == len(ref["ids"])
    assert np.array_equal(gpu["ids"], ref["ids"])
    starts = ref["starts"]
    counts = np.diff(starts)
    rg = gpu["ranges"].astype(np.int64)
    nonempty = counts > 0
    assert np.array_equal(rg[nonempty, 0], starts[:-1][nonempty])
    assert np.array_equal(rg[nonempty, 1], starts[1:][nonempty])
    assert np.all(rg[~nonempty, 0] == rg[~nonempty, 1])


@pytest.mark.parametrize("name", SMALL)
def test_pixel_work_bit_exact(name):
    """The exported per-pixel work counts (entries examined until the pixel stopped, and those
    past the distance cut) equal the oracle's, pixel for pixel."""
    sc, obs, ref, gpu = _case(name)
    assert gpu["work"].shape == ref["work"].shape
    assert np.array_equal(gpu["work"], ref["work"])


# The needle-like stress scene has conics with condition numbers up to ~7e4; the
# float32 quadratic form of the exponent (like the float32 conic entries
# themselves) then carries a relative error of order 2^-24 * cond, so its colour
# is held to 1e-3 instead of 1e-5.  Its decisions (counts, transmittance, lists)
# remain bit-exact.  Every workload configuration is held to 1e-5.
# The 4200-px-wide scene evaluates Gaussians at offsets from float32 centres of
# magnitude up to ~4200 px, rounded to half an ulp (1.2e-4 px) while the
# oracle's values use the float64 centre; with offsets of a few px and conic
# entries ~0.05-0.5 px^-2 that moves each alpha by up to ~1e-5 relative, summed
# over ~16 contributions per pixel: held to 5e-5.
COLOR_ATOL_OVERRIDE = {"elongated": 1e-3, "wide_grid": 5e-5}


@pytest.mark.parametrize("name", SMALL)
def test_render_parity(name):
    sc, obs, ref, gpu = _case(name)
    assert np.array_equal(gpu["n"], ref["n"]), np.argwhere(gpu["n"] != ref["n"])[:5]
    assert np.array_equal(gpu["T"].view(np.uint32), ref["T"].view(np.uint32))
    err = np.abs(gpu["color"] - ref["color"]).max()
    print(name, "max colour error", err)
    assert err <= COLOR_ATOL_OVERRIDE.get(name, COLOR_ATOL), err


def token_errors(z, zr, d):
    """Per-Gaussian relative L2 error of the whole token and per block."""
    blocks = {"b_mu": slice(0, 3), "s_alpha": slice(3, 4), "s_sh": slice(4, 4 + 3 * d),
              "stats": slice(4 + 3 * d, 9 + 3 * d)}
    denom = np.maximum(np.linalg.norm(zr, axis=1), 1e-6)
    rel = np.linalg.norm(z - zr, axis=1) / denom
    per_block = {}
    for k, s in blocks.items():
        e = np.linalg.norm(z[:, s] - zr[:, s], axis=1)
        nrm = np.linalg.norm(zr[:, s], axis=1)
        per_block[k] = float(np.max(e / np.maximum(nrm, 1e-3 * np.median(nrm) + 1e-30)))
    return rel, per_block


@pytest.mark.parametrize("name", SMALL)
def test_token_parity(name):
    sc, obs, ref, gpu = _case(name)
    z = gpu["tokens"].astype(np.float64)
    zr = ref["tokens"]
    rel, per_block = token_errors(z, zr, sc.d)
    print(name, "max rel", rel.max(), "per block", per_block)
    assert np.all(np.isfinite(gpu["tokens"]))
    assert rel.max() <= TOKEN_RTOL, (rel.max(), int(rel.argmax()), per_block)
    # Per block, each score is a sum of signed per-pixel terms, so the block is
    # held to 1e-3 of its value, plus 1e-4 of the sum of the terms' magnitudes
    # (float32 sums may cancel; the oracle accumulates both), plus what the
    # colour tolerance (1e-5 on C_hat, hence on r) moves it: |B| <= 1 and
    # |c - C+| <= 2 give 1e-5 W / Q for the SH block and 2e-5 (1 - o) W / Q for
    # the opacity block.
    acc = ref["oracle"].acc()                       # [G, V, 8 + 6d]
    d = sc.d
    W = acc[:, :, 0].sum(axis=1)
    Q = 1e-6 + np.sum(1e-6 + acc[:, :, 0], axis=1)
    o = sc.opacities.astype(np.float64)
    abs_alpha = acc[:, :, 4].sum(axis=1) / Q
    catol = COLOR_ATOL_OVERRIDE.get(name, COLOR_ATOL)
    bound_a = 1e-3 * np.abs(zr[:, 3]) + 1e-4 * abs_alpha + 2 * catol * (1 - o) * W / Q + 1e-9
    ratio_a = np.abs(z[:, 3] - zr[:, 3]) / bound_a
    assert ratio_a.max() <= 1.0, (ratio_a.max(), int(ratio_a.argmax()))
    abs_sh = acc[:, :, 8 + 3 * d: 8 + 6 * d].sum(axis=1) / Q[:, None]
    bound = 1e-3 * np.abs(zr[:, 4:4 + 3 * d]) + 1e-4 * abs_sh + (catol * W / Q)[:, None] + 1e-9
    ratio = np.abs(z[:, 4:4 + 3 * d] - zr[:, 4:4 + 3 * d]) / bound
    g, k = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, (ratio.max(), int(g), int(k), z[g, 4 + k], zr[g, 4 + k], abs_sh[g, k])


def test_exp2_bit_identical():
    _need_gpu()
    b = _binding()
    # every float32 in [-8, -0.5] (exponents -1..2), a stride through (-0.5, 0] and a grid up to 0.5
    lo = int(np.float32(-8.0).view(np.uint32))
    hi = int(np.float32(-0.5).view(np.uint32))
    dense = np.arange(hi, lo + 1, dtype=np.uint64).astype(np.uint32).view(np.float32)
    small = np.arange(0x80000000, hi, 97, dtype=np.uint64).astype(np.uint32).view(np.float32)
    pos = np.linspace(0.0, 0.5, 100001, dtype=np.float32)
    x = np.concatenate([dense, small, pos])
    xt = torch.from_numpy(x).cuda()
    yt = torch.empty_like(xt)
    b.gs_debug_exp2(xt, yt)
    torch.cuda.synchronize()
    y = yt.cpu().numpy()
    want = oracle.exp2f(x)
    bad = np.nonzero(y.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, (bad.size, x[bad[:5]], y[bad[:5]], want[bad[:5]])


def test_profile_stage_mask():
    """Only the stages named in the mask record launches; with every stage timed, one
    step records one launch of each of its nine stages."""
    _need_gpu()
    from gaussian_splatting_rasterizer_amd import binding
    sc = scenes.tiny_scene(seed=3, n=40, n_views=2, W=40, H=24, sh_degree=1)
    obs = torch.zeros((sc.n_views, sc.height, sc.width, 3), dtype=torch.float32, device="cuda")
    r = binding.rasterizer_for_scene(sc)
    try:
        binding.gs_profile_stages(r.ctx, ["render", "finalize"])
        r.step(obs)
        torch.cuda.synchronize()
        prof = binding.gs_profile_read(r.ctx)
        assert {k for k, (ms, n) in prof.items() if n > 0} == {"render", "finalize"}
        assert prof["render"][1] == 1 and prof["render"][0] > 0.0
        binding.gs_profile_enable(r.ctx, True)
        r.step(obs)
        torch.cuda.synchronize()
        prof = binding.gs_profile_read(r.ctx)
        step_stages = ("project", "depth_sort", "scan", "emit", "tile_sort", "ranges", "render", "replay", "finalize")
        assert all(prof[k][1] == 1 for k in step_stages), prof
        binding.gs_profile_enable(r.ctx, False)
        r.step(obs)
        torch.cuda.synchronize()
        assert all(n == 0 for ms, n in binding.gs_profile_read(r.ctx).values())
    finally:
        r.close()


def test_second_bin_sort_after_one_project():
    """gs_bin_sort may run again on the same preprocess: the second sort (which cannot
    reuse the packed rectangles the first consumed) gives identical lists and ranges."""
    _need_gpu()
    b = _binding()
    sc = scenes.c2_resplat_step(n_views=2, W=112, H=64)
    r = b.rasterizer_for_scene(sc)
    try:
        r.project_and_bin()
        ids1 = r.export(b.GS_EXPORT_SORTED_IDS).cpu().numpy()[: r.n_pairs].copy()
        rg1 = r.export(b.GS_EXPORT_RANGES).cpu().numpy().copy()
        st, n = b.gs_bin_sort(r.ctx, None, raise_on_overflow=False)
        assert st == b.GS_OK and n == r.n_pairs
        ids2 = r.export(b.GS_EXPORT_SORTED_IDS).cpu().numpy()[: r.n_pairs]
        rg2 = r.export(b.GS_EXPORT_RANGES).cpu().numpy()
        torch.cuda.synchronize()
        assert np.array_equal(ids1, ids2) and np.array_equal(rg1, rg2)
    finally:
        r.close()


@pytest.mark.parametrize("name", ["c2_small", "c5_small", "elongated"])
def test_tile_order_leaves_outputs_unchanged(name):
    """The first render of a context takes the tiles in index order, the next one in the
    order the first measured (longest first), and the traversals after each render in
    its measured order: every output of two steps on the same inputs is bit-identical."""
    _need_gpu()
    b = _binding()
    sc = _small_scenes()[name]()
    obs = torch.from_numpy(oracle.render_observation(sc)).cuda()
    r = b.rasterizer_for_scene(sc)
    try:
        outs = []
        for _ in range(2):
            (color, T, n), tok = r.step(obs)
            torch.cuda.synchronize()
            outs.append([x.cpu().numpy().copy() for x in (color, T, n, tok)])
        for a, c in zip(outs[0], outs[1]):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  c.view(np.uint32) if c.dtype == np.float32 else c)
    finally:
        r.close()
