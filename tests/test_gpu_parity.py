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
import ctypes
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
        # tile lists of 4,710-5,000 faint Gaussians, every entry processed (no pixel saturates): the score
        # replay walks each list as the most segments the render leaves checkpoints for, the last one long
        "deep_lists": lambda: scenes.tiny_scene(seed=41, n=5000, n_views=2, W=40, H=32, sh_degree=1,
                                                log_scale=(-0.7, 0.2), logit=(-6.0, 0.5), spread=0.2),
        # 3,000-entry lists whose tiles are done after 324-1,997 entries: segments that end where the render
        # stopped
        "deep_saturating": lambda: scenes.tiny_scene(seed=42, n=3000, n_views=1, W=48, H=40, sh_degree=2,
                                                     log_scale=(-0.3, 0.2), logit=(-3.0, 0.5), spread=0.3),
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
                    rec[1, :, 2], rec[1, :, 3], rec[2, :, 0], rec[2, :, 2], rec[2, :, 3]], axis=1)[live]
    want = r32[live][:, [1, 2, 5, 6, 7, 9, 10, 11, 12, 3, 4]]
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), np.argwhere(got != want)[:5]
    lo = rec[3, live, 0].view(np.uint32)
    hi = rec[3, live, 1].view(np.uint32)
    rect = np.stack([lo & 0xFFFF, lo >> 16, hi & 0xFFFF, hi >> 16], axis=1)
    assert np.array_equal(rect, r32[live][:, 15:19].astype(np.uint32))


def _box_f64(s1, s2, s3, opac):
    """Reference half-widths of the region where an entry can pass the alpha test: with
    K = L L^T, L = [[s1, 0], [s2, s3]], S*(d) = d^T K d <= t_eff,
    t_eff = (min(8, log2 255 o) + 1e-5) / (1 - u (8 + 10 sqrt(kappa))), u = 2^-24,
    kappa = max(Kinv_xx, Kinv_yy)^2 / det(Kinv), widened by 0.01 px; float64 from the
    float32 factors.  Returns (wx, wy, kind) with kind 0 finite, 1 unbounded (never
    skipped), -1 empty."""
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        tt = np.log2(255.0 * opac)
        p1, p3 = s1 * s1, s3 * s3
        kxx, kyy, kdet = (s2 * s2 + p3) / (p1 * p3), 1.0 / p3, 1.0 / (p1 * p3)
        kmax = np.maximum(kxx, kyy)
        grow = 2.0 ** -24 * (8.0 + 10.0 * np.sqrt(kmax * kmax / kdet))
        te = (np.minimum(tt, 8.0) + 1e-5) / (1.0 - grow)
        wx, wy = np.sqrt(te * kxx) + 0.01, np.sqrt(te * kyy) + 0.01
    kind = np.where(~(tt > -1e-5), -1, np.where(~(p1 > 0) | ~(p3 > 0) | ~(grow < 0.5), 1, 0))
    return wx, wy, kind


@pytest.mark.parametrize("name", SMALL)
def test_entry_boxes_conservative(name):
    """Every live record's packed entry box (two binary16 half-widths, rounded up) holds
    the float64 box computed from the record's own float32 factors: the render may skip
    an entry only where it provably cannot pass the alpha test."""
    sc, obs, ref, gpu = _case(name)
    rec = gpu["rec"]
    live = gpu["keys"] != 0xFFFFFFFF
    r0, r1, r2 = rec[0, live].astype(np.float64), rec[1, live].astype(np.float64), rec[2, live]
    wx, wy, kind = _box_f64(r0[:, 2], r0[:, 3], r1[:, 0], r1[:, 1])
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


# Every scene, the needle-like footprints (conic condition numbers up to ~7e4) and the
# 4200-px-wide image included, is held to the same colour bar: the exponent is evaluated as a
# sum of squares from its Cholesky factor and the centre relative to the tile (see the
# preprocess), so neither the conditioning nor the distance from the image origin costs precision.
@pytest.mark.parametrize("name", SMALL)
def test_render_parity(name):
    sc, obs, ref, gpu = _case(name)
    assert np.array_equal(gpu["n"], ref["n"]), np.argwhere(gpu["n"] != ref["n"])[:5]
    assert np.array_equal(gpu["T"].view(np.uint32), ref["T"].view(np.uint32))
    err = np.abs(gpu["color"] - ref["color"]).max()
    print(name, "max colour error", err)
    assert err <= COLOR_ATOL, err





@pytest.mark.parametrize("name", SMALL)
def test_token_parity(name):
    """Every Gaussian's token: the whole token within 1e-3 relative L2, and each block
    (b_mu, s_alpha, s_SH, the statistics) within 1e-3 of its own norm plus the float32
    floor derived in oracle.token_block_errors (cancelling per-pixel terms, and what the
    colour tolerance moves the residual and the suffix by)."""
    sc, obs, ref, gpu = _case(name)
    z = gpu["tokens"].astype(np.float64)
    zr = ref["tokens"]
    rel = np.linalg.norm(z - zr, axis=1) / np.maximum(np.linalg.norm(zr, axis=1), 1e-6)
    blocks = oracle.token_block_errors(ref["oracle"], z, zr, catol=COLOR_ATOL)
    print(name, "max rel", rel.max(), "per block (error / bound)", {k: round(v[0], 4) for k, v in blocks.items()})
    assert np.all(np.isfinite(gpu["tokens"]))
    assert rel.max() <= TOKEN_RTOL, (rel.max(), int(rel.argmax()))
    bad = {k: v for k, v in blocks.items() if not v[0] <= 1.0}
    assert not bad, bad


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
        step_stages = ("project", "depth_sort", "scan", "emit", "tile_sort", "render", "replay", "finalize")
        assert all(prof[k][1] == 1 for k in step_stages), prof
        assert prof["ranges"][1] == 0, prof  # the emission sets the ranges: no launch of its own
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


@pytest.mark.parametrize("name", ["c2_small", "c5_small", "elongated", "deep_saturating"])
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


def test_rejected_project_leaves_the_context_unchanged():
    """gs_project validates every camera before it changes the context: a call rejected for a
    bad camera of its last view leaves the cameras and the state of the previous render, so a
    following score replay gives the same tokens as one without the rejected call."""
    _need_gpu()
    b = _binding()
    sc = scenes.tiny_scene(seed=5, n=30, n_views=3, W=33, H=17, sh_degree=1, background=(0.3, 0.6, 0.1))
    obs = torch.from_numpy(oracle.render_observation(sc)).cuda()
    r = b.rasterizer_for_scene(sc)
    try:
        r.project_and_bin()
        r.render()
        want = r.score_replay(obs).clone()
        bad = sc.cams.copy()
        bad[2, 12] = 0.0                      # focal length of the last view
        st = b.load_library().gs_project(r.ctx, ctypes.byref(r.gauss), b.make_cameras(bad), ctypes.byref(r.params),
                                         None)
        assert st == b.GS_ERR_INVALID_ARGUMENT
        got = r.score_replay(obs)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
    finally:
        r.close()


@pytest.mark.parametrize("name", ["deep_saturating", "c2_small"])
def test_workspace_contents_are_never_assumed(name):
    """A workspace filled with 0xff bytes before the first call (so that every event byte past the entries the
    render processes names all four waves) gives the oracle's outputs, and a second step and a second
    backward on it are bit-identical to the first: the traversals after the render read only the entries it
    processed."""
    sc, obs, ref, _ = _case(name)
    b = _binding()
    r = b.rasterizer_for_scene(sc)
    try:
        r.workspace.fill_(255)
        torch.cuda.synchronize()
        obs_d = torch.from_numpy(obs).cuda()
        gC = torch.from_numpy(np.random.default_rng(7).uniform(-1, 1, size=obs.shape).astype(np.float32)).cuda()
        outs, grads = [], []
        for _ in range(2):
            (color, T, n), tok = r.step(obs_d)
            g = r.backward(gC)
            torch.cuda.synchronize()
            outs.append([x.cpu().numpy().copy() for x in (color, T, n, tok)])
            grads.append({k: v.cpu().numpy().copy() for k, v in g.items()})
        color, T, n, tok = outs[0]
        assert np.array_equal(n, ref["n"]) and np.array_equal(T.view(np.uint32), ref["T"].view(np.uint32))
        assert np.abs(color - ref["color"]).max() <= COLOR_ATOL
        z, zr = tok.astype(np.float64), ref["tokens"]
        rel = np.linalg.norm(z - zr, axis=1) / np.maximum(np.linalg.norm(zr, axis=1), 1e-6)
        assert rel.max() <= TOKEN_RTOL, rel.max()
        blocks = oracle.token_block_errors(ref["oracle"], z, zr, catol=COLOR_ATOL)
        assert all(v[0] <= 1.0 for v in blocks.values()), blocks
        for a, c in zip(outs[0], outs[1]):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  c.view(np.uint32) if c.dtype == np.float32 else c)
        for k in grads[0]:
            assert np.array_equal(grads[0][k].view(np.uint32), grads[1][k].view(np.uint32)), k
    finally:
        r.close()
