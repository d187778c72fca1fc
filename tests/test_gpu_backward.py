"""Parity of the HIP renderer backward (gs_backward, through the C ABI) with the
oracle's float64 chain rule, on the same seeded scenes and upstream gradients.

Bar: per parameter group (means, quaternions, scales, opacities, SH), the
relative L2 error over all Gaussians within GRAD_RTOL, and per Gaussian within
GRAD_RTOL_ONE of that Gaussian's group norm plus a floor of 1e-2 of the
group's RMS per-Gaussian norm.  The GPU sums the per-pixel terms in float32
(pixel offsets from the float32 centre), so a sum whose terms cancel carries
an absolute error of about 1e-7 of the summed magnitudes: a Gaussian whose
opacity terms cancel a thousandfold has a small gradient with a relative
error near 1e-4 (measured 1.3e-3 of a 1e-3-RMS floor on the two-view
ReSplat-like scene), which the floor turns into an absolute allowance of
1e-5 of the typical gradient.  The chain rule itself runs in float64 on both
sides.  Gaussians that no pixel reached get exactly zero.
"""
import zlib

import numpy as np
import pytest

import oracle
import scenes

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

GRAD_RTOL = 1e-4
GRAD_RTOL_ONE = 1e-3
GROUPS = {"means": slice(0, 3), "quats": slice(3, 7), "scales": slice(7, 10), "opacities": slice(10, 11)}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _scenes():
    return {
        "rotated_clip": lambda: scenes.rotated_clip_scene(),
        "c1_toy": lambda: scenes.make_scene(1),
        "tiny_bg_deg1": lambda: scenes.tiny_scene(seed=5, n=30, n_views=3, W=33, H=17, sh_degree=1,
                                                  background=(0.3, 0.6, 0.1)),
        "c2_small": lambda: scenes.c2_resplat_step(n_views=2, W=112, H=64),
        "c5_small": lambda: scenes.c5_multiview_layers(n_views=3, W=100, H=56, n=12000),
        "elongated": lambda: scenes.tiny_scene(seed=8, n=400, n_views=2, W=96, H=80, sh_degree=3,
                                               log_scale=(-3.0, 1.6), spread=0.6),
        "tiny_deg0": lambda: scenes.tiny_scene(seed=13, n=50, n_views=2, W=48, H=40, sh_degree=0),
        # antialiased (opacity-compensated) mode: the compensation's covariance path
        "rotated_clip_aa": lambda: scenes.rotated_clip_scene(),
        "c2_small_aa": lambda: scenes.c2_resplat_step(n_views=2, W=112, H=64),
    }


def _aa(name):
    return name.endswith("_aa")


_CACHE = {}


def _grad_input(name, sc):
    """Upstream gradient: the residual of a rendered observation for the workloads
    (the gradient of 1/2 |C_hat - C|^2), uniform(-1, 1) for the synthetic cases."""
    if name in ("c2_small", "c5_small", "c1_toy", "c2_small_aa"):
        obs = oracle.render_observation(sc, antialiased=_aa(name))
        o = oracle.OracleScene(sc, antialiased=_aa(name))
        color, _, _, _ = o.render()
        o.close()
        return (color - obs.astype(np.float64)).astype(np.float32)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    return rng.uniform(-1, 1, size=(sc.n_views, sc.height, sc.width, 3)).astype(np.float32)


def _flat(grads, d):
    n = grads["means"].shape[0]
    return np.concatenate([grads["means"].reshape(n, 3), grads["quats"].reshape(n, 4),
                           grads["scales"].reshape(n, 3), grads["opacities"].reshape(n, 1),
                           grads["sh"].reshape(n, 3 * d)], axis=1).astype(np.float64)


def _case(name):
    if name not in _CACHE:
        _need_gpu()
        from gaussian_splatting_rasterizer_amd import binding
        sc = _scenes()[name]()
        gC = _grad_input(name, sc)
        o = oracle.OracleScene(sc, antialiased=_aa(name))
        o.build_lists()
        ref, g2d = o.backward(gC, with_image_sums=True)
        o.close()
        r = binding.rasterizer_for_scene(sc, antialiased=_aa(name))
        r.project_and_bin()
        r.render()
        grads = r.backward(torch.from_numpy(gC).cuda())
        torch.cuda.synchronize()
        got = _flat({k: v.cpu().numpy() for k, v in grads.items()}, sc.d)
        r.close()
        _CACHE[name] = (sc, gC, ref, g2d, got)
    return _CACHE[name]


NAMES = list(_scenes().keys())


def _group_slices(d):
    out = dict(GROUPS)
    out["sh"] = slice(11, 11 + 3 * d)
    return out


@pytest.mark.parametrize("name", NAMES)
def test_backward_parity(name):
    sc, gC, ref, g2d, got = _case(name)
    assert np.all(np.isfinite(got))
    rtol, rtol_one = GRAD_RTOL, GRAD_RTOL_ONE
    bad = []
    for group, sl in _group_slices(sc.d).items():
        a, b = got[:, sl], ref[:, sl]
        nb = np.linalg.norm(b)
        rel = np.linalg.norm(a - b) / max(nb, 1e-30)
        per = np.linalg.norm(a - b, axis=1)
        norms = np.linalg.norm(b, axis=1)
        floor = 1e-2 * np.sqrt(np.mean(norms ** 2))
        worst = (per / (norms + floor)).max()
        print(f"{name} {group}: rel L2 {rel:.2e}, worst per-Gaussian {worst:.2e}, |ref| {nb:.3e}")
        if not (rel <= rtol and worst <= rtol_one):
            bad.append((group, rel, worst, int((per / (norms + floor)).argmax())))
    assert not bad, bad


@pytest.mark.parametrize("name", NAMES)
def test_unreached_gaussians_get_zero(name):
    sc, gC, ref, g2d, got = _case(name)
    unreached = np.abs(g2d).sum(axis=(0, 2)) == 0
    assert np.all(got[unreached] == 0.0)
    assert np.all(ref[unreached] == 0.0)


def test_backward_null_members_and_repeat():
    """Null gradient members are skipped (their buffers untouched); a second call
    after a score replay on the same render gives the same gradients."""
    _need_gpu()
    from gaussian_splatting_rasterizer_amd import binding
    sc = scenes.tiny_scene(seed=5, n=30, n_views=3, W=33, H=17, sh_degree=1, background=(0.3, 0.6, 0.1))
    gC = torch.from_numpy(np.random.default_rng(3).uniform(-1, 1, size=(3, 17, 33, 3)).astype(np.float32)).cuda()
    r = binding.rasterizer_for_scene(sc)
    r.project_and_bin()
    r.render()
    full = {k: v.clone() for k, v in r.backward(gC).items()}
    part = r.new_grads()
    for k in part:
        part[k].fill_(7.0)
    part["quats"] = None
    part["sh"] = None
    r.backward(gC, part)
    for k in ("means", "scales", "opacities"):
        assert torch.equal(part[k], full[k])
    obs = torch.zeros((3, 17, 33, 3), dtype=torch.float32, device="cuda")
    r.score_replay(obs)
    again = r.backward(gC)
    for k in full:
        assert torch.equal(again[k], full[k]), k
    torch.cuda.synchronize()
    r.close()


def test_backward_before_render_is_a_state_error():
    _need_gpu()
    from gaussian_splatting_rasterizer_amd import binding
    sc = scenes.tiny_scene(seed=5, n=10, n_views=1, W=16, H=16, sh_degree=0)
    r = binding.rasterizer_for_scene(sc)
    r.project_and_bin()
    gC = torch.zeros((1, 16, 16, 3), dtype=torch.float32, device="cuda")
    with pytest.raises(binding.GsrError) as ei:
        r.backward(gC)
    assert ei.value.status == binding.GS_ERR_STATE
    r.close()
