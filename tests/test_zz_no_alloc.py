"""The no-allocation entry point (gs_render_score_noalloc, for callers that cannot
allocate) against the four-call path on the same inputs, through the C ABI: two calls
in a row on the one scratch array of the GPU, the second with a smaller scene, each
bit-identical to gs_project -> gs_bin_sort -> gs_render -> gs_score_replay on a
caller-allocated workspace (colour within 1e-5, counts and transmittance exact,
tokens within 1e-3 relative L2 is the bar; the kernels are the same, so the outputs
are expected identical).  A problem beyond the array's size is rejected with
GS_ERR_WORKSPACE_TOO_SMALL before anything is written."""
import ctypes

import numpy as np
import pytest

import scenes

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _regular(sc, obs):
    from gaussian_splatting_rasterizer_amd import binding
    r = binding.rasterizer_for_scene(sc)
    (color, T, n), tok = r.step(obs)
    torch.cuda.synchronize()
    out = [x.cpu().numpy().copy() for x in (color, T, n, tok)]
    r.close()
    return out


def _noalloc(sc, obs):
    from gaussian_splatting_rasterizer_amd import binding
    lib = binding.load_library()
    f32 = dict(dtype=torch.float32, device="cuda")
    keep = [torch.as_tensor(getattr(sc, k), **f32).contiguous() for k in ("means", "quats", "scales", "opacities", "sh")]
    gauss = binding.gs_gaussians(*[ctypes.c_void_p(t.data_ptr()) for t in keep], sc.n, sc.sh_degree)
    cams = binding.make_cameras(sc.cams)
    params = binding.gs_default_params()
    params.background[:] = [float(x) for x in np.asarray(sc.background, dtype=np.float32)]
    V, H, W = sc.n_views, sc.height, sc.width
    color = torch.full((V, H, W, 3), -1.0, **f32)
    T = torch.full((V, H, W), -1.0, **f32)
    n = torch.full((V, H, W), -1, dtype=torch.int32, device="cuda")
    tok = torch.full((sc.n, 9 + 3 * sc.d), -1.0, **f32)
    st = lib.gs_render_score_noalloc(ctypes.byref(gauss), cams, V, W, H, ctypes.byref(params),
                                     ctypes.c_void_p(obs.data_ptr()), ctypes.c_void_p(color.data_ptr()),
                                     ctypes.c_void_p(T.data_ptr()), ctypes.c_void_p(n.data_ptr()),
                                     ctypes.c_void_p(tok.data_ptr()), None)
    assert st == binding.GS_OK, lib.gs_last_error().decode()
    torch.cuda.synchronize()
    return [x.cpu().numpy().copy() for x in (color, T, n, tok)]


def _check(sc):
    obs = torch.from_numpy((0.5 + 5.0 * sc.pixel_noise).astype(np.float32)).cuda()
    want = _regular(sc, obs)
    got = _noalloc(sc, obs)
    color, T, n, tok = got
    assert np.array_equal(n, want[2])
    assert np.array_equal(T.view(np.uint32), want[1].view(np.uint32))
    assert np.abs(color - want[0]).max() <= 1e-5
    rel = np.linalg.norm(tok - want[3], axis=1) / np.maximum(np.linalg.norm(want[3], axis=1), 1e-6)
    assert rel.max() <= 1e-3, rel.max()
    # the same kernels on the same inputs: identical outputs
    assert np.array_equal(color.view(np.uint32), want[0].view(np.uint32))
    assert np.array_equal(tok.view(np.uint32), want[3].view(np.uint32))
    return int(np.count_nonzero(n))


def test_noalloc_matches_the_four_calls_twice_then_smaller():
    _need_gpu()
    big = scenes.c2_resplat_step(n_views=2, W=112, H=64)
    small = scenes.tiny_scene(seed=21, n=60, n_views=2, W=40, H=24, sh_degree=2)
    print(f"no-alloc call 1: {big.n} Gaussians, {big.n_views} views {big.width}x{big.height}", flush=True)
    assert _check(big) > 0
    print(f"no-alloc call 2: {small.n} Gaussians, {small.n_views} views {small.width}x{small.height}", flush=True)
    assert _check(small) > 0


def test_noalloc_rejects_a_problem_beyond_the_scratch_array():
    _need_gpu()
    from gaussian_splatting_rasterizer_amd import binding
    lib = binding.load_library()
    n = 600_000   # ~ 600k records of ~170 workspace bytes each: beyond 64 MiB before any pair
    dummy = torch.zeros(16 * n, dtype=torch.float32, device="cuda")
    p = ctypes.c_void_p(dummy.data_ptr())
    gauss = binding.gs_gaussians(p, p, p, p, p, n, 3)
    cams = binding.make_cameras(np.tile(np.array([1, 0, 0, 0, 1, 0, 0, 0, 1, 0, 0, 0, 64, 64, 32, 32],
                                                 np.float32), (1, 1)))
    params = binding.gs_default_params()
    st = lib.gs_render_score_noalloc(ctypes.byref(gauss), cams, 1, 64, 64, ctypes.byref(params), p, p, p, p, p,
                                     None)
    assert st == binding.GS_ERR_WORKSPACE_TOO_SMALL
    assert "scratch array" in lib.gs_last_error().decode()
