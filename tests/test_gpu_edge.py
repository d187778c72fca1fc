"""Parity with the oracle on the degenerate inputs of the method, through the C ABI:

  * non-finite parameters (NaN / +-Inf means, quaternion, scale, opacity; an
    opacity outside [0, 1]; a zero quaternion): the boundary's reading is that
    such (Gaussian, view) pairs are culled -- never an error --, and a
    non-finite SH coefficient makes its channel's colour clamped and masked
    (the page "Research Proposal: Renderer Score Tokens for Recurrent Gaussian
    Splatting", Stage 2: explicit masks for numerically unstable
    contributions);
  * a scene whose every Gaussian is culled: no (tile, Gaussian) pair, so the
    tile sort runs on zero keys and every tile range is empty;
  * no Gaussians at all.

Each case is checked against the oracle, whose behaviour on them is pinned on
the CPU (tests/test_oracle_pins.py, degenerate inputs): records, lists, every
pixel, every token (whole and per block) and the renderer backward.
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle
import scenes
from test_oracle_pins import NONFINITE_CULLED, nonfinite_scene

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

COLOR_ATOL = 1e-5


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _scene(name):
    base = scenes.tiny_scene(seed=21, n=30, n_views=2, W=40, H=24, sh_degree=1, background=(0.3, 0.6, 0.1))
    if name == "nonfinite":
        return nonfinite_scene(base)
    if name == "all_culled":
        m = base.means.copy()
        m[:, 2] = -m[:, 2]
        return dataclasses.replace(base, means=m, means_perturbed=m)
    if name == "no_gaussians":
        keep = np.zeros(0, dtype=np.int64)
        return dataclasses.replace(base, means=base.means[keep], quats=base.quats[keep],
                                   scales=base.scales[keep], opacities=base.opacities[keep],
                                   sh=base.sh[keep], means_perturbed=base.means[keep])
    raise KeyError(name)


def _run(name):
    _need_gpu()
    from gaussian_splatting_rasterizer_amd import binding
    sc = _scene(name)
    obs = np.random.default_rng(4).uniform(0, 1, size=(sc.n_views, sc.height, sc.width, 3)).astype(np.float32)
    gC = np.random.default_rng(5).uniform(-1, 1, size=obs.shape).astype(np.float32)
    print(f"edge case {name}: {sc.n} Gaussians, {sc.n_views} views {sc.width}x{sc.height}", flush=True)
    r = binding.rasterizer_for_scene(sc)
    r.project_and_bin()
    gpu = dict(n_pairs=r.n_pairs)
    if sc.n > 0:
        gpu["rec"] = r.export(binding.GS_EXPORT_RECORDS).cpu().numpy()
        gpu["keys"] = r.export(binding.GS_EXPORT_DEPTH_KEYS).cpu().numpy().view(np.uint32)
    gpu["ids"] = r.export(binding.GS_EXPORT_SORTED_IDS).cpu().numpy()[: r.n_pairs]
    gpu["ranges"] = r.export(binding.GS_EXPORT_RANGES).cpu().numpy()
    color, T, n = r.render()
    tok = r.score_replay(torch.from_numpy(obs).cuda())
    grads = r.backward(torch.from_numpy(gC).cuda())
    torch.cuda.synchronize()
    gpu.update(color=color.cpu().numpy(), T=T.cpu().numpy(), n=n.cpu().numpy(), tokens=tok.cpu().numpy(),
               grads={k: v.cpu().numpy() for k, v in grads.items()})
    r.close()
    ref = oracle.full_reference(sc, obs)
    ref["starts"], ref["ids"] = ref["oracle"].lists()
    ref["grads"] = ref["oracle"].backward(gC)
    return sc, gpu, ref


@pytest.mark.parametrize("name", ["nonfinite", "all_culled", "no_gaussians"])
def test_degenerate_inputs_match_oracle(name):
    sc, gpu, ref = _run(name)
    o = ref["oracle"]
    # records: culled exactly where the oracle culls, live ones bit-exact (NaN pre-clamp colours
    # compared as NaN: their payload bits are not specified)
    if sc.n > 0:
        r32 = o.records32().reshape(-1, 20)
        live = r32[:, 0] == 0
        assert np.array_equal(gpu["keys"] == 0xFFFFFFFF, ~live)
        rec = gpu["rec"]
        got = np.stack([rec[0, :, 0], rec[0, :, 1], rec[0, :, 2], rec[0, :, 3], rec[1, :, 0], rec[1, :, 1],
                        rec[1, :, 2], rec[1, :, 3], rec[2, :, 0], rec[2, :, 2], rec[2, :, 3]], axis=1)[live]
        want = r32[live][:, [1, 2, 5, 6, 7, 9, 10, 11, 12, 3, 4]]
        same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
        assert same.all(), np.argwhere(~same)[:5]
    # lists and ranges
    assert gpu["n_pairs"] == len(ref["ids"])
    assert np.array_equal(gpu["ids"], ref["ids"])
    starts = ref["starts"]
    nonempty = np.diff(starts) > 0
    rg = gpu["ranges"].astype(np.int64)
    assert np.array_equal(rg[nonempty, 0], starts[:-1][nonempty])
    assert np.array_equal(rg[nonempty, 1], starts[1:][nonempty])
    assert np.all(rg[~nonempty, 0] == rg[~nonempty, 1])
    # every pixel
    assert np.array_equal(gpu["n"], ref["n"])
    assert np.array_equal(gpu["T"].view(np.uint32), ref["T"].view(np.uint32))
    assert np.all(np.isfinite(gpu["color"]))
    assert np.abs(gpu["color"] - ref["color"]).max() <= COLOR_ATOL
    if gpu["n_pairs"] == 0:
        bg = np.broadcast_to(sc.background.astype(np.float32), gpu["color"].shape)
        assert np.array_equal(gpu["color"], bg) and np.all(gpu["T"] == 1.0) and np.all(gpu["n"] == 0)
    # every token
    z, zr = gpu["tokens"].astype(np.float64), ref["tokens"]
    assert z.shape == zr.shape == (sc.n, 9 + 3 * sc.d)
    assert np.all(np.isfinite(z))
    if sc.n > 0:
        rel = np.linalg.norm(z - zr, axis=1) / np.maximum(np.linalg.norm(zr, axis=1), 1e-6)
        assert rel.max() <= 1e-3, rel.max()
        blocks = oracle.token_block_errors(o, z, zr, catol=COLOR_ATOL)
        bad = {k: v for k, v in blocks.items() if not v[0] <= 1.0}
        assert not bad, bad
        culled_everywhere = np.all(o.records32()[:, :, 0] != 0, axis=0)
        if name == "nonfinite":
            assert culled_everywhere[:len(NONFINITE_CULLED)].all()
        # a Gaussian culled in every view has the zero-support token
        d, V = sc.d, sc.n_views
        want = np.zeros(9 + 3 * d)
        want[4 + 3 * d] = math.log((V + 1) * 1e-6)
        want[5 + 3 * d: 8 + 3 * d] = 1.0 / (3.0 + 1e-6)
        want[8 + 3 * d] = math.log(3.0 + 1e-6)
        assert np.allclose(z[culled_everywhere], want[None, :], rtol=1e-6, atol=1e-7)
    # renderer backward: finite, zero where nothing contributes, and per group within 1e-4
    g = gpu["grads"]
    got = np.concatenate([g["means"], g["quats"], g["scales"], g["opacities"][:, None],
                          g["sh"].reshape(sc.n, 3 * sc.d)], axis=1).astype(np.float64)
    assert np.all(np.isfinite(got))
    want = ref["grads"]
    for sl in (slice(0, 3), slice(3, 7), slice(7, 10), slice(10, 11), slice(11, None)):
        nw = np.linalg.norm(want[:, sl])
        assert np.linalg.norm(got[:, sl] - want[:, sl]) <= 1e-4 * nw
    if sc.n > 0:
        culled_everywhere = np.all(o.records32()[:, :, 0] != 0, axis=0)
        assert np.all(got[culled_everywhere] == 0.0)
