"""Parity at the full sizes of the five workloads, over whole frames: every tile
list (bit-exact against the oracle's brute-force lists), every pixel (colour
<= 1e-5, counts and final transmittance bit-exact), the token of every Gaussian
(<= 1e-3 relative L2 for the whole token, and per block: b_mu, s_alpha, s_SH and
the statistics block each within 1e-3 of its own norm plus the float32 floor of
oracle.token_block_errors), and the renderer-backward gradients of every
Gaussian for a seeded upstream gradient (<= 1e-4 relative L2 per parameter
group).  The GPU runs the same launch configuration as bench.py; the observation
is the workload's own (the oracle's render of the perturbed scene plus pixel
noise).

Each configuration is one test that runs every check and reports all failures
together, so that its full-frame arrays can be dropped before the next one.
"""
import time

import numpy as np
import pytest

import oracle
import scenes

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TOKEN_RTOL = 1e-3
COLOR_ATOL = 1e-5
GRAD_RTOL = 1e-4


def _gpu_pass(sc, obs, gC):
    from gaussian_splatting_rasterizer_amd import binding
    r = binding.rasterizer_for_scene(sc)
    r.project_and_bin()
    ids = r.export(binding.GS_EXPORT_SORTED_IDS).cpu().numpy()[: r.n_pairs]
    ranges = r.export(binding.GS_EXPORT_RANGES).cpu().numpy()
    color, T, n = r.render()
    tok = r.score_replay(torch.from_numpy(obs).cuda())
    grads = r.backward(torch.from_numpy(gC).cuda())
    torch.cuda.synchronize()
    gpu = dict(ids=ids, ranges=ranges, n_pairs=r.n_pairs, color=color.cpu().numpy(), T=T.cpu().numpy(),
               n=n.cpu().numpy(), tokens=tok.cpu().numpy(),
               grads=np.concatenate([grads["means"].cpu().numpy(), grads["quats"].cpu().numpy(),
                                     grads["scales"].cpu().numpy(), grads["opacities"].cpu().numpy()[:, None],
                                     grads["sh"].cpu().numpy().reshape(sc.n, -1)], axis=1).astype(np.float64))
    r.close()
    del r, color, T, n, tok, grads
    torch.cuda.empty_cache()
    return gpu


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5])
def test_fullsize(config):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    t0 = time.perf_counter()
    sc = scenes.make_scene(config)
    obs = oracle.render_observation(sc)
    gC = np.random.default_rng(200 + config).uniform(
        -1, 1, size=(sc.n_views, sc.height, sc.width, 3)).astype(np.float32)
    gpu = _gpu_pass(sc, obs, gC)
    t1 = time.perf_counter()
    ref = oracle.full_reference(sc, obs)
    o = ref["oracle"]
    starts, ids = o.lists()
    t2 = time.perf_counter()
    fails = []

    # tile lists and ranges
    if gpu["n_pairs"] != len(ids) or not np.array_equal(gpu["ids"], ids):
        fails.append(("lists", gpu["n_pairs"], len(ids)))
    rg = gpu["ranges"].astype(np.int64)
    nonempty = np.diff(starts) > 0
    if not (np.array_equal(rg[nonempty, 0], starts[:-1][nonempty])
            and np.array_equal(rg[nonempty, 1], starts[1:][nonempty])
            and np.all(rg[~nonempty, 0] == rg[~nonempty, 1])):
        fails.append(("ranges",))

    # every pixel
    if not np.array_equal(gpu["n"], ref["n"]):
        fails.append(("n_contrib", int((gpu["n"] != ref["n"]).sum())))
    if not np.array_equal(gpu["T"].view(np.uint32), ref["T"].view(np.uint32)):
        fails.append(("T_final", int((gpu["T"] != ref["T"]).sum())))
    cerr = float(np.abs(gpu["color"] - ref["color"]).max())
    if not cerr <= COLOR_ATOL:
        fails.append(("colour", cerr))

    # every Gaussian's token: whole and per block
    z = gpu["tokens"].astype(np.float64)
    zr = ref["tokens"]
    if not np.all(np.isfinite(z)):
        fails.append(("tokens not finite", int((~np.isfinite(z)).sum())))
    rel = np.linalg.norm(z - zr, axis=1) / np.maximum(np.linalg.norm(zr, axis=1), 1e-6)
    if not rel.max() <= TOKEN_RTOL:
        fails.append(("token", float(rel.max()), int(rel.argmax())))
    blocks = oracle.token_block_errors(o, z, zr, catol=COLOR_ATOL)
    for name, (ratio, k) in blocks.items():
        if not ratio <= 1.0:
            fails.append((name, ratio, k))

    # renderer backward of every Gaussian
    g_ref = o.backward(gC)
    t3 = time.perf_counter()
    groups = {"means": slice(0, 3), "quats": slice(3, 7), "scales": slice(7, 10), "opacities": slice(10, 11),
              "sh": slice(11, 11 + 3 * sc.d)}
    grel = {}
    if not np.all(np.isfinite(gpu["grads"])):
        fails.append(("grads not finite",))
    for name, sl in groups.items():
        grel[name] = float(np.linalg.norm(gpu["grads"][:, sl] - g_ref[:, sl])
                           / max(np.linalg.norm(g_ref[:, sl]), 1e-30))
        if not grel[name] <= GRAD_RTOL:
            fails.append(("grad " + name, grel[name]))

    print(f"config {config}: {sc.n} Gaussians, {gpu['n_pairs']} pairs, {sc.n_views * sc.height * sc.width} px; "
          f"max colour error {cerr:.2e}; max token rel {rel.max():.2e}; per block "
          f"{ {k: round(v[0], 4) for k, v in blocks.items()} } (error / bound); grad rel {grel}; "
          f"seconds: setup + GPU {t1 - t0:.1f}, oracle forward {t2 - t1:.1f}, oracle backward {t3 - t2:.1f}")
    o.close()
    assert not fails, fails
