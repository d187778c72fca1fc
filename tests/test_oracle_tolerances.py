"""Checks of the per-block token tolerance (oracle.token_block_errors) on the CPU.

The tolerance floors rest on the oracle's sensitivity sums: for each masked score
term f_p <r, c - C+> (opacity, centre x, centre y) they hold sum_p |f_p| |c - C+|_1
and sum_p |f_p| |r|_1 / (T (1 - alpha) + eps).  The first bounds how far the score
moves when the residual moves by at most h per channel; this is checked here by
moving the observation.  The comparison itself must pass the oracle's own tokens
and fail tokens with a one-percent error in any single block.
"""
import numpy as np
import pytest

import oracle
import scenes


@pytest.fixture(scope="module")
def replay():
    sc = scenes.tiny_scene(seed=17, n=40, n_views=2, W=48, H=32, sh_degree=2)
    obs = np.random.default_rng(3).uniform(0, 1, size=(2, 32, 48, 3)).astype(np.float32)
    o = oracle.OracleScene(sc)
    o.select(None)
    o.render(obs=obs)
    return sc, obs, o, o.acc(), o.tokens()


def test_residual_sensitivity_bounds_a_moved_observation(replay):
    sc, obs, o, acc, tok = replay
    h = 1e-4
    delta = h * np.sign(np.random.default_rng(4).normal(size=obs.shape))
    o2 = oracle.OracleScene(sc)
    o2.select(None)
    o2.render(obs=(obs.astype(np.float64) + delta).astype(np.float32))
    acc2 = o2.acc()
    na = acc.shape[2]
    sens_c = acc[:, :, na - oracle.NACC_SENS: na - oracle.NACC_SENS + 3]
    moved = np.abs(acc2[:, :, 1:4] - acc[:, :, 1:4])
    # the float32 observation rounds delta by at most 2^-24 per channel
    assert np.all(moved <= (h + 1e-7) * sens_c + 1e-12), (moved / np.maximum(sens_c * h, 1e-30)).max()
    assert (sens_c > 0).sum() > 20 and moved.max() > 0


def test_block_errors_pass_the_oracle_and_fail_planted_block_errors(replay):
    sc, obs, o, acc, tok = replay
    res = oracle.token_block_errors(o, tok, tok)
    assert all(r <= 1e-9 for r, _ in res.values()), res
    supported = acc[:, :, 0].sum(axis=1) > 1.0
    d = sc.d
    for name, sl in (("b_mu", slice(0, 3)), ("s_alpha", slice(3, 4)), ("s_sh", slice(4, 4 + 3 * d)),
                     ("stats", slice(4 + 3 * d, 9 + 3 * d))):
        bad = tok.copy()
        bad[:, sl] *= 1.01
        res = oracle.token_block_errors(o, bad, tok)
        assert res[name][0] > 1.0, (name, res[name])
        # the planted error is invisible in the whole-token norm for most supported Gaussians
        # when the block is small next to log Q and log tr A
        if name in ("b_mu", "s_alpha"):
            rel = np.linalg.norm(bad - tok, axis=1) / np.linalg.norm(tok, axis=1)
            assert np.median(rel[supported]) < 1e-3


def test_centre_sensitivity_bounds_a_moved_centre(replay):
    """The centre sensitivity sums bound how far the opacity and centre terms move when every
    projected centre moves by at most h px along each axis (decisions frozen, first order)."""
    sc, obs, o, acc, tok = replay
    h = 1e-5
    na = acc.shape[2]
    sens_m = acc[:, :, na - 3: na]
    r64 = o.records64()
    rng = np.random.default_rng(6)
    checked = 0
    for g in rng.choice(sc.n, size=12, replace=False):
        for v in range(sc.n_views):
            if acc[g, v, 0] < 1e-3:
                continue
            mx, my = r64[v, g, 0], r64[v, g, 1]
            sx, sy = rng.choice([-1.0, 1.0], size=2)
            o.set_mean2d64(int(g), v, mx + sx * h, my + sy * h)
            o.select(None)
            o.render(obs=obs)
            moved = np.abs(o.acc()[g, v, 1:4] - acc[g, v, 1:4])
            o.values_reset()
            assert np.all(moved <= 1.01 * h * sens_m[g, v] + 1e-13), (g, v, moved, h * sens_m[g, v])
            checked += 1
    o.select(None)
    o.render(obs=obs)
    assert checked >= 6
