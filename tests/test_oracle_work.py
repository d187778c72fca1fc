"""Pins of the oracle's per-pixel work counts of the render pass (`pixel_work`):
list entries examined up to and including the one at which the pixel stopped
(the whole list when it never did), and those of them past the distance cut
G >= 2^-8.  They are the evaluation counts of the front-to-back loop of the
Standard Render stage (Renderer Score Tokens proposal, "Two-Stage Algorithm"),
which the benchmark's work model multiplies by per-evaluation costs.

Pinned by a closed form (a stack of identical Gaussians saturating a pixel
after a number of entries fixed by (1 - alpha)^k < 1e-4) and by a per-pixel
brute force over the toy scene in float64.
"""
import math

import numpy as np

import oracle
import scenes
from test_oracle_pins import _single


def test_stack_of_identical_gaussians_closed_form():
    # six identical Gaussians at one point: every pixel sees the same alpha six times
    k_stack = 6
    sc = _single([[0.0, 0.0, 2.0]] * k_stack, [1, 0, 0, 0], [0.08, 0.08, 0.08], opac=0.95)
    o = oracle.OracleScene(sc)
    work = o.pixel_work()
    color, T, n, T64 = o.render()
    starts, ids = o.lists()
    r64 = o.records64()[0, 0]
    checked = 0
    for y in range(64):
        for x in range(64):
            tile = (y // 16) * 4 + x // 16
            L = int(starts[tile + 1] - starts[tile])
            dx, dy = x + 0.5 - r64[0], y + 0.5 - r64[1]
            sig = 0.5 * (r64[2] * dx * dx + 2 * r64[3] * dx * dy + r64[4] * dy * dy)
            log2g = -sig / math.log(2.0)
            a = min(0.99, 0.95 * math.exp(-sig))
            if abs(log2g + 8.0) < 1e-4 or abs(a - 1 / 255) < 1e-6:
                continue  # a float32 rounding tie at one of the cuts
            if L == 0:
                assert tuple(work[0, y, x]) == (0, 0)
                continue
            assert L == k_stack
            if a < 1 / 255:  # never contributes: every entry examined, none stops the pixel
                want_e, near = L, (L if log2g >= -8.0 else 0)
            else:
                # contributions k = 0, 1, ... while (1 - a)^(k + 1) >= 1e-4; the next entry stops the pixel
                k = 0
                while k < L and (1 - a) ** (k + 1) >= 1e-4:
                    k += 1
                if k < L and abs((1 - a) ** (k + 1) - 1e-4) < 1e-7:
                    continue  # transmittance tie
                want_e = min(k + 1, L)
                near = want_e
                assert n[0, y, x] == k
            assert tuple(work[0, y, x]) == (want_e, near), (x, y)
            checked += 1
    assert checked >= 1000  # the four tiles the rectangle covers
    # the centre saturates: (1 - 0.95 G)^k with G ~ 0.96 crosses 1e-4 within the stack
    assert work[0, 32, 32, 0] < k_stack


def test_work_counts_by_per_pixel_brute_force():
    """Every pixel of a sample on the toy scene: the tile list walked in float64 with the
    pass's cuts; agrees with the float32-decision counts except at rounding ties."""
    sc = scenes.make_scene(1)
    o = oracle.OracleScene(sc)
    work = o.pixel_work()
    starts, ids = o.lists()
    r64 = o.records64()[0]
    mism = 0
    total = 0
    for y in range(1, 64, 3):
        for x in range(0, 64, 3):
            tile = (y // 16) * 4 + x // 16
            lst = ids[starts[tile]:starts[tile + 1]]
            px, py = x + 0.5, y + 0.5
            Tb, e_cnt, near = 1.0, 0, 0
            for g in lst:
                e_cnt += 1
                dx, dy = px - r64[g, 0], py - r64[g, 1]
                sig = 0.5 * (r64[g, 2] * dx * dx + 2 * r64[g, 3] * dx * dy + r64[g, 4] * dy * dy)
                if -sig / math.log(2.0) < -8.0:
                    continue
                near += 1
                a = min(0.99, r64[g, 5] * math.exp(-sig))
                if a < 1 / 255:
                    continue
                if Tb * (1 - a) < 1e-4:
                    break
                Tb *= 1 - a
            total += 1
            if (e_cnt, near) != tuple(work[0, y, x]):
                mism += 1
    assert total > 400
    assert mism <= 2, mism


def test_work_counts_bound_the_contributions():
    """Invariants on a multi-view scene: contributions <= entries past the cut <= entries
    examined <= list length, and a pixel examines its whole list unless it stopped."""
    sc = scenes.tiny_scene(seed=21, n=60, n_views=2, W=40, H=24, sh_degree=2)
    o = oracle.OracleScene(sc)
    work = o.pixel_work().astype(np.int64)
    color, T, n, T64 = o.render()
    starts, ids = o.lists()
    V, H, W = n.shape
    ty, tx = np.mgrid[0:H, 0:W]
    tiles = (ty // 16) * o.TX + tx // 16
    for v in range(V):
        L = (starts[v * o.T + tiles + 1] - starts[v * o.T + tiles]).astype(np.int64)
        e, near = work[v, ..., 0], work[v, ..., 1]
        assert np.all(n[v] <= near) and np.all(near <= e) and np.all(e <= L)
        stopped = e < L
        # a pixel that stopped early did so at an entry that would have taken T below 1e-4
        assert np.all(T[v][stopped] >= 1e-4)
