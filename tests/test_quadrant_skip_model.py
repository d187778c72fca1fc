"""The render's quadrant skip, checked on a float32 model by brute force (CPU).

Before a wave walks a list entry, the render asks whether any pixel centre of
the wave's 8x8 quadrant can pass the entry's alpha test: the entry's packed
box must meet the quadrant, and so must the region S*(p - m) <= t_eff, whose
threshold is bounded from the box half-widths and whose minimum over the
quadrant's rectangle is found on the (at most two) edges facing the centre,
all in float32 with margins (gsr_device.hpp, ellipse_meets_rect).  A wrong
"no" would drop a contribution.  This test models the box packing (float64,
binary16 rounded up), the float32 test with the hardware reciprocal's error
(up to 4e-7 relative, drawn at random) and the float32 per-pixel decision
(S <= 8 and o 2^-S >= 1/255), over random ellipses of every orientation and a
wide range of conditioning, and requires that every pixel that passes lies in
a quadrant the test keeps.  Parity of the GPU render with the oracle (every
pixel, bit-exact transmittance and counts) checks the device code itself.
"""
import numpy as np

f32 = np.float32


def _fma32(a, b, c):
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def _half_up(v):
    v = v.astype(np.float32)
    h = v.astype(np.float16)
    hb = h.view(np.uint16).copy()
    hb[h.astype(np.float32) < v] += 1
    out = hb.view(np.float16).astype(np.float32)
    out[~(v <= 65504)] = np.inf
    return out


def test_quadrant_skip_never_drops_a_passing_pixel():
    rng = np.random.default_rng(1)
    n = 120_000
    s1 = (10 ** rng.uniform(-2.5, 1.2, n)).astype(f32)
    s3 = (10 ** rng.uniform(-2.5, 1.2, n)).astype(f32)
    s2 = (rng.normal(0, 1, n) * 10 ** rng.uniform(-2.5, 1.5, n)).astype(f32)
    op = rng.uniform(0.004, 0.99, n).astype(f32)
    mx = rng.uniform(-30, 46, n).astype(f32)
    my = rng.uniform(-30, 46, n).astype(f32)
    q = rng.integers(0, 4, n)
    x0 = ((q & 1) * 8 + 0.5).astype(f32)
    x1 = (x0 + 7).astype(f32)
    y0 = ((q >> 1) * 8 + 0.5).astype(f32)
    y1 = (y0 + 7).astype(f32)
    with np.errstate(all="ignore"):
        # the packed box (float64, as the preprocess computes it)
        S1, S2, S3 = s1.astype(np.float64), s2.astype(np.float64), s3.astype(np.float64)
        tt = np.log2(255.0 * op.astype(np.float64))
        P1, P3 = S1 * S1, S3 * S3
        KXX, KYY, KDET = (S2 * S2 + P3) / (P1 * P3), 1 / P3, 1 / (P1 * P3)
        GROW = 2.0 ** -24 * (8 + 10 * np.sqrt(np.maximum(KXX, KYY) ** 2 / KDET))
        TE = (np.minimum(tt, 8) + 1e-5) / (1 - GROW)
        ex = _half_up((np.sqrt(TE * KXX) + 0.01) * (1 + 1e-6))
        ey = _half_up((np.sqrt(TE * KYY) + 0.01) * (1 + 1e-6))
        never = ~(tt > -1e-5)
        ex[~(GROW < 0.5)] = np.inf
        ey[~(GROW < 0.5)] = np.inf
        # the float32 test
        pert = lambda: (1 + rng.uniform(-4e-7, 4e-7, n)).astype(f32)
        a, b, p3 = s1 * s1, s1 * s2, s3 * s3
        c = s2 * s2 + p3
        ra, rc = (f32(1) / a * pert()).astype(f32), (f32(1) / c * pert()).astype(f32)
        t = np.minimum(ex * ex * a * p3 * rc, ey * ey * p3)
        te = np.where((ex < np.inf) & (ey < np.inf) & (t == t), t * f32(1 + 1e-4) + f32(1e-3), f32(np.inf))
        box = (mx - ex <= x1) & (mx + ex >= x0) & (my - ey <= y1) & (my + ey >= y0) & ~never
        cx, cy = np.minimum(np.maximum(mx, x0), x1), np.minimum(np.maximum(my, y0), y1)
        dx = cx - mx
        dy = np.minimum(np.maximum(-b * dx * rc, y0 - my), y1 - my)
        t0, t1, t2 = a * dx * dx, f32(2) * b * dx * dy, c * dy * dy
        mv = (cx != mx) & (((t0 + t1) + t2 - f32(2.0 ** -16) * (t0 + np.abs(t1) + t2)) <= te)
        dy = cy - my
        dx = np.minimum(np.maximum(-b * dy * ra, x0 - mx), x1 - mx)
        t0, t1, t2 = a * dx * dx, f32(2) * b * dx * dy, c * dy * dy
        mh = (cy != my) & (((t0 + t1) + t2 - f32(2.0 ** -16) * (t0 + np.abs(t1) + t2)) <= te)
        keep = box & (~(te < np.inf) | ((cx == mx) & (cy == my)) | mv | mh)
    passes_total = 0
    for k in range(8):
        for l in range(8):
            ddx = ((x0 + f32(k)) - mx).astype(f32)
            ddy = ((y0 + f32(l)) - my).astype(f32)
            u = _fma32(s1, ddx, (s2 * ddy).astype(f32))
            w = (s3 * ddy).astype(f32)
            S = _fma32(u, u, (w * w).astype(f32))
            alpha = np.minimum(op.astype(np.float64) * np.exp2(-S.astype(np.float64)), 0.99)
            passes = (S <= 8) & (alpha >= (1 - 1e-6) / 255)
            passes_total += int(passes.sum())
            assert not np.any(passes & ~keep), np.flatnonzero(passes & ~keep)[:5]
    assert passes_total > 100_000
    # and the test does skip: most box hits of these random ellipses are dropped
    assert keep.sum() < 0.7 * box.sum()
