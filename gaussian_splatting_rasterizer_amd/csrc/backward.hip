// backward.hip -- renderer backward (vector-Jacobian product of the colour
// image) on gfx950.
//
// The forward is Stage 1 of the Renderer Score Tokens proposal ("Two-Stage
// Algorithm", Standard Render) with the 3DGS primitive of the ATSplat summary
// page (EWA projection of R S S^T R^T, SH colour along the view direction,
// alpha = o G, front-to-back compositing).  Given dL/dC_hat per pixel, the
// backward returns dL/d(means, quaternions, scales, opacities, SH) with the
// float32 decisions of the render frozen (contributor sets, alpha clamp,
// colour clamp, field-of-view clamp).
//
// k_backward: the same tiles, lists, order and decisions as the render, and
// the same traversal as the score replay (event entries only; the suffix
// enters only through <g, S>, so each pixel carries that scalar, <g, C_hat - P>,
// and takes w <g, c> off it per contribution).  With g = dL/dC_hat and, for each
// contribution,
//     S = C_hat - P - T alpha c          (everything composited behind it, background included)
//     dL/dalpha = T <g, c> - <g, S> / (1 - alpha)
//     u = alpha dL/dalpha                (0 where the alpha clamp is active)
// the nine per-pixel partials are
//     U = u, U_x = u dx, U_y = u dy, U_xx = u dx^2, U_xy = u dx dy, U_yy = u dy^2,
//     V_c = T alpha g_c (c = r, g, b),    (dx, dy) = p - mu2D.
// As alpha = o G with G = exp(-(ca dx^2 + 2 cb dx dy + cc dy^2) / 2), the
// per-(Gaussian, view) sums give
//     dL/do = U / o,   dL/dmu2D = conic (U_x, U_y),   dL/d(ca, cb, cc) = -(U_xx / 2, U_xy, U_yy / 2),
//     dL/dcolour = V (where the colour clamp is inactive).
// The wave reduces the nine values (reduce-scatter of eight plus one full
// sum), the four waves meet in LDS and one 48-byte partial per event entry is
// stored with plain stores at the pair's slot; the slot's bit is set in
// slot_bits.  The slot gather then sums each record's partials.  Every listed
// entry has a contribution or a saturation in some lane of the wave and a
// wave's list ends at its last one, so the walk tests for neither.
//
// k_grads: after the slot gather (per record, the sums of its flagged slots),
// one thread per Gaussian loops over the views in float64: projected centre ->
// camera-space centre; conic -> dilated 2D covariance -> (perspective Jacobian
// at the clamped centre, camera covariance R Sigma R^T) -> world covariance;
// SH colour -> coefficients and, through the basis, the view direction ->
// centre.  The world-covariance gradient is summed over the views and pulled
// back once through M M^T, M = R_q diag(s), to the scales and the unit
// quaternion, then to the input quaternion.  The per-Gaussian work (R_q, M,
// M M^T) is shared by all views, which is why the views are a loop and not
// threads: the kernel is bound by float64 issue, so work per view is what
// counts.  The SH part runs as a second pass over the views (re-reading its
// three sums and the view direction), so that its 3 d accumulators are not
// live during the covariance chain (204 instead of 256+ registers).  Its
// arithmetic is value arithmetic only and is contracted to fused
// multiply-adds.
#include "gsr_internal.hpp"

namespace gsr {

// Entries staged per batch: 96 keeps the block's LDS near 25 KB (six blocks per CU).
constexpr int kBwdBatch = 96;

__global__ __launch_bounds__(256) void k_backward(const uint2* __restrict__ ranges,
                                                  const uint32_t* __restrict__ sorted_g,
                                                  const uint32_t* __restrict__ slot_base,
                                                  const float4* __restrict__ rec0, const float4* __restrict__ rec1,
                                                  const float4* __restrict__ rec2, const uint2* __restrict__ rect,
                                                  int64_t G, int T, int TX, int W, int H,
                                                  const float4* __restrict__ pixel,
                                                  const float* __restrict__ grad_color,
                                                  const uint8_t* __restrict__ events, float4* __restrict__ partials,
                                                  uint32_t* __restrict__ slot_bits,
                                                  const uint32_t* __restrict__ tile_order,
                                                  const uint32_t* __restrict__ tile_work) {
    // an entry's three staged vectors sit at the same byte offset of three arrays, so one offset (16 j,
    // kept in the wave's list) addresses all of them
    __shared__ float4 s0[kBwdBatch];  // {tile-relative centre (2), s1, s2}
    __shared__ float4 s1[kBwdBatch];  // {s3, opacity, colour r, colour g}
    __shared__ float4 s2[kBwdBatch];  // {colour b, unused}
    __shared__ uint8_t s_evb[kBwdBatch];    // event bits of each staged entry (bit w: wave w)
    __shared__ uint32_t s_slot[kBwdBatch];  // partial slot of each staged pair
    __shared__ uint8_t s_mask[kBwdBatch];   // colour clamp mask bits (pre-clamp colour finite and >= 0), r g b
    __shared__ uint32_t slist[4][kBwdBatch];
    __shared__ __align__(16) float sp[4][kBwdBatch][12];

    const int tile = (int)tile_order[blockIdx.x];
    const int v = tile / T;
    const int t = tile - v * T;
    const int ty = t / TX, tx = t - ty * TX;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int qx = tx * kTile + (wave & 1) * 8, qy = ty * kTile + (wave >> 1) * 8;
    const int pxi = qx + (lane & 7);
    const int pyi = qy + (lane >> 3);
    const bool inside = pxi < W && pyi < H;
    // pixel centre relative to the tile origin (entry centres are staged tile-relative too)
    const float px = (float)(pxi - tx * kTile) + 0.5f, py = (float)(pyi - ty * kTile) + 0.5f;
    const uint2 rg = ranges[tile];
    const int64_t vG = (int64_t)v * G;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    float Ch0 = 0.f, Ch1 = 0.f, Ch2 = 0.f, g0 = 0.f, g1 = 0.f, g2 = 0.f;
    if (inside) {
        const int64_t pix = ((int64_t)v * H + pyi) * W + pxi;
        const float4 c = pixel[pix];
        Ch0 = c.x;
        Ch1 = c.y;
        Ch2 = c.z;
        g0 = grad_color[3 * pix];
        g1 = grad_color[3 * pix + 1];
        g2 = grad_color[3 * pix + 2];
    }
    float Tr = 1.0f;
    // <g, S> with S the suffix composite times the transmittance in front of it (C_hat minus the prefix colour)
    float qg = __builtin_fmaf(g2, Ch2, __builtin_fmaf(g1, Ch1, g0 * Ch0));
    bool done = !inside;

    // the entries the render processed (every event lies there: past them the event bytes are not this frame's,
    // and a wave whose pixels are all done would leave its partial rows unwritten for one it names); an empty
    // range ({~0u, 0}) has none
    const uint32_t rend = rg.x + min(tile_work[tile], rg.y > rg.x ? rg.y - rg.x : 0u);
    for (uint32_t base = rg.x; base < rend; base += kBwdBatch) {
        if (__syncthreads_count(!done) == 0) break;
        const uint32_t i = base + threadIdx.x;
        if (threadIdx.x < kBwdBatch && i < rend) {
            const int64_t rid = vG + sorted_g[i];
            const float4 a = rec0[rid];
            const float4 b = rec1[rid];
            const float4 c = rec2[rid];
            const uint2 rc = rect[rid];
            s0[threadIdx.x] = make_float4(tile_centre(a.x, c.z, tx), tile_centre(a.y, c.w, ty), a.z, a.w);
            s1[threadIdx.x] = make_float4(b.x, b.y, clamp_colour(b.z), clamp_colour(b.w));
            s2[threadIdx.x] = make_float4(clamp_colour(c.x), 0.0f, 0.0f, 0.0f);
            s_evb[threadIdx.x] = events[i];
            const uint32_t x0 = rc.x & 0xffffu, y0 = rc.x >> 16, wx = (rc.y & 0xffffu) - x0;
            s_slot[threadIdx.x] = slot_base[rid] + ((uint32_t)ty - y0) * wx + ((uint32_t)tx - x0);
            s_mask[threadIdx.x] = (uint8_t)((colour_ok(b.z) ? 1u : 0u) | (colour_ok(b.w) ? 2u : 0u) | (colour_ok(c.x) ? 4u : 0u));
        }
        const int cnt = (int)min((uint32_t)kBwdBatch, rend - base);
        // (a wave writes the partial row of every entry it walks; the flush reads only those rows)
        __syncthreads();
        if (__ballot(!done) != 0ull) {
            int nw = 0;
            for (int c = 0; c < cnt; c += 64) {
                const int j = c + lane;
                const bool hit = j < cnt && ((s_evb[j] >> wave) & 1u);
                const uint64_t m = __ballot(hit);
                if (hit) slist[wave][nw + __popcll(m & lt_mask)] = (uint32_t)(j * sizeof(float4));
                nw += __popcll(m);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // one entry: the float32 decisions and the state updates of every lane, and the nine values whose
            // wave sums are the entry's partial row
            auto step = [&](uint32_t off, float (&x)[8], float& x8) {
                const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(s0) + off);
                const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(s1) + off);
                const float cbl = reinterpret_cast<const float4*>(reinterpret_cast<const char*>(s2) + off)->x;
                const float dx = px - a.x, dy = py - a.y;
                const float S = quad_S(a.z, a.w, b.x, dx, dy);
                const bool near = !done && S <= kSCutoff;
                const float aG = b.y * exp2_spec(-S);
                const bool clamped = !(aG < kAlphaMax);
                const float alpha = clamped ? kAlphaMax : aG;
                const bool pass = near && alpha >= kAlphaMin;
                const float tT = Tr * (1.0f - alpha);
                const bool sat = pass && tT < kTMin;
                const bool contrib = pass != sat;  // (sat implies pass: a mask difference, no second compare)
                done = done || sat;
                // every listed entry has a contribution or saturation in some lane of the wave
                const float cr = b.z, cg = b.w;
                const float w = contrib ? alpha * Tr : 0.0f;
                const float gc = __builtin_fmaf(g2, cbl, __builtin_fmaf(g1, cg, g0 * cr));
                // <g, S> behind this entry: the prefix now includes it (lanes without a contribution subtract 0)
                qg = __builtin_fmaf(-w, gc, qg);
                const float gS = qg;
                // u = alpha (T <g, c> - <g, S> / (1 - alpha)) = w <g, c> - alpha <g, S> / (1 - alpha)
                const float u = (contrib && !clamped)
                                    ? __builtin_fmaf(-alpha * gS, __builtin_amdgcn_rcpf(1.0f - alpha), w * gc)
                                    : 0.0f;
                const float ux = u * dx, uy = u * dy;
                x[0] = u;
                x[1] = ux;
                x[2] = uy;
                x[3] = ux * dx;
                x[4] = ux * dy;
                x[5] = uy * dy;
                x[6] = w * g0;
                x[7] = w * g1;
                x8 = w * g2;
                Tr = contrib ? tT : Tr;
            };
            // every lane of a group of eight holds its component's sum: all store (the same value to the same
            // word); sp[wave][j] rows are 48 bytes, 3 off
            char* spw = reinterpret_cast<char*>(&sp[wave][0][0]);
            auto put = [&](uint32_t off, float red, float red8) {
                *reinterpret_cast<float*>(spw + 3 * off + 4 * (lane >> 3)) = red;
                if (lane == 0) *reinterpret_cast<float*>(spw + 3 * off + 32) = red8;
            };
            // two entries per round: the second entry's decisions follow the first's state updates, and the
            // wave reductions of the two, independent of each other, run interleaved
            int k = 0;
            for (; k + 1 < nw; k += 2) {
                const uint32_t o0 = slist[wave][k], o1 = slist[wave][k + 1];
                float x0[8], x1[8], y0, y1;
                step(o0, x0, y0);
                step(o1, x1, y1);
                const float red0 = wave_reduce8(x0, lane), red1 = wave_reduce8(x1, lane);
                const float s0v = wave_sum1(y0), s1v = wave_sum1(y1);
                put(o0, red0, s0v);
                put(o1, red1, s1v);
            }
            if (k < nw) {
                const uint32_t o0 = slist[wave][k];
                float x0[8], y0;
                step(o0, x0, y0);
                const float red0 = wave_reduce8(x0, lane);
                put(o0, red0, wave_sum1(y0));
            }
        }
        __syncthreads();
        // one 48-byte partial per entry at which some wave had an event, flagged in the slot bits
        for (int idx = threadIdx.x; idx < 3 * cnt; idx += 256) {
            const int j = idx / 3, h = idx - 3 * j;
            const uint32_t evb = s_evb[j];
            if (evb == 0) continue;
            // the rows of the waves that walked the entry (every other wave's share is zero)
            float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if (!((evb >> w) & 1u)) continue;
                const float4 q = *reinterpret_cast<const float4*>(&sp[w][j][4 * h]);
                acc.x += q.x;
                acc.y += q.y;
                acc.z += q.z;
                acc.w += q.w;
            }
            const uint32_t m = s_mask[j];
            if (h == 1) {
                acc.z = (m & 1u) ? acc.z : 0.0f;
                acc.w = (m & 2u) ? acc.w : 0.0f;
            } else if (h == 2) {  // components 9-11 of a row are never written
                acc = make_float4((m & 4u) ? acc.x : 0.0f, 0.0f, 0.0f, 0.0f);
            }
            const uint32_t slot = s_slot[j];
            partials[3 * (int64_t)slot + h] = acc;
            if (h == 0) atomicOr(&slot_bits[slot >> 5], 1u << (slot & 31u));
        }
    }
}

hipError_t launch_backward(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, const float* grad_color,
                           hipStream_t st) {
    const int64_t tiles = (int64_t)s.V * s.T;
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_backward, dim3((unsigned)tiles), dim3(256), 0, st, ws.ranges, sorted_g, ws.slot_base,
                       ws.rec0, ws.rec1, ws.rec2, ws.rect, s.G, s.T, s.TX, s.W, s.H, ws.pixel, grad_color,
                       ws.events, ws.partials, ws.slot_bits, ws.tile_order, ws.tile_work);
    return hipGetLastError();
}

constexpr int kGradThreads = 128;

template <int D>
__global__ __launch_bounds__(kGradThreads) void k_grads(const float* __restrict__ means,
                                                        const float* __restrict__ quats,
                                                        const float* __restrict__ scales,
                                                        const float* __restrict__ opac, const float* __restrict__ sh,
                                                        int64_t G, int V, int W, int H, CamPack cams,
                                                        int antialiased, const uint64_t* __restrict__ rec_masks,
                                                        const float4* __restrict__ gv_sums, gs_gaussian_grads out) {
#pragma clang fp contract(fast)
    const int64_t g = (int64_t)blockIdx.x * kGradThreads + threadIdx.x;
    if (g >= G) return;
    const double mu[3] = {means[3 * g], means[3 * g + 1], means[3 * g + 2]};
    const double qi[4] = {quats[4 * g], quats[4 * g + 1], quats[4 * g + 2], quats[4 * g + 3]};
    const double sc[3] = {scales[3 * g], scales[3 * g + 1], scales[3 * g + 2]};
    const double o = opac[g];
    const float* shg = sh + 3 * D * g;

    const double iqn = 1.0 / sqrt(qi[0] * qi[0] + qi[1] * qi[1] + qi[2] * qi[2] + qi[3] * qi[3]);
    const double qw = qi[0] * iqn, qx = qi[1] * iqn, qy = qi[2] * iqn, qz = qi[3] * iqn;
    const double Rq[9] = {1 - 2 * (qy * qy + qz * qz), 2 * (qx * qy - qw * qz), 2 * (qx * qz + qw * qy),
                          2 * (qx * qy + qw * qz), 1 - 2 * (qx * qx + qz * qz), 2 * (qy * qz - qw * qx),
                          2 * (qx * qz - qw * qy), 2 * (qy * qz + qw * qx), 1 - 2 * (qx * qx + qy * qy)};
    double M[9];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int k = 0; k < 3; ++k) M[3 * i + k] = Rq[3 * i + k] * sc[k];
    // world covariance M M^T, symmetric: s00 s01 s02 s11 s12 s22
    double S3[9];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) S3[3 * i + j] = M[3 * i] * M[3 * j] + M[3 * i + 1] * M[3 * j + 1] + M[3 * i + 2] * M[3 * j + 2];

    double gmu[3] = {0.0, 0.0, 0.0};
    double GS[9] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};  // dL/d(M M^T)
    double sumU = 0.0;
    bool any = false;

    for (int v = 0; v < V; ++v) {
        const int64_t rid = (int64_t)v * G + g;
        const uint64_t bit = 1ull << (rid & 63);
        if (!(rec_masks[2 * (rid >> 6) + 1] & bit)) continue;  // culled or never reached: no gradient
        any = true;
        const float4 p0 = gv_sums[3 * rid], p1 = gv_sums[3 * rid + 1];
        const float* cam = cams.c[v];
        double R[9];
#pragma unroll
        for (int k = 0; k < 9; ++k) R[k] = cam[k];
        const double t0 = cam[9], t1 = cam[10], t2 = cam[11];
        const double fx = cam[12], fy = cam[13];
        const double tx = R[0] * mu[0] + R[1] * mu[1] + R[2] * mu[2] + t0;
        const double ty = R[3] * mu[0] + R[4] * mu[1] + R[5] * mu[2] + t1;
        const double tz = R[6] * mu[0] + R[7] * mu[1] + R[8] * mu[2] + t2;
        const double iz = 1.0 / tz, iz2 = iz * iz;

        // camera covariance Cc = R S3 R^T
        double Tm[9], Cc[9];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j) Tm[3 * i + j] = R[3 * i] * S3[j] + R[3 * i + 1] * S3[3 + j] + R[3 * i + 2] * S3[6 + j];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = i; j < 3; ++j) {
                Cc[3 * i + j] = Tm[3 * i] * R[3 * j] + Tm[3 * i + 1] * R[3 * j + 1] + Tm[3 * i + 2] * R[3 * j + 2];
                Cc[3 * j + i] = Cc[3 * i + j];
            }

        // perspective Jacobian at the centre clamped to 1.3x the half field of view
        // the clamp state is the preprocess decision, re-taken by the same function from the same inputs
        // (its float64 operations are not contracted), so the backward differentiates the rendered branch
        double tdec[3];
        camera_centre_f64(cam, mu, tdec);
        const int clip = fov_clip_bits(tdec, cams.lim[v]);
        const bool clip_x = (clip & 1) != 0, clip_y = (clip & 2) != 0;
        const double limx = cams.lim[v][0], limy = cams.lim[v][1];
        const double ux = tx * iz, uy = ty * iz;
        const double uxc = clip_x ? (ux < 0.0 ? -limx : limx) : ux;
        const double uyc = clip_y ? (uy < 0.0 ? -limy : limy) : uy;
        const double j00 = fx * iz, j02 = -fx * uxc * iz, j11 = fy * iz, j12 = -fy * uyc * iz;
        // Jc Cc (rows 0, 1) and the dilated 2D covariance [[a, b], [b, c]]
        const double A0[3] = {j00 * Cc[0] + j02 * Cc[6], j00 * Cc[1] + j02 * Cc[7], j00 * Cc[2] + j02 * Cc[8]};
        const double A1[3] = {j11 * Cc[3] + j12 * Cc[6], j11 * Cc[4] + j12 * Cc[7], j11 * Cc[5] + j12 * Cc[8]};
        const double ar = A0[0] * j00 + A0[2] * j02, cr = A1[1] * j11 + A1[2] * j12;  // undilated
        const double a = ar + 0.3;
        const double b = A0[1] * j11 + A0[2] * j12;
        const double c = cr + 0.3;
        const double det = a * c - b * b, idet = 1.0 / det;
        const double ca = c * idet, cb = -b * idet, cc = a * idet;

        // image-space gradients of this (Gaussian, view)
        const double U = p0.x, Ux = p0.y, Uy = p0.z, Uxx = p0.w, Uxy = p1.x, Uyy = p1.y;
        sumU += U;
        const double gmx = ca * Ux + cb * Uy, gmy = cb * Ux + cc * Uy;
        const double gca = -0.5 * Uxx, gcb = -Uxy, gcc = -0.5 * Uyy;
        // conic (c, -b, a) / det -> (a, b, c)
        const double id2 = idet * idet;
        double ga = (-c * c * gca + b * c * gcb - b * b * gcc) * id2;
        double gb = (2.0 * b * c * gca - (a * c + b * b) * gcb + 2.0 * a * b * gcc) * id2;
        double gc = (-b * b * gca + a * b * gcb - a * a * gcc) * id2;
        if (antialiased) {
            // alpha = o comp G with comp = sqrt(det_r / det): U d log comp, d log comp = (d log det_r - d log det) / 2
            const double detr = ar * cr - b * b;
            if (detr > 0.0) {
                const double idr = 1.0 / detr;
                ga += U * (0.5 * cr * idr - 0.5 * c * idet);
                gb += U * (b * idet - b * idr);
                gc += U * (0.5 * ar * idr - 0.5 * a * idet);
            }
        }
        const double g00 = ga, g01 = 0.5 * gb, g11 = gc;  // dL/dS2, S2 = Jc Cc Jc^T
        // dL/dCc = Jc^T G2 Jc
        const double GC00 = j00 * j00 * g00, GC01 = j00 * j11 * g01, GC02 = j00 * (g00 * j02 + g01 * j12);
        const double GC11 = j11 * j11 * g11, GC12 = j11 * (g01 * j02 + g11 * j12);
        const double GC22 = j02 * j02 * g00 + 2.0 * j02 * j12 * g01 + j12 * j12 * g11;
        const double GC[9] = {GC00, GC01, GC02, GC01, GC11, GC12, GC02, GC12, GC22};
        // dL/dS3 += R^T GC R
        double X[9];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j) X[3 * i + j] = GC[3 * i] * R[j] + GC[3 * i + 1] * R[3 + j] + GC[3 * i + 2] * R[6 + j];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j) GS[3 * i + j] += R[i] * X[j] + R[3 + i] * X[3 + j] + R[6 + i] * X[6 + j];
        // dL/dJc = 2 G2 (Jc Cc), entries (0,0), (0,2), (1,1), (1,2)
        const double GJ00 = 2.0 * (g00 * A0[0] + g01 * A1[0]);
        const double GJ02 = 2.0 * (g00 * A0[2] + g01 * A1[2]);
        const double GJ11 = 2.0 * (g01 * A0[1] + g11 * A1[1]);
        const double GJ12 = 2.0 * (g01 * A0[2] + g11 * A1[2]);
        // camera-space centre: projected centre (unclamped) and Jacobian (clamped)
        double gtx = gmx * fx * iz, gty = gmy * fy * iz;
        double gtz = -(gmx * fx * tx + gmy * fy * ty) * iz2 - (GJ00 * fx + GJ11 * fy) * iz2;
        if (clip_x) {
            gtz += GJ02 * fx * uxc * iz2;
        } else {
            gtx -= GJ02 * fx * iz2;
            gtz += 2.0 * GJ02 * fx * tx * iz2 * iz;
        }
        if (clip_y) {
            gtz += GJ12 * fy * uyc * iz2;
        } else {
            gty -= GJ12 * fy * iz2;
            gtz += 2.0 * GJ12 * fy * ty * iz2 * iz;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) gmu[j] += R[j] * gtx + R[3 + j] * gty + R[6 + j] * gtz;

    }

    double gs_[3] = {0.0, 0.0, 0.0}, gq[4] = {0.0, 0.0, 0.0, 0.0};
    double go = 0.0;
    if (any) {
        go = o > 0.0 ? sumU / o : 0.0;
        // S3 = M M^T: dL/dM = (GS + GS^T) M;  M = Rq diag(s)
        double GR[9];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const double gm = (GS[3 * i] + GS[i]) * M[k] + (GS[3 * i + 1] + GS[3 + i]) * M[3 + k] +
                                  (GS[3 * i + 2] + GS[6 + i]) * M[6 + k];
                gs_[k] += gm * Rq[3 * i + k];
                GR[3 * i + k] = gm * sc[k];
            }
        // Rq of the unit quaternion (w, x, y, z)
        const double hw = 2.0 * (-qz * GR[1] + qy * GR[2] + qz * GR[3] - qx * GR[5] - qy * GR[6] + qx * GR[7]);
        const double hx = 2.0 * (qy * GR[1] + qz * GR[2] + qy * GR[3] - 2.0 * qx * GR[4] - qw * GR[5] + qz * GR[6] +
                                 qw * GR[7] - 2.0 * qx * GR[8]);
        const double hy = 2.0 * (-2.0 * qy * GR[0] + qx * GR[1] + qw * GR[2] + qx * GR[3] + qz * GR[5] - qw * GR[6] +
                                 qz * GR[7] - 2.0 * qy * GR[8]);
        const double hz = 2.0 * (-2.0 * qz * GR[0] - qw * GR[1] + qx * GR[2] + qw * GR[3] - 2.0 * qz * GR[4] +
                                 qy * GR[5] + qx * GR[6] + qy * GR[7]);
        // q / |q|
        const double dot = qw * hw + qx * hx + qy * hy + qz * hz;
        gq[0] = (hw - qw * dot) * iqn;
        gq[1] = (hx - qx * dot) * iqn;
        gq[2] = (hy - qy * dot) * iqn;
        gq[3] = (hz - qz * dot) * iqn;
    }
    // second pass over the views: SH colour along the view direction (colour clamp already
    // applied to the sums) -> coefficients, and the view-direction term of the centre
    float gsh[3 * D];
#pragma unroll
    for (int k = 0; k < 3 * D; ++k) gsh[k] = 0.0f;
    if (any) {
        for (int v = 0; v < V; ++v) {
            const int64_t rid = (int64_t)v * G + g;
            if (!((rec_masks[2 * (rid >> 6) + 1] >> (rid & 63)) & 1ull)) continue;
            const float4 p1 = gv_sums[3 * rid + 1], p2 = gv_sums[3 * rid + 2];
            const float* cam = cams.c[v];
            const double R0 = cam[0], R1 = cam[1], R2 = cam[2], R3 = cam[3], R4 = cam[4], R5 = cam[5];
            const double R6 = cam[6], R7 = cam[7], R8 = cam[8];
            const double t0 = cam[9], t1 = cam[10], t2 = cam[11];
            const double ccx = -(R0 * t0 + R3 * t1 + R6 * t2);
            const double ccy = -(R1 * t0 + R4 * t1 + R7 * t2);
            const double ccz = -(R2 * t0 + R5 * t1 + R8 * t2);
            const double dvx = mu[0] - ccx, dvy = mu[1] - ccy, dvz = mu[2] - ccz;
            const double len = sqrt(dvx * dvx + dvy * dvy + dvz * dvz), il = 1.0 / len;
            const double dirx = dvx * il, diry = dvy * il, dirz = dvz * il;
            const float gp0 = p1.z, gp1 = p1.w, gp2 = p2.x;
            float B[D], dB[3 * D];
            sh_basis_f32((float)dirx, (float)diry, (float)dirz, D, B);
            sh_basis_grad_f32((float)dirx, (float)diry, (float)dirz, D, dB);
            float gd0 = 0.f, gd1 = 0.f, gd2 = 0.f;
#pragma unroll
            for (int k = 0; k < D; ++k) {
                gsh[3 * k] += B[k] * gp0;
                gsh[3 * k + 1] += B[k] * gp1;
                gsh[3 * k + 2] += B[k] * gp2;
                // a masked (clamped) channel has a zero colour gradient and no direction term, also when
                // its coefficients are not finite
                const float gB = (gp0 != 0.0f ? shg[3 * k] * gp0 : 0.0f) + (gp1 != 0.0f ? shg[3 * k + 1] * gp1 : 0.0f) +
                                 (gp2 != 0.0f ? shg[3 * k + 2] * gp2 : 0.0f);
                gd0 += gB * dB[3 * k];
                gd1 += gB * dB[3 * k + 1];
                gd2 += gB * dB[3 * k + 2];
            }
            const double dd = (double)gd0 * dirx + (double)gd1 * diry + (double)gd2 * dirz;
            gmu[0] += ((double)gd0 - dirx * dd) * il;
            gmu[1] += ((double)gd1 - diry * dd) * il;
            gmu[2] += ((double)gd2 - dirz * dd) * il;
        }
    }
    if (out.means) {
        out.means[3 * g] = (float)gmu[0];
        out.means[3 * g + 1] = (float)gmu[1];
        out.means[3 * g + 2] = (float)gmu[2];
    }
    if (out.quats) {
#pragma unroll
        for (int i = 0; i < 4; ++i) out.quats[4 * g + i] = (float)gq[i];
    }
    if (out.scales) {
#pragma unroll
        for (int i = 0; i < 3; ++i) out.scales[3 * g + i] = (float)gs_[i];
    }
    if (out.opacities) out.opacities[g] = (float)go;
    if (out.sh) {
#pragma unroll
        for (int k = 0; k < 3 * D; ++k) out.sh[3 * D * g + k] = gsh[k];
    }
}

hipError_t launch_backward_finalize(const gs_gaussians& sc, const CamPack& cams, const Sizes& s, const Workspace& ws,
                                    int antialiased, const gs_gaussian_grads& out, hipStream_t st) {
    if (s.G == 0) return hipSuccess;
    const dim3 block(kGradThreads), grid((unsigned)((s.G + kGradThreads - 1) / kGradThreads));
#define GSR_LAUNCH_GRADS(DD)                                                                                   \
    hipLaunchKernelGGL(k_grads<DD>, grid, block, 0, st, sc.means, sc.quats, sc.scales, sc.opacities, sc.sh, s.G, \
                       s.V, s.W, s.H, cams, antialiased, ws.rec_masks, ws.gv_sums, out)
    switch (s.d) {
        case 1: GSR_LAUNCH_GRADS(1); break;
        case 4: GSR_LAUNCH_GRADS(4); break;
        case 9: GSR_LAUNCH_GRADS(9); break;
        default: GSR_LAUNCH_GRADS(16); break;
    }
#undef GSR_LAUNCH_GRADS
    return hipGetLastError();
}

}  // namespace gsr
