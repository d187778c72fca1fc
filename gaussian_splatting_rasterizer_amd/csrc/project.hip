// project.hip -- per-(Gaussian, view) preprocess on gfx950.
//
// One thread per Gaussian reads its parameters once (SH coefficients in
// registers, the degree is a template parameter so nothing is indexed
// dynamically) and loops over the views, writing per (view, Gaussian) a 48-byte
// record, its tile rectangle, the depth sort key and the tile count with
// coalesced stores.
//
// Math: EWA splatting of the 3D covariance R(q) S S^T R(q)^T through the
// view rotation and the perspective Jacobian (lateral offset clamped to 1.3x the
// field of view), plus a 0.3 px^2 dilation, all in float64 from the float32
// inputs; the radius is 3 sqrt(lambda_max) rounded up (eigenvalue gap floored
// at 0.1) in float32 from the rounded covariance; the exponent is kept as the
// Cholesky factor of log2(e)/2 times the inverse covariance and the centre as a
// float32 pair, so that the float32 evaluation per pixel keeps its precision
// for elongated footprints and far from the image origin; colour is the SH
// expansion along the unit direction from the camera centre, +0.5, clamped
// below at 0 with the clamp state kept.  The 2D Gaussian kernel and the SH
// colour are those of the Exact Score Operators of the Renderer Score Tokens
// proposal; the rest is the standard 3DGS preprocess that Stage 1 ("original
// gsplat tile binning") refers to.  Operation order and rounding are fixed
// (see gsr_device.hpp).
#include "gsr_internal.hpp"

namespace gsr {

template <int D, bool AA>
__global__ __launch_bounds__(256) void k_project(const float* __restrict__ means, const float* __restrict__ quats,
                                                  const float* __restrict__ scales, const float* __restrict__ opac,
                                                  const float* __restrict__ sh, int64_t G, int V, CamPack cams,
                                                  int W, int H, int TX, int TY, float near_plane, float far_plane,
                                                  float4* __restrict__ rec0, float4* __restrict__ rec1,
                                                  float4* __restrict__ rec2, uint2* __restrict__ rect,
                                                  uint32_t* __restrict__ depth_key,
                                                  uint32_t* __restrict__ tiles_touched,
                                                  uint32_t* __restrict__ pay_init) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= G) return;

    const double mu[3] = {means[3 * g], means[3 * g + 1], means[3 * g + 2]};
    const float op = opac[g];
    float c[3 * D];
#pragma unroll
    for (int k = 0; k < 3 * D; ++k) c[k] = sh[(int64_t)3 * D * g + k];

    // view-independent part (float64): rotation of the unnormalised quaternion scaled by 2 / |q|^2,
    // M = R(q) diag(s), Sigma3 = M M^T
    const double qw = quats[4 * g], qx = quats[4 * g + 1], qy = quats[4 * g + 2], qz = quats[4 * g + 3];
    const double n2 = ((qw * qw + qx * qx) + qy * qy) + qz * qz;
    bool ok_g = (n2 > 0.0) && (n2 <= 1.7976931348623157e308) && (op >= 0.0f) && (op <= 1.0f);
    double S3[9];
    {
        const double q2 = 2.0 / n2;
        double Rq[9];
        Rq[0] = 1.0 - q2 * (qy * qy + qz * qz);
        Rq[1] = q2 * (qx * qy - qw * qz);
        Rq[2] = q2 * (qx * qz + qw * qy);
        Rq[3] = q2 * (qx * qy + qw * qz);
        Rq[4] = 1.0 - q2 * (qx * qx + qz * qz);
        Rq[5] = q2 * (qy * qz - qw * qx);
        Rq[6] = q2 * (qx * qz - qw * qy);
        Rq[7] = q2 * (qy * qz + qw * qx);
        Rq[8] = 1.0 - q2 * (qx * qx + qy * qy);
        const double s0 = scales[3 * g], s1 = scales[3 * g + 1], s2 = scales[3 * g + 2];
        double M[9];
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            M[3 * i] = Rq[3 * i] * s0;
            M[3 * i + 1] = Rq[3 * i + 1] * s1;
            M[3 * i + 2] = Rq[3 * i + 2] * s2;
        }
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j)
                S3[3 * i + j] = (M[3 * i] * M[3 * j] + M[3 * i + 1] * M[3 * j + 1]) + M[3 * i + 2] * M[3 * j + 2];
    }

    for (int v = 0; v < V; ++v) {
        const float* cam = cams.c[v];
        const int64_t rid = (int64_t)v * G + g;
        const double R[9] = {cam[0], cam[1], cam[2], cam[3], cam[4], cam[5], cam[6], cam[7], cam[8]};
        const float fx = cam[12], fy = cam[13], cx = cam[14], cy = cam[15];
        double t[3];
        camera_centre_f64(cam, mu, t);
        const double tx = t[0], ty = t[1], tz = t[2];
        bool ok = ok_g && (tz >= (double)near_plane) && (tz <= (double)far_plane);

        // camera-frame covariance Rv Sigma3 Rv^T
        double Tm[9], Cc[9];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j)
                Tm[3 * i + j] = (R[3 * i] * S3[j] + R[3 * i + 1] * S3[3 + j]) + R[3 * i + 2] * S3[6 + j];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j)
                Cc[3 * i + j] = (Tm[3 * i] * R[3 * j] + Tm[3 * i + 1] * R[3 * j + 1]) + Tm[3 * i + 2] * R[3 * j + 2];

        // perspective Jacobian at the centre clamped to kFovClamp x the half field of view
        const double limx = cams.lim[v][0], limy = cams.lim[v][1];
        const int clip = fov_clip_bits(t, cams.lim[v]);
        const double iz = 1.0 / tz;
        const double ux = tx * iz, uy = ty * iz;
        const double uxc = (clip & 1) ? (ux < 0.0 ? -limx : limx) : ux;
        const double uyc = (clip & 2) ? (uy < 0.0 ? -limy : limy) : uy;
        const double j00 = (double)fx * iz, j02 = -((double)fx * uxc) * iz;
        const double j11 = (double)fy * iz, j12 = -((double)fy * uyc) * iz;
        const double u00 = j00 * Cc[0] + j02 * Cc[6];
        const double u01 = j00 * Cc[1] + j02 * Cc[7];
        const double u02 = j00 * Cc[2] + j02 * Cc[8];
        const double u11 = j11 * Cc[4] + j12 * Cc[7];
        const double u12 = j11 * Cc[5] + j12 * Cc[8];
        const double ar = u00 * j00 + u02 * j02, cr = u11 * j11 + u12 * j12;
        const double a = ar + kDilation;
        const double b = u01 * j11 + u02 * j12;
        const double cq = cr + kDilation;
        const double det = a * cq - b * b;
        const double kDblMax = 1.7976931348623157e308;
        ok = ok && (det > 0.0) && (det <= kDblMax) && (a <= kDblMax) && (cq <= kDblMax);
        const float a32 = (float)a, b32 = (float)b, c32 = (float)cq, d32 = (float)det;
        ok = ok && (d32 > 0.0f) && (d32 <= 3.40282347e+38f) && (a32 <= 3.40282347e+38f) && (c32 <= 3.40282347e+38f);
        // antialiased mode: opacity scaled by sqrt(det of the undilated covariance / det)
        float opx = op;
        if (AA) {
            const double det_r = ar * cr - b * b;
            opx = op * (det_r > 0.0 ? __builtin_sqrtf((float)(det_r / det)) : 0.0f);
        }
        // 3-sigma radius (float32)
        const float mid = 0.5f * (a32 + c32);
        const float disc = mid * mid - d32;
        const float lam = mid + __builtin_sqrtf(disc > kEigFloor ? disc : kEigFloor);
        const float rad = __builtin_ceilf(3.0f * __builtin_sqrtf(lam));
        // projected centre in float64, kept as the float32 pair hi + lo
        const double mx = (double)fx * ux + (double)cx;
        const double my = (double)fy * uy + (double)cy;
        const float hx = (float)mx, hy = (float)my;
        const float lx = (float)(mx - (double)hx), ly = (float)(my - (double)hy);

        const float fx0 = (hx - rad) * 0.0625f, fx1 = ((hx + rad) + 15.0f) * 0.0625f;
        const float fy0 = (hy - rad) * 0.0625f, fy1 = ((hy + rad) + 15.0f) * 0.0625f;
        auto clamp_tile = [](float f, int n) -> int {
            return !(f > 0.0f) ? 0 : (f >= (float)n ? n : (int)f);
        };
        int x0 = clamp_tile(fx0, TX), x1 = clamp_tile(fx1, TX);
        int y0 = clamp_tile(fy0, TY), y1 = clamp_tile(fy1, TY);
        ok = ok && (x1 > x0) && (y1 > y0);

        if (!ok) {
            rec0[rid] = make_float4(0.f, 0.f, 0.f, 0.f);
            rec1[rid] = make_float4(0.f, 0.f, 0.f, 0.f);
            rec2[rid] = make_float4(0.f, 0.f, 0.f, 0.f);
            rect[rid] = make_uint2(0u, 0u);
            depth_key[rid] = 0xffffffffu;
            tiles_touched[rid] = 0u;
            if (pay_init) pay_init[rid] = pack_rect(make_uint2(0u, 0u));
            continue;
        }

        // exponent factors (float32): k Sigma2^-1 = L L^T, L = [[s1, 0], [s2, s3]]
        const float s3 = __builtin_sqrtf(kHalfLog2e / c32);
        const float s1 = __builtin_sqrtf((kHalfLog2e * c32) / d32);
        const float s2 = -((kHalfLog2e * b32) / d32) / s1;

        // colour along the direction from the camera centre -Rv^T t (float32)
        const float R0 = cam[0], R1 = cam[1], R2 = cam[2], R3 = cam[3], R4 = cam[4], R5 = cam[5];
        const float R6 = cam[6], R7 = cam[7], R8 = cam[8];
        const float t0 = cam[9], t1 = cam[10], t2 = cam[11];
        const float ccx = -((R0 * t0 + R3 * t1) + R6 * t2);
        const float ccy = -((R1 * t0 + R4 * t1) + R7 * t2);
        const float ccz = -((R2 * t0 + R5 * t1) + R8 * t2);
        const float dx = means[3 * g] - ccx, dy = means[3 * g + 1] - ccy, dz = means[3 * g + 2] - ccz;
        const float len = __builtin_sqrtf((dx * dx + dy * dy) + dz * dz);
        const float il = 1.0f / len;
        float B[D];
        sh_basis_f32(dx * il, dy * il, dz * il, D, B);
        float pre[3];
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) {
            float acc = B[0] * c[ch];
#pragma unroll
            for (int k = 1; k < D; ++k) acc = __builtin_fmaf(B[k], c[3 * k + ch], acc);
            pre[ch] = acc + 0.5f;
        }

        rec0[rid] = make_float4(hx, hy, s1, s2);
        rec1[rid] = make_float4(s3, opx, pre[0], pre[1]);
        rec2[rid] = make_float4(pre[2], __uint_as_float(entry_box_pack(s1, s2, s3, opx)), lx, ly);
        const uint2 rc = make_uint2((uint32_t)x0 | ((uint32_t)y0 << 16), (uint32_t)x1 | ((uint32_t)y1 << 16));
        rect[rid] = rc;
        depth_key[rid] = __float_as_uint((float)tz);
        tiles_touched[rid] = (uint32_t)((x1 - x0) * (y1 - y0));
        if (pay_init) pay_init[rid] = pack_rect(rc);
    }
}

hipError_t launch_project(const gs_gaussians& sc, const CamPack& cams, const Sizes& s, float near_plane,
                          float far_plane, int antialiased, uint32_t* pay_init, Workspace& ws, hipStream_t st) {
    if (s.G == 0) return hipSuccess;
    const dim3 block(256), grid((unsigned)((s.G + 255) / 256));
#define GSR_LAUNCH_PROJECT(DD, AAA)                                                                        \
    hipLaunchKernelGGL(HIP_KERNEL_NAME(k_project<DD, AAA>), grid, block, 0, st, sc.means, sc.quats, sc.scales,   \
                       sc.opacities,                                                                      \
                       sc.sh, s.G, s.V, cams, s.W, s.H, s.TX, s.TY, near_plane, far_plane, ws.rec0, ws.rec1, \
                       ws.rec2, ws.rect, ws.depth_key, ws.tiles_touched, pay_init)
#define GSR_LAUNCH_PROJECT_D(DD)                 \
    if (antialiased) GSR_LAUNCH_PROJECT(DD, true); \
    else GSR_LAUNCH_PROJECT(DD, false)
    switch (s.d) {
        case 1: GSR_LAUNCH_PROJECT_D(1); break;
        case 4: GSR_LAUNCH_PROJECT_D(4); break;
        case 9: GSR_LAUNCH_PROJECT_D(9); break;
        default: GSR_LAUNCH_PROJECT_D(16); break;
    }
#undef GSR_LAUNCH_PROJECT_D
#undef GSR_LAUNCH_PROJECT
    return hipGetLastError();
}

}  // namespace gsr
