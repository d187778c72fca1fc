// project.hip -- per-(Gaussian, view) preprocess on gfx950.
//
// One thread per Gaussian reads its parameters once (SH coefficients in
// registers, the degree is a template parameter so nothing is indexed
// dynamically) and loops over the views, writing per (view, Gaussian) a 40-byte
// record, its tile rectangle, the depth sort key and the tile count with
// coalesced stores.
//
// Math: EWA splatting of the 3D covariance R(q) S S^T R(q)^T through the
// view rotation and the perspective Jacobian (lateral offset clamped to 1.3x the
// field of view), plus a 0.3 px^2 dilation; the conic is the inverse 2D
// covariance; the radius is 3 sqrt(lambda_max) rounded up (eigenvalue gap
// floored at 0.1); colour is the SH expansion along the unit direction from the
// camera centre, +0.5, clamped below at 0 with the clamp state kept.  The 2D
// Gaussian kernel and the SH colour are those of the Exact Score Operators of
// the Renderer Score Tokens proposal; the rest is the standard 3DGS preprocess
// that Stage 1 ("original gsplat tile binning") refers to.  Operation order
// and rounding are fixed (see gsr_device.hpp).
#include "gsr_internal.hpp"

namespace gsr {

template <int D, bool AA>
__global__ __launch_bounds__(256) void k_project(const float* __restrict__ means, const float* __restrict__ quats,
                                                  const float* __restrict__ scales, const float* __restrict__ opac,
                                                  const float* __restrict__ sh, int64_t G, int V, CamPack cams,
                                                  int W, int H, int TX, int TY, float near_plane, float far_plane,
                                                  float4* __restrict__ rec0, float4* __restrict__ rec1,
                                                  float2* __restrict__ rec2, uint2* __restrict__ rect,
                                                  uint32_t* __restrict__ depth_key,
                                                  uint32_t* __restrict__ tiles_touched,
                                                  uint32_t* __restrict__ pay_init) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= G) return;

    const float mu0 = means[3 * g], mu1 = means[3 * g + 1], mu2 = means[3 * g + 2];
    const float op = opac[g];
    float c[3 * D];
#pragma unroll
    for (int k = 0; k < 3 * D; ++k) c[k] = sh[(int64_t)3 * D * g + k];

    // view-independent part: normalised quaternion, rotation, 3D covariance
    const float q0 = quats[4 * g], q1 = quats[4 * g + 1], q2 = quats[4 * g + 2], q3 = quats[4 * g + 3];
    const float n2 = ((q0 * q0 + q1 * q1) + q2 * q2) + q3 * q3;
    bool ok_g = (n2 > 0.0f) && (n2 <= 3.40282347e+38f) && (op >= 0.0f) && (op <= 1.0f);
    float S3[9];
    {
        const float inv = 1.0f / __builtin_sqrtf(n2);
        const float w = q0 * inv, x = q1 * inv, y = q2 * inv, z = q3 * inv;
        float Rq[9];
        Rq[0] = 1.0f - 2.0f * (y * y + z * z);
        Rq[1] = 2.0f * (x * y - w * z);
        Rq[2] = 2.0f * (x * z + w * y);
        Rq[3] = 2.0f * (x * y + w * z);
        Rq[4] = 1.0f - 2.0f * (x * x + z * z);
        Rq[5] = 2.0f * (y * z - w * x);
        Rq[6] = 2.0f * (x * z - w * y);
        Rq[7] = 2.0f * (y * z + w * x);
        Rq[8] = 1.0f - 2.0f * (x * x + y * y);
        const float s0 = scales[3 * g], s1 = scales[3 * g + 1], s2 = scales[3 * g + 2];
        float M[9];
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
                S3[3 * i + j] = __builtin_fmaf(M[3 * i + 2], M[3 * j + 2],
                                               __builtin_fmaf(M[3 * i + 1], M[3 * j + 1], M[3 * i] * M[3 * j]));
    }

    for (int v = 0; v < V; ++v) {
        const float* cam = cams.c[v];
        const int64_t rid = (int64_t)v * G + g;
        const float R0 = cam[0], R1 = cam[1], R2 = cam[2], R3 = cam[3], R4 = cam[4], R5 = cam[5];
        const float R6 = cam[6], R7 = cam[7], R8 = cam[8];
        const float t0 = cam[9], t1 = cam[10], t2 = cam[11];
        const float fx = cam[12], fy = cam[13], cx = cam[14], cy = cam[15];

        // three-term dot products as fused multiply-add chains: fma(a2, b2, fma(a1, b1, a0 b0))
        const float tx = __builtin_fmaf(R2, mu2, __builtin_fmaf(R1, mu1, R0 * mu0)) + t0;
        const float ty = __builtin_fmaf(R5, mu2, __builtin_fmaf(R4, mu1, R3 * mu0)) + t1;
        const float tz = __builtin_fmaf(R8, mu2, __builtin_fmaf(R7, mu1, R6 * mu0)) + t2;
        bool ok = ok_g && (tz >= near_plane) && (tz <= far_plane);

        // camera-frame covariance Rv S3 Rv^T
        const float Rv[9] = {R0, R1, R2, R3, R4, R5, R6, R7, R8};
        float Tm[9], Cc[9];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j)
                Tm[3 * i + j] = __builtin_fmaf(Rv[3 * i + 2], S3[6 + j],
                                               __builtin_fmaf(Rv[3 * i + 1], S3[3 + j], Rv[3 * i] * S3[j]));
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j)
                Cc[3 * i + j] = __builtin_fmaf(Tm[3 * i + 2], Rv[3 * j + 2],
                                               __builtin_fmaf(Tm[3 * i + 1], Rv[3 * j + 1], Tm[3 * i] * Rv[3 * j]));

        const float limx = cams.lim[v][0], limy = cams.lim[v][1];  // kFovClamp ((W / 2) / fx), likewise y
        const float ux = tx / tz, uy = ty / tz;
        const float uxc = ux < -limx ? -limx : (ux > limx ? limx : ux);
        const float uyc = uy < -limy ? -limy : (uy > limy ? limy : uy);
        const float txc = uxc * tz, tyc = uyc * tz;
        const float tz2 = tz * tz;
        const float j00 = fx / tz, j02 = -(fx * txc) / tz2;
        const float j11 = fy / tz, j12 = -(fy * tyc) / tz2;
        const float u00 = j00 * Cc[0] + j02 * Cc[6];
        const float u01 = j00 * Cc[1] + j02 * Cc[7];
        const float u02 = j00 * Cc[2] + j02 * Cc[8];
        const float u11 = j11 * Cc[4] + j12 * Cc[7];
        const float u12 = j11 * Cc[5] + j12 * Cc[8];
        const float a = (u00 * j00 + u02 * j02) + kDilation;
        const float b = u01 * j11 + u02 * j12;
        const float cq = (u11 * j11 + u12 * j12) + kDilation;
        const float det = a * cq - b * b;
        ok = ok && (det > 0.0f);
        // antialiased mode: opacity scaled by sqrt(det of the undilated covariance / det)
        float opx = op;
        if (AA) {
            const float a_r = u00 * j00 + u02 * j02;
            const float c_r = u11 * j11 + u12 * j12;
            const float det_r = a_r * c_r - b * b;
            opx = op * (det_r > 0.0f ? __builtin_sqrtf(det_r / det) : 0.0f);
        }
        const float idet = 1.0f / det;
        const float ca = cq * idet, cb = -b * idet, cc = a * idet;
        const float mid = 0.5f * (a + cq);
        const float disc = mid * mid - det;
        const float lam = mid + __builtin_sqrtf(disc > kEigFloor ? disc : kEigFloor);
        const float rad = __builtin_ceilf(3.0f * __builtin_sqrtf(lam));
        const float mx = fx * (tx / tz) + cx;
        const float my = fy * (ty / tz) + cy;

        const float fx0 = (mx - rad) * 0.0625f, fx1 = ((mx + rad) + 15.0f) * 0.0625f;
        const float fy0 = (my - rad) * 0.0625f, fy1 = ((my + rad) + 15.0f) * 0.0625f;
        auto clamp_tile = [](float f, int n) -> int {
            return !(f > 0.0f) ? 0 : (f >= (float)n ? n : (int)f);
        };
        int x0 = clamp_tile(fx0, TX), x1 = clamp_tile(fx1, TX);
        int y0 = clamp_tile(fy0, TY), y1 = clamp_tile(fy1, TY);
        ok = ok && (x1 > x0) && (y1 > y0);

        if (!ok) {
            rec0[rid] = make_float4(0.f, 0.f, 0.f, 0.f);
            rec1[rid] = make_float4(0.f, 0.f, 0.f, 0.f);
            rec2[rid] = make_float2(0.f, 0.f);
            rect[rid] = make_uint2(0u, 0u);
            depth_key[rid] = 0xffffffffu;
            tiles_touched[rid] = 0u;
            if (pay_init) pay_init[rid] = pack_rect(make_uint2(0u, 0u));
            continue;
        }

        // colour along the direction from the camera centre -Rv^T t
        const float ccx = -((R0 * t0 + R3 * t1) + R6 * t2);
        const float ccy = -((R1 * t0 + R4 * t1) + R7 * t2);
        const float ccz = -((R2 * t0 + R5 * t1) + R8 * t2);
        const float dx = mu0 - ccx, dy = mu1 - ccy, dz = mu2 - ccz;
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

        const float4 r0v = make_float4(mx, my, ca * kNegHalfLog2e, cb * kNegLog2e);
        const float qcv = cc * kNegHalfLog2e;
        rec0[rid] = r0v;
        rec1[rid] = make_float4(qcv, opx, pre[0], pre[1]);
        rec2[rid] = make_float2(pre[2], __uint_as_float(entry_box_pack(r0v, qcv, opx)));
        const uint2 rc = make_uint2((uint32_t)x0 | ((uint32_t)y0 << 16), (uint32_t)x1 | ((uint32_t)y1 << 16));
        rect[rid] = rc;
        depth_key[rid] = __float_as_uint(tz);
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
