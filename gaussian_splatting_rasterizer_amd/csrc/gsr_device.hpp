// gsr_device.hpp -- device-side definitions shared by the gfx950 kernels.
//
// Floating-point decisions (culling, field-of-view clamp, radius, tile
// rectangle, colour clamp, alpha skip/clamp, early termination,
// suffix-denominator mask) follow a fixed operation order with no FMA
// contraction (the library is compiled with -ffp-contract=off; fused
// multiply-adds appear only where written as __builtin_fmaf / __builtin_fma):
// preprocess geometry in float64, everything per pixel in float32.  This makes
// every such integer decision reproducible by any implementation of the same
// order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gsr {

constexpr int kTile = 16;
constexpr int kMaxViews = 32;

// Thresholds of the standard 3DGS compositing rule (readings of "the original
// gsplat tile binning and front-to-back compositing" of the Stage 1 step).
constexpr float kAlphaMax = 0.99f;
constexpr float kAlphaMin = 0x1.010102p-8f;   // float32 nearest to 1/255
constexpr float kTMin = 1e-4f;
constexpr double kDilation = 0.3;             // px^2 added to the projected covariance (float64 geometry)
constexpr float kEigFloor = 0.1f;
constexpr double kFovClamp = 1.3;
constexpr float kSCutoff = 8.0f;              // 2^-8 < 1/255: no alpha can pass beyond this exponent
constexpr float kHalfLog2e = 0x1.715476p-1f;  // float32 nearest to log2(e) / 2
constexpr float kInvHalfLog2e = 1.0f / kHalfLog2e;

// 2^e for e in [-8, 1/2]: k = rint(e), f = e - k (exact, |f| <= 1/2), 2^f by
// the degree-7 Taylor polynomial sum_j (f ln 2)^j / j! with each coefficient
// rounded to float32 (Horner, fused multiply-adds), then exact scaling by 2^k.
__device__ __forceinline__ float exp2_spec(float e) {
    const float k = __builtin_rintf(e);
    const float f = e - k;
    float p = 0x1.ffcbfcp-17f;
    p = __builtin_fmaf(p, f, 0x1.430912p-13f);
    p = __builtin_fmaf(p, f, 0x1.5d87fep-10f);
    p = __builtin_fmaf(p, f, 0x1.3b2ab6p-7f);
    p = __builtin_fmaf(p, f, 0x1.c6b08ep-5f);
    p = __builtin_fmaf(p, f, 0x1.ebfbe0p-3f);
    p = __builtin_fmaf(p, f, 0x1.62e430p-1f);
    p = __builtin_fmaf(p, f, 1.0f);
    return __builtin_amdgcn_ldexpf(p, (int)k);
}

// Real spherical harmonics up to degree 3 (m = -l..l order, graphics sign
// convention), float32 normalisation constants.
constexpr float kSH0 = 0x1.20dd76p-2f;     // 1/(2 sqrt(pi))
constexpr float kSH1 = 0x1.f45438p-2f;     // sqrt(3/(4 pi))
constexpr float kSH2a = 0x1.17b142p+0f;    // sqrt(15/pi)/2
constexpr float kSH2b = 0x1.42f602p-2f;    // sqrt(5/pi)/4
constexpr float kSH2c = 0x1.17b142p-1f;    // sqrt(15/pi)/4
constexpr float kSH3a = 0x1.2e1a32p-1f;    // sqrt(35/(2 pi))/4
constexpr float kSH3b = 0x1.71ff8ep+1f;    // sqrt(105/pi)/2
constexpr float kSH3c = 0x1.d403d0p-2f;    // sqrt(21/(2 pi))/4
constexpr float kSH3d = 0x1.7e21f0p-2f;    // sqrt(7/pi)/4
constexpr float kSH3e = 0x1.71ff8ep+0f;    // sqrt(105/pi)/4

__device__ __forceinline__ void sh_basis_f32(float x, float y, float z, int d, float* B) {
    B[0] = kSH0;
    if (d <= 1) return;
    B[1] = -kSH1 * y;
    B[2] = kSH1 * z;
    B[3] = -kSH1 * x;
    if (d <= 4) return;
    const float xx = x * x, yy = y * y, zz = z * z;
    const float xy = x * y, yz = y * z, xz = x * z;
    B[4] = kSH2a * xy;
    B[5] = -kSH2a * yz;
    B[6] = kSH2b * ((2.0f * zz - xx) - yy);
    B[7] = -kSH2a * xz;
    B[8] = kSH2c * (xx - yy);
    if (d <= 9) return;
    B[9] = (-kSH3a * y) * (3.0f * xx - yy);
    B[10] = (kSH3b * xy) * z;
    B[11] = (-kSH3c * y) * ((4.0f * zz - xx) - yy);
    B[12] = (kSH3d * z) * ((2.0f * zz - 3.0f * xx) - 3.0f * yy);
    B[13] = (-kSH3c * x) * ((4.0f * zz - xx) - yy);
    B[14] = (kSH3e * z) * (xx - yy);
    B[15] = (-kSH3a * x) * (xx - 3.0f * yy);
}

__device__ __forceinline__ void sh_basis_f64(double x, double y, double z, int d, double* B) {
    const double c0 = 0.28209479177387814, c1 = 0.48860251190291992;
    const double c2a = 1.0925484305920792, c2b = 0.31539156525252005, c2c = 0.54627421529603959;
    const double c3a = 0.59004358992664352, c3b = 2.8906114426405538, c3c = 0.45704579946446572;
    const double c3d = 0.3731763325901154, c3e = 1.4453057213202769;
    B[0] = c0;
    if (d <= 1) return;
    B[1] = -c1 * y;
    B[2] = c1 * z;
    B[3] = -c1 * x;
    if (d <= 4) return;
    const double xx = x * x, yy = y * y, zz = z * z;
    B[4] = c2a * x * y;
    B[5] = -c2a * y * z;
    B[6] = c2b * (2.0 * zz - xx - yy);
    B[7] = -c2a * x * z;
    B[8] = c2c * (xx - yy);
    if (d <= 9) return;
    B[9] = -c3a * y * (3.0 * xx - yy);
    B[10] = c3b * x * y * z;
    B[11] = -c3c * y * (4.0 * zz - xx - yy);
    B[12] = c3d * z * (2.0 * zz - 3.0 * xx - 3.0 * yy);
    B[13] = -c3c * x * (4.0 * zz - xx - yy);
    B[14] = c3e * z * (xx - yy);
    B[15] = -c3a * x * (xx - 3.0 * yy);
}

// Camera as passed by value to the kernels: [R (9), t (3), fx, fy, cx, cy].
struct CamPack {
    float c[kMaxViews][16];    // R (9, row-major), t (3), fx, fy, cx, cy
    double lim[kMaxViews][2];  // field-of-view clamp kFovClamp ((W / 2) / fx), kFovClamp ((H / 2) / fy),
                               // evaluated on the host in that float64 order
};

// Per-(view, Gaussian) record, three float4 at index rid = v * G + g:
//   r0 = {mx, my, s1, s2}
//   r1 = {s3, opacity, pre_r, pre_g}
//   r2 = {pre_b, entry box (two binary16 half-widths), mx_lo, my_lo}
// The projected centre is the float64 value mx + mx_lo (likewise y) split into two float32s.
// The Gaussian weight at pixel offset (dx, dy) = p - mu is 2^-S with
// S = (s1 dx + s2 dy)^2 + (s3 dy)^2 = k (dx, dy) Sigma2^-1 (dx, dy)^T, k = log2(e) / 2:
// [[s1, 0], [s2, s3]] is the Cholesky factor of k times the conic, so S is a sum of squares
// and keeps its relative precision however elongated the footprint.

// Camera-space centre t = R mu + t_v in float64 from the float32 inputs, in the written order
// (each product of two float32 values is exact; the sums round once each, left to right).
__device__ __forceinline__ void camera_centre_f64(const float* cam, const double mu[3], double t[3]) {
#pragma unroll
    for (int i = 0; i < 3; ++i)
        t[i] = (((double)cam[3 * i] * mu[0] + (double)cam[3 * i + 1] * mu[1]) + (double)cam[3 * i + 2] * mu[2]) +
               (double)cam[9 + i];
}

// Field-of-view clamp of the perspective Jacobian's lateral offset: bit 0 when |tx (1 / tz)| exceeds
// lim[0], bit 1 likewise in y.  One function for the preprocess and the backward, so both take
// the same decision from the same float64 operations.
__device__ __forceinline__ int fov_clip_bits(const double t[3], const double lim[2]) {
    const double iz = 1.0 / t[2];
    const double ux = t[0] * iz, uy = t[1] * iz;
    return ((ux < -lim[0] || ux > lim[0]) ? 1 : 0) | ((uy < -lim[1] || uy > lim[1]) ? 2 : 0);
}

// The centre relative to the origin of the tile with index tc along that axis: hi - 16 tc is exact
// whenever the entry can reach the tile, then lo is added with one rounding.
__device__ __forceinline__ float tile_centre(float hi, float lo, int tc) {
    return (hi - (float)(kTile * tc)) + lo;
}

// S at the offset (dx, dy), in the written order.
__device__ __forceinline__ float quad_S(float s1, float s2, float s3, float dx, float dy) {
    const float u = __builtin_fmaf(s1, dx, s2 * dy);
    const float w = s3 * dy;
    return __builtin_fmaf(u, u, w * w);
}

// colour clamp: a pre-clamp colour that is negative or not finite is clamped to 0 and its
// clamp bit cleared (the clamp mask of the SH score)
__device__ __forceinline__ bool colour_ok(float pre) { return pre >= 0.0f && pre <= 3.40282347e+38f; }
__device__ __forceinline__ float clamp_colour(float pre) { return colour_ok(pre) ? pre : 0.0f; }

// A tile rectangle in 32 bits, for tile grids of at most 256 x 256: x0, y0,
// width - 1, height - 1 in bytes; 0xffffffff marks an empty rectangle (culled
// record), which no real rectangle can encode (x0 + width <= 256).
__device__ __forceinline__ uint32_t pack_rect(uint2 r) {
    if (r.y == 0u) return 0xffffffffu;
    const uint32_t x0 = r.x & 0xffffu, y0 = r.x >> 16, x1 = r.y & 0xffffu, y1 = r.y >> 16;
    return x0 | (y0 << 8) | ((x1 - x0 - 1u) << 16) | ((y1 - y0 - 1u) << 24);
}

__device__ __forceinline__ uint2 unpack_rect(uint32_t q) {
    if (q == 0xffffffffu) return make_uint2(0u, 0u);
    const uint32_t x0 = q & 0xffu, y0 = (q >> 8) & 0xffu, x1 = x0 + ((q >> 16) & 0xffu) + 1u,
                   y1 = y0 + (q >> 24) + 1u;
    return make_uint2(x0 | (y0 << 16), x1 | (y1 << 16));
}

// Conservative pixel bounding box of the region where an entry can pass the
// alpha test, used only to skip entries that cannot pass anywhere in a block
// of pixels.  With K = L L^T, L = [[s1, 0], [s2, s3]] (the record's float32
// factors taken as exact), the exact exponent magnitude is S*(d) = d^T K d and
// alpha = o 2^-S >= 1/255 needs S <= t with t = min(8, log2(255 o)).  The
// float32 evaluation (offsets rounded once, the products and two fused
// multiply-adds of quad_S) differs from S* by at most
// u (6.1 S* + 4.04 E sqrt(S*)) with u = 2^-24 and E = |s1 dx| + |s2 dy| <=
// 2 sqrt(kappa S*), kappa = max(Kinv_xx, Kinv_yy)^2 / det(Kinv); so a pixel can
// pass only if S*(d) <= t_eff = (t + 1e-5) / (1 - u (8 + 10 sqrt(kappa))) (1e-5
// covers the float32 exponential and the product o * G).  The region S* <= t_eff
// has half-widths sqrt(t_eff Kinv_xx) and sqrt(t_eff Kinv_yy), widened by
// 0.01 px (more than the rounding of the float32 box edges around a
// tile-relative centre) and stored as two binary16 values rounded up (infinite
// when too large or when the growth factor reaches 1/2: never skip; -infinity
// when the entry can never pass, o <= 1/255: the box is empty).  Evaluated in
// float64 from the float32 factors; every float64 rounding is far below the
// margins.
__device__ __forceinline__ uint32_t half_bits_up(float v) {  // least binary16 >= v, for v > 0
    if (!(v <= 65504.0f)) return 0x7c00u;
    const _Float16 h = (_Float16)v;
    uint32_t b = (uint32_t)__builtin_bit_cast(uint16_t, h);
    if ((float)h < v) ++b;
    return b;
}

__device__ __forceinline__ uint32_t entry_box_pack(float s1f, float s2f, float s3f, float opac) {
    const double tt = log2(255.0 * (double)opac);
    if (!(tt > -1e-5)) return 0xfc00fc00u;
    const double s1 = s1f, s2 = s2f, s3 = s3f;
    const double p1 = s1 * s1, p3 = s3 * s3;
    if (!(p1 > 0.0) || !(p3 > 0.0)) return 0x7c007c00u;
    const double kxx = (s2 * s2 + p3) / (p1 * p3), kyy = 1.0 / p3, kdet = 1.0 / (p1 * p3);
    const double kmax = kxx > kyy ? kxx : kyy;
    const double grow = 0x1p-24 * (8.0 + 10.0 * sqrt(kmax * kmax / kdet));
    if (!(grow < 0.5)) return 0x7c007c00u;
    const double te = ((tt < 8.0 ? tt : 8.0) + 1e-5) / (1.0 - grow);
    // (1 + 1e-6) keeps the float32 rounding above the float64 value
    const double wx = (sqrt(te * kxx) + 0.01) * (1.0 + 1e-6), wy = (sqrt(te * kyy) + 0.01) * (1.0 + 1e-6);
    return half_bits_up((float)wx) | (half_bits_up((float)wy) << 16);
}

// Whether some point of the rectangle [x0, x1] x [y0, y1] (the tile-relative pixel-centre bounds of a
// quadrant) can pass an entry's alpha test, decided in float32 with margins that make a false result safe.
// The region that can pass is S*(p - m) <= t_eff (see above), S*(d) = (s1 dx + s2 dy)^2 + (s3 dy)^2 exact
// on the float32 values.  The packed box bounds t_eff from above: its half-widths are at least
// sqrt(t_eff Kinv_xx) and sqrt(t_eff Kinv_yy), so t_eff <= min(ex^2 / Kinv_xx, ey^2 / Kinv_yy) =
// min(ex^2 s1^2 s3^2 / (s2^2 + s3^2), ey^2 s3^2), taken here with a relative 1e-4 and an absolute 1e-3 on
// top (infinite half-widths: never skip; an empty box never reaches this test).  S* is convex with its
// minimum 0 at m, so over a rectangle that does not hold m its minimum lies on an edge facing m (the
// segment from m to any other point of the rectangle crosses such an edge first, where S* is no larger):
// at most two edges, each a one-dimensional quadratic minimised at a clamped point.  That float32 minimum
// is compared after subtracting 2^-16 of the sum of its terms' magnitudes, far above its rounding
// (including the rounding of the edge offsets and of the minimiser, whose error moves a quadratic's value
// at its minimum only to second order).  The minimum over the rectangle is no larger than over its pixel
// centres, so a false result means no pixel of the quadrant passes.
// (The reciprocals are the hardware approximation, within an ulp or two: the threshold's margin covers it,
// and an approximate minimiser changes an edge quadratic's minimum only to second order.)
struct EntryConic {
    float a, b, c, ra, rc;  // S* = a dx^2 + 2 b dx dy + c dy^2, ra = 1/a, rc = 1/c
    float te;               // the bound on t_eff (infinite: never skip)
};

__device__ __forceinline__ EntryConic entry_conic_from_box(float s1, float s2, float s3, uint32_t packed) {
    EntryConic k;
    k.a = s1 * s1;
    k.b = s1 * s2;
    const float p3 = s3 * s3;
    k.c = s2 * s2 + p3;
    k.ra = __builtin_amdgcn_rcpf(k.a);
    k.rc = __builtin_amdgcn_rcpf(k.c);
    const float ex = (float)__builtin_bit_cast(_Float16, (uint16_t)(packed & 0xffffu));
    const float ey = (float)__builtin_bit_cast(_Float16, (uint16_t)(packed >> 16));
    const float tx = ex * ex * k.a * p3 * k.rc, ty = ey * ey * p3;
    const float t = tx < ty ? tx : ty;
    k.te = (ex < __builtin_inff() && ey < __builtin_inff() && t == t) ? t * (1.0f + 1e-4f) + 1e-3f
                                                                      : __builtin_inff();
    return k;
}

__device__ __forceinline__ bool ellipse_meets_rect(float mx, float my, const EntryConic& k, float x0, float x1,
                                                   float y0, float y1) {
    if (!(k.te < __builtin_inff())) return true;
    const float cx = fminf(fmaxf(mx, x0), x1), cy = fminf(fmaxf(my, y0), y1);
    if (cx == mx && cy == my) return true;
    bool meets = false;
    if (cx != mx) {  // the vertical edge x = cx faces m
        const float dx = cx - mx;
        const float dy = fminf(fmaxf(-k.b * dx * k.rc, y0 - my), y1 - my);
        const float t0 = k.a * dx * dx, t1 = 2.0f * k.b * dx * dy, t2 = k.c * dy * dy;
        meets = meets || (t0 + t1) + t2 - 0x1p-16f * (t0 + fabsf(t1) + t2) <= k.te;
    }
    if (cy != my) {  // the horizontal edge y = cy faces m
        const float dy = cy - my;
        const float dx = fminf(fmaxf(-k.b * dy * k.ra, x0 - mx), x1 - mx);
        const float t0 = k.a * dx * dx, t1 = 2.0f * k.b * dx * dy, t2 = k.c * dy * dy;
        meets = meets || (t0 + t1) + t2 - 0x1p-16f * (t0 + fabsf(t1) + t2) <= k.te;
    }
    return meets;
}

// {x0, x1, y0, y1} of the packed box around the (tile-relative) centre (mx, my).
__device__ __forceinline__ float4 entry_box_unpack(float mx, float my, uint32_t packed) {
    const float ex = (float)__builtin_bit_cast(_Float16, (uint16_t)(packed & 0xffffu));
    const float ey = (float)__builtin_bit_cast(_Float16, (uint16_t)(packed >> 16));
    return make_float4(mx - ex, mx + ex, my - ey, my + ey);
}

// Reduce eight values over the 64 lanes; returns in every lane the total of
// component (lane >> 3) & 7.  Reduce-scatter with gfx950 lane permutations:
//   permlane32_swap pairs component i (kept in lanes 0-31) with i + 4 (lanes 32-63),
//   permlane16_swap pairs rows, a row_ror:8 exchange splits each row in halves,
//   then quad_perm / row_half_mirror adds finish the sum inside 8-lane groups.
template <int CTRL>
__device__ __forceinline__ float fadd_dpp(float keep, float send) {
    return keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_reduce8(const float (&x)[8], int lane) {
    float a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[i]), __float_as_uint(x[i + 4]), false, false);
        a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const auto s0 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[0]), __float_as_uint(a[2]), false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[1]), __float_as_uint(a[3]), false, false);
    const float b0 = __uint_as_float(s0[0]) + __uint_as_float(s0[1]);  // rows hold components 0, 2, 4, 6
    const float b1 = __uint_as_float(s1[0]) + __uint_as_float(s1[1]);  // rows hold components 1, 3, 5, 7
    const bool hi8 = lane & 8;
    float c = fadd_dpp<0x128>(hi8 ? b1 : b0, hi8 ? b0 : b1);  // row_ror:8
    c = fadd_dpp<0xB1>(c, c);                                  // quad_perm [1,0,3,2]
    c = fadd_dpp<0x4E>(c, c);                                  // quad_perm [2,3,0,1]
    c = fadd_dpp<0x141>(c, c);                                 // row_half_mirror
    return c;
}

// Sum of one value over the 64 lanes, in every lane: the same permutation
// sequence with each value paired with itself.
__device__ __forceinline__ float wave_sum1(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    const float b = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    float c = fadd_dpp<0x128>(b, b);  // row_ror:8
    c = fadd_dpp<0xB1>(c, c);          // quad_perm [1,0,3,2]
    c = fadd_dpp<0x4E>(c, c);          // quad_perm [2,3,0,1]
    c = fadd_dpp<0x141>(c, c);         // row_half_mirror
    return c;
}

// d B_k / d(x, y, z) of sh_basis_f32, (x, y, z) as independent variables; dB[3 k + j].
__device__ __forceinline__ void sh_basis_grad_f32(float x, float y, float z, int d, float* dB) {
    for (int i = 0; i < 3 * d; ++i) dB[i] = 0.0f;
    if (d <= 1) return;
    dB[3 * 1 + 1] = -kSH1;
    dB[3 * 2 + 2] = kSH1;
    dB[3 * 3 + 0] = -kSH1;
    if (d <= 4) return;
    dB[3 * 4 + 0] = kSH2a * y;
    dB[3 * 4 + 1] = kSH2a * x;
    dB[3 * 5 + 1] = -kSH2a * z;
    dB[3 * 5 + 2] = -kSH2a * y;
    dB[3 * 6 + 0] = -2.0f * kSH2b * x;
    dB[3 * 6 + 1] = -2.0f * kSH2b * y;
    dB[3 * 6 + 2] = 4.0f * kSH2b * z;
    dB[3 * 7 + 0] = -kSH2a * z;
    dB[3 * 7 + 2] = -kSH2a * x;
    dB[3 * 8 + 0] = 2.0f * kSH2c * x;
    dB[3 * 8 + 1] = -2.0f * kSH2c * y;
    if (d <= 9) return;
    const float xx = x * x, yy = y * y, zz = z * z;
    dB[3 * 9 + 0] = -6.0f * kSH3a * x * y;
    dB[3 * 9 + 1] = -kSH3a * (3.0f * xx - 3.0f * yy);
    dB[3 * 10 + 0] = kSH3b * y * z;
    dB[3 * 10 + 1] = kSH3b * x * z;
    dB[3 * 10 + 2] = kSH3b * x * y;
    dB[3 * 11 + 0] = 2.0f * kSH3c * x * y;
    dB[3 * 11 + 1] = -kSH3c * (4.0f * zz - xx - 3.0f * yy);
    dB[3 * 11 + 2] = -8.0f * kSH3c * y * z;
    dB[3 * 12 + 0] = -6.0f * kSH3d * x * z;
    dB[3 * 12 + 1] = -6.0f * kSH3d * y * z;
    dB[3 * 12 + 2] = kSH3d * (6.0f * zz - 3.0f * xx - 3.0f * yy);
    dB[3 * 13 + 0] = -kSH3c * (4.0f * zz - 3.0f * xx - yy);
    dB[3 * 13 + 1] = 2.0f * kSH3c * x * y;
    dB[3 * 13 + 2] = -8.0f * kSH3c * x * z;
    dB[3 * 14 + 0] = 2.0f * kSH3e * x * z;
    dB[3 * 14 + 1] = -2.0f * kSH3e * y * z;
    dB[3 * 14 + 2] = kSH3e * (xx - yy);
    dB[3 * 15 + 0] = -kSH3a * (3.0f * xx - 3.0f * yy);
    dB[3 * 15 + 1] = 6.0f * kSH3a * x * y;
}

}  // namespace gsr
