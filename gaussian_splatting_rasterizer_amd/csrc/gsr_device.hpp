// gsr_device.hpp -- device-side definitions shared by the gfx950 kernels.
//
// Floating-point decisions (culling, radius, tile rectangle, colour clamp,
// alpha skip/clamp, early termination, suffix-denominator mask) follow a fixed
// float32 operation order with no FMA contraction (the library is compiled
// with -ffp-contract=off; fused multiply-adds appear only where written as
// __builtin_fmaf).  This makes every such integer decision reproducible by any
// implementation of the same order.
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
constexpr float kDilation = 0.3f;
constexpr float kEigFloor = 0.1f;
constexpr float kFovClamp = 1.3f;
constexpr float kECutoff = -8.0f;             // 2^-8 < 1/255: no alpha can pass below this
constexpr float kNegLog2e = -0x1.715476p+0f;  // float32 nearest to -log2(e)
constexpr float kNegHalfLog2e = -0x1.715476p-1f;

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
    float lim[kMaxViews][2];   // field-of-view clamp kFovClamp ((W / 2) / fx), kFovClamp ((H / 2) / fy),
                               // evaluated on the host in that float32 order
};

// Per-(view, Gaussian) record, three float4 (48 B) at index rid = v * G + g:
//   r0 = {mx, my, qa, qb}
//   r1 = {qc, opacity, pre_r, pre_g}
//   r2 = {pre_b, bits(pair offset), bits(x0 | y0 << 16), bits(x1 | y1 << 16)}
// The Gaussian weight at pixel offset (dx, dy) = p - mu is 2^(qa dx^2 + qb dx dy + qc dy^2),
// i.e. qa = -log2(e)/2 A, qb = -log2(e) B, qc = -log2(e)/2 C for the conic [[A, B], [B, C]].

__device__ __forceinline__ float clamp_colour(float pre) { return pre >= 0.0f ? pre : 0.0f; }

// Evaluate one list entry at one pixel with the canonical float32 order.
// Returns 0 when the pixel is beyond the distance cut, 1 when alpha < 1/255,
// 2 when the entry contributes (alpha, clamped and the offset (dx, dy) set).
__device__ __forceinline__ int eval_alpha(float4 r0, float qc, float opac, float px, float py, float& dx,
                                          float& dy, float& alpha, bool& clamped) {
    dx = px - r0.x;
    dy = py - r0.y;
    const float e = __builtin_fmaf(dx, __builtin_fmaf(r0.z, dx, r0.w * dy), (qc * dy) * dy);
    if (!(e >= kECutoff)) return 0;
    const float aG = opac * exp2_spec(e);
    clamped = !(aG < kAlphaMax);
    alpha = clamped ? kAlphaMax : aG;
    return alpha >= kAlphaMin ? 2 : 1;
}

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
// of pixels.  With Q(d) = a' dx^2 + 2 b' dx dy + c' dy^2 (a' = -qa, b' = -qb/2,
// c' = -qc, positive definite) the exact exponent is -Q(d), and alpha = o G >=
// 1/255 needs it to be >= -t with t = min(8, log2(255 o)).  The float32
// evaluation of the exponent (offsets rounded once, then three products and two
// fused multiply-adds) differs from -Q(d) by at most 3u Qabs(d) + 3u Q(d) with
// u = 2^-24 and Qabs <= cond(A) Q, and the float32 exponential and product
// o * G add a few more units of u; so a pixel can pass only if
// Q(d) <= t_eff = (t + 1e-5) / (1 - 8 u (cond + 1)).  The region Q <= t_eff has
// half-widths sqrt(t_eff c' / det) and sqrt(t_eff a' / det), widened by 0.01 px
// plus 1e-6 of (|centre| + half-width) -- more than the rounding of the float32
// centre +- half-width at use -- and stored as two binary16 values rounded up
// (infinite when too large or when 8 u (cond + 1) >= 1/2: never skip; -infinity
// when the entry can never pass, o <= 1/255: the box is empty).
//
// All of it is evaluated in float32 from the exact float32 coefficients, every
// operation rounded once (no contraction; IEEE division and square root), and
// kept above the exact values: log2f is within 1 ulp (<= 1e-6 for |t| <= 8,
// with the rounding of 255 o), so t gets 1.2e-5 instead of 1e-5; det = a'c' - b'^2
// comes from Kahan's difference of products (fused multiply-adds; within 2u of
// the exact value however much it cancels), so the radicand is within ~20u and
// the half-width within ~11u, which the factor 1 + 2^-17 covers; the last sums
// (4 roundings) get 1 + 2^-20.  Empty when log2(255 o) <= -1e-5 + 1e-6 < 0.
__device__ __forceinline__ uint32_t half_bits_up(float v) {  // least binary16 >= v, for v > 0
    if (!(v <= 65504.0f)) return 0x7c00u;
    const _Float16 h = (_Float16)v;
    uint32_t b = (uint32_t)__builtin_bit_cast(uint16_t, h);
    if ((float)h < v) ++b;
    return b;
}

__device__ __forceinline__ uint32_t entry_box_pack(float4 r0, float qc, float opac) {
    const float a = -r0.z, b = -0.5f * r0.w, c = -qc;  // exact
    const float tt = log2f(255.0f * opac);
    if (!(tt > -1e-5f)) return 0xfc00fc00u;
    const float w = b * b;
    const float det = __builtin_fmaf(a, c, -w) + __builtin_fmaf(-b, b, w);
    if (!(det > 0.0f) || !(a > 0.0f) || !(c > 0.0f)) return 0x7c007c00u;
    const float t = (tt < 8.0f ? tt : 8.0f) + 1.2e-5f;
    const float amc = a - c;
    const float mid = 0.5f * (a + c), hd = __builtin_sqrtf(0.25f * (amc * amc) + b * b);
    const float lmax = mid + hd, lmin = det / lmax;
    const float grow = 0x1p-21f * (lmax / lmin + 1.0f);  // 8 u (cond + 1)
    if (!(grow < 0.5f)) return 0x7c007c00u;
    const float te = t / (1.0f - grow);
    const float kw = 1.0f + 0x1p-17f, ks = 1.0f + 0x1p-20f;
    const float ex = __builtin_sqrtf(te * c / det) * kw, ey = __builtin_sqrtf(te * a / det) * kw;
    const float wx = ((ex + 0.01f) + 1e-6f * (__builtin_fabsf(r0.x) + ex)) * ks;
    const float wy = ((ey + 0.01f) + 1e-6f * (__builtin_fabsf(r0.y) + ey)) * ks;
    return half_bits_up(wx) | (half_bits_up(wy) << 16);
}

// {x0, x1, y0, y1} of the packed box around the centre (mx, my).
__device__ __forceinline__ float4 entry_box_unpack(float mx, float my, uint32_t packed) {
    const float ex = (float)__builtin_bit_cast(_Float16, (uint16_t)(packed & 0xffffu));
    const float ey = (float)__builtin_bit_cast(_Float16, (uint16_t)(packed >> 16));
    return make_float4(mx - ex, mx + ex, my - ey, my + ey);
}

// Compensated (Kahan) accumulation of the prefix colour; the true sum is hi - comp.
__device__ __forceinline__ void kahan_add(float& hi, float& comp, float x) {
    const float y = x - comp;
    const float t = hi + y;
    comp = (t - hi) - y;
    hi = t;
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
