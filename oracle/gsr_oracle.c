/*
 * gsr_oracle.c -- CPU oracle for the tile-binned Gaussian-splat render and the
 * analytic score replay.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test-suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code with the HIP path.
 *
 * Source of the method: the page "Research Proposal: Renderer Score Tokens for
 * Recurrent Gaussian Splatting" -- section "Two-Stage Algorithm" (Stage 1
 * standard render, residual equation; Stage 2 analytic score replay, suffix
 * equation, masks), section "Exact Score Operators" (alpha/weight definitions,
 * residual-suffix contrast and support, opacity-logit score, SH score, 2D
 * Gaussian kernel and its centre gradient, projected-centre mean score,
 * projection Jacobian, cross-view weight, covector pullback, conditioning
 * matrix and its statistics, appearance aggregation) and "Final Token and
 * Updater" (token layout).  The 3D Gaussian primitive is the one of the ATSplat
 * summary page ("前置知识: 3DGS").
 *
 * How it computes:
 *  - Every floating-point DECISION (culling, radius, tile rectangle, the SH
 *    colour clamp, alpha skip, alpha clamp, early termination, the suffix
 *    denominator mask) is taken in float32 following the written canonical
 *    operation order, so that an independent GPU implementation of the same
 *    order reaches the same integers.  The float32 exponential used by those
 *    decisions is the published range-reduction + Taylor method (exp2 split
 *    into an integer power and a fraction in [-1/2, 1/2], degree-7 Taylor
 *    polynomial of 2^f in Horner form with fused multiply-adds).
 *  - Every VALUE (colours, alpha, transmittance, suffix composites, scores,
 *    tokens) is computed in float64 from float64 copies of the inputs, with
 *    the float32 decisions frozen.  This is also what makes the finite
 *    difference pins exact: the loss is a smooth function of the values once
 *    the contributor sets and clamp states are fixed.
 *  - Candidate lists are brute force (every Gaussian whose tile rectangle
 *    holds the tile), ordered by (depth bits, Gaussian index).
 *  - The suffix composite is computed by explicit back-to-front summation,
 *    never by the subtraction formula of the replay.
 *  - Scores are the literal per-pixel sums of the score operators; tokens are
 *    the literal cross-view formulas; eigenvalues by cyclic Jacobi rotations.
 *  - Feature composite and attribution scatter: per-Gaussian attribute vectors
 *    composited with the render weights w = T alpha, and per-pixel maps sent
 *    back to the Gaussians along the same weights (literal sums).
 *  - The renderer backward (the gradient of the image through the composite,
 *    the 2D Gaussian, the EWA projection, the covariance from quaternion and
 *    scales, and the SH colour including its view direction) is an explicit
 *    chain rule per contribution and per (Gaussian, view), in float64, with the
 *    same frozen decisions; the forward formulas it differentiates are those
 *    of the ATSplat summary page's 3DGS primitive.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ----------------------------------------------------------------------------
 * Fixed readings shared with the GPU path by specification (not by code).
 * ------------------------------------------------------------------------- */
#define TILE 16
#define ALPHA_MAX_F 0.99f
#define ALPHA_MAX_D 0.99
#define T_MIN_F 1e-4f
#define EIG_FLOOR_F 0.1f
#define FOV_CLAMP_D 1.3
#define DILATION_D 0.3
#define S_CUTOFF_F 8.0f

static float g_alpha_min;     /* float32 nearest to 1/255 */
static float g_exp2_coef[8];  /* float32 nearest to ln(2)^j / j! */
static float g_hl2e;          /* float32 nearest to log2(e) / 2 */
static float g_sh32[16];      /* float32 SH normalisation constants (signed) */
static double g_sh64[16];

static void init_constants(void)
{
    static int done = 0;
    if (done) return;
    g_alpha_min = (float)(1.0L / 255.0L);
    long double c = 1.0L;
    const long double ln2 = 0.693147180559945309417232121458176568L;
    for (int j = 0; j < 8; ++j) {
        g_exp2_coef[j] = (float)c;
        c = c * ln2 / (long double)(j + 1);
    }
    const long double log2e = 1.442695040888963407359924681001892137L;
    g_hl2e = (float)(0.5L * log2e);
    const long double pi = 3.141592653589793238462643383279502884L;
    long double k[16];
    /* real spherical harmonics, l <= 3, m = -l..l, classic graphics sign convention */
    k[0] = 0.5L * sqrtl(1.0L / pi);
    k[1] = -sqrtl(3.0L / (4.0L * pi));
    k[2] = sqrtl(3.0L / (4.0L * pi));
    k[3] = -sqrtl(3.0L / (4.0L * pi));
    k[4] = 0.5L * sqrtl(15.0L / pi);
    k[5] = -0.5L * sqrtl(15.0L / pi);
    k[6] = 0.25L * sqrtl(5.0L / pi);
    k[7] = -0.5L * sqrtl(15.0L / pi);
    k[8] = 0.25L * sqrtl(15.0L / pi);
    k[9] = -0.25L * sqrtl(35.0L / (2.0L * pi));
    k[10] = 0.5L * sqrtl(105.0L / pi);
    k[11] = -0.25L * sqrtl(21.0L / (2.0L * pi));
    k[12] = 0.25L * sqrtl(7.0L / pi);
    k[13] = -0.25L * sqrtl(21.0L / (2.0L * pi));
    k[14] = 0.25L * sqrtl(105.0L / pi);
    k[15] = -0.25L * sqrtl(35.0L / (2.0L * pi));
    for (int i = 0; i < 16; ++i) {
        g_sh32[i] = (float)k[i];
        g_sh64[i] = (double)k[i];
    }
    done = 1;
}

/* float32 2^e for e in [-8, 1/2]: e = k + f with k = rint(e) and |f| <= 1/2 exact,
 * 2^f by the degree-7 Taylor polynomial in Horner form with fused multiply-adds,
 * then an exact scaling by 2^k. */
float orc_exp2f(float e)
{
    init_constants();
    float k = rintf(e);
    float f = e - k;
    float p = g_exp2_coef[7];
    for (int j = 6; j >= 0; --j) p = fmaf(p, f, g_exp2_coef[j]);
    return ldexpf(p, (int)k);
}

void orc_exp2f_array(const float* in, float* out, int64_t n)
{
    init_constants();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_exp2f(in[i]);
}

void orc_constants(float* out /* [28] */)
{
    init_constants();
    out[0] = g_alpha_min;
    for (int j = 0; j < 8; ++j) out[1 + j] = g_exp2_coef[j];
    out[9] = g_hl2e;
    out[10] = 0.0f;
    for (int i = 0; i < 16; ++i) out[11 + i] = g_sh32[i];
    out[27] = 0.0f;
}

/* ----------------------------------------------------------------------------
 * SH basis (degree <= 3) in float32 canonical order and in float64.
 * ------------------------------------------------------------------------- */
static void sh_basis32(float x, float y, float z, int d, float* B)
{
    const float* K = g_sh32;
    B[0] = K[0];
    if (d <= 1) return;
    B[1] = K[1] * y;
    B[2] = K[2] * z;
    B[3] = K[3] * x;
    if (d <= 4) return;
    float xx = x * x, yy = y * y, zz = z * z;
    float xy = x * y, yz = y * z, xz = x * z;
    B[4] = K[4] * xy;
    B[5] = K[5] * yz;
    B[6] = K[6] * ((2.0f * zz - xx) - yy);
    B[7] = K[7] * xz;
    B[8] = K[8] * (xx - yy);
    if (d <= 9) return;
    B[9] = (K[9] * y) * (3.0f * xx - yy);
    B[10] = (K[10] * xy) * z;
    B[11] = (K[11] * y) * ((4.0f * zz - xx) - yy);
    B[12] = (K[12] * z) * ((2.0f * zz - 3.0f * xx) - 3.0f * yy);
    B[13] = (K[13] * x) * ((4.0f * zz - xx) - yy);
    B[14] = (K[14] * z) * (xx - yy);
    B[15] = (K[15] * x) * (xx - 3.0f * yy);
}

static void sh_basis64(double x, double y, double z, int d, double* B)
{
    const double* K = g_sh64;
    B[0] = K[0];
    if (d <= 1) return;
    B[1] = K[1] * y;
    B[2] = K[2] * z;
    B[3] = K[3] * x;
    if (d <= 4) return;
    double xx = x * x, yy = y * y, zz = z * z;
    B[4] = K[4] * x * y;
    B[5] = K[5] * y * z;
    B[6] = K[6] * (2.0 * zz - xx - yy);
    B[7] = K[7] * x * z;
    B[8] = K[8] * (xx - yy);
    if (d <= 9) return;
    B[9] = K[9] * y * (3.0 * xx - yy);
    B[10] = K[10] * x * y * z;
    B[11] = K[11] * y * (4.0 * zz - xx - yy);
    B[12] = K[12] * z * (2.0 * zz - 3.0 * xx - 3.0 * yy);
    B[13] = K[13] * x * (4.0 * zz - xx - yy);
    B[14] = K[14] * z * (xx - yy);
    B[15] = K[15] * x * (xx - 3.0 * yy);
}

void orc_sh_basis64(const double* dirs, int64_t n, int d, double* out)
{
    init_constants();
    for (int64_t i = 0; i < n; ++i)
        sh_basis64(dirs[3 * i], dirs[3 * i + 1], dirs[3 * i + 2], d, out + i * d);
}

/* ----------------------------------------------------------------------------
 * Scene, per-(Gaussian, view) records.
 * ------------------------------------------------------------------------- */
typedef struct {
    int culled;
    float mx, my;        /* projected centre, pixels: the float32 nearest to the float64 centre */
    float mx_lo, my_lo;  /* the float64 centre minus (mx, my), rounded to float32 */
    float s1, s2, s3;    /* G = 2^-((s1 dx + s2 dy)^2 + (s3 dy)^2) */
    int clip[2];         /* field-of-view clamp of the Jacobian active in x, y */
    float opac;
    float pre[3];        /* SH colour + 0.5 before the clamp */
    float col[3];        /* clamped colour */
    int clamp_ok[3];     /* 1 where 0 <= pre <= FLT_MAX (clamp inactive) */
    int comp_ok;         /* antialiased mode: undilated 2D covariance determinant > 0 */
    float depth;
    float radius;
    int rect[4];         /* x0, y0, x1, y1 in tiles, half-open */
} rec32;

typedef struct {
    double mx, my;       /* projected centre */
    double ca, cb, cc;   /* conic */
    double opac;         /* opacity used in alpha (compensated in antialiased mode) */
    double opac_raw;     /* the Gaussian's opacity o */
    double comp;         /* antialiased mode: sqrt(det S2 / det(S2 + 0.3 I)), else 1 */
    double col[3];       /* colour value with the float32 clamp decision frozen */
    double J[6];         /* d(pixel)/d(mean), unclamped, row-major 2x3 */
    double B[16];        /* SH basis at the view direction */
} rec64;

typedef struct {
    int G, d, V, W, H, TX, TY;
    int antialiased;     /* opacity-compensated 2D filter (see project32) */
    float near_plane, far_plane;
    double bg[3];
    float* means;  /* [G,3] */
    float* quats;  /* [G,4] */
    float* scales; /* [G,3] */
    float* opac;   /* [G] */
    float* sh;     /* [G,d,3] */
    double* sh64;  /* [G,d,3] value copy (finite-difference probes edit it) */
    double* p64;   /* [G,11] value copies of mean (3), quaternion (4), scale (3), opacity (1) */
    float* cams;   /* [V,16] */
    rec32* r32;    /* [V*G] */
    rec64* r64;    /* [V*G] */
    rec64* r64_base;
    /* tile lists */
    int64_t* starts; /* [V*T+1] */
    int32_t* ids;    /* [P] */
    int64_t n_pairs;
    /* score accumulation for selected Gaussians */
    int32_t* slot;   /* [G], -1 if not selected */
    int n_sel;
    int32_t* sel;    /* [n_sel] gids */
    double* acc;     /* [n_sel][V][NACC] */
} scene;

#define NACC_FIXED 8   /* W, Aa, Amu_x, Amu_y, |Aa|, |Amu_x|, |Amu_y|, n_pix */
#define NACC_SENS 9    /* sensitivity sums, after the SH sums (see orc_render_tiles) */
static int nacc(const scene* s) { return NACC_FIXED + 6 * s->d + NACC_SENS; } /* + ASH[d][3] + |ASH|[d][3] + sens */

/* The decision record of one (Gaussian, view) -- the written specification the
 * GPU preprocess implements independently:
 *  - geometry in float64 from the float32 inputs, every operation rounded once
 *    in the order written (no fused multiply-adds): camera-space centre, the
 *    quaternion's rotation (R(q) of the unnormalised quaternion scaled by
 *    2 / |q|^2, which equals the rotation of q / |q|), M = R(q) diag(s),
 *    Sigma3 = M M^T, Sigma_cam = R_v Sigma3 R_v^T, the perspective Jacobian at
 *    the centre clamped to 1.3x the half field of view (with 1/t_z taken once:
 *    u = t_x (1/t_z), j00 = f_x (1/t_z), j02 = -(f_x u_c) (1/t_z)), the dilated 2D
 *    covariance [[a, b], [b, c]] and its determinant, the projected centre;
 *  - the 2D covariance and determinant rounded to float32, then in float32
 *    (correctly rounded division and square root): the 3-sigma radius, the
 *    exponent factors s1 = sqrt(k c / det), s2 = -((k b) / det) / s1,
 *    s3 = sqrt(k / c) with k = RN(log2(e) / 2), so that the exponent at offset
 *    (dx, dy) is -((s1 dx + s2 dy)^2 + (s3 dy)^2) = -k (dx, dy) Sigma2^-1 (dx, dy)^T
 *    without the cancellation of the expanded quadratic form;
 *  - the centre as a float32 pair hi + lo (hi = RN(mx), lo = RN(mx - hi)): the
 *    rectangle is taken from hi, and evaluation uses the centre relative to the
 *    tile, (hi - 16 tx) + lo, so that pixel offsets keep their precision far
 *    from the image origin;
 *  - the SH colour in float32 as before. */
static void project32(const scene* s, int g, int v, rec32* r)
{
    const float* mu = s->means + 3 * (int64_t)g;
    const float* qi = s->quats + 4 * (int64_t)g;
    const float* sc = s->scales + 3 * (int64_t)g;
    const float op = s->opac[g];
    const float* sh = s->sh + (int64_t)g * s->d * 3;
    const float* cam = s->cams + 16 * v;
    const float* R = cam;
    const float* t = cam + 9;
    const float fx = cam[12], fy = cam[13], cx = cam[14], cy = cam[15];

    memset(r, 0, sizeof *r);
    r->culled = 1;
    double Rd[9];
    for (int i = 0; i < 9; ++i) Rd[i] = R[i];
    const double m0 = mu[0], m1 = mu[1], m2 = mu[2];
    const double tx = ((Rd[0] * m0 + Rd[1] * m1) + Rd[2] * m2) + (double)t[0];
    const double ty = ((Rd[3] * m0 + Rd[4] * m1) + Rd[5] * m2) + (double)t[1];
    const double tz = ((Rd[6] * m0 + Rd[7] * m1) + Rd[8] * m2) + (double)t[2];
    if (!(tz >= (double)s->near_plane) || !(tz <= (double)s->far_plane)) return;
    if (!(op >= 0.0f) || !(op <= 1.0f)) return;

    const double w = qi[0], x = qi[1], y = qi[2], z = qi[3];
    const double n2 = ((w * w + x * x) + y * y) + z * z;
    if (!(n2 > 0.0) || !(n2 <= DBL_MAX)) return;
    const double q2 = 2.0 / n2;
    double Rq[9];
    Rq[0] = 1.0 - q2 * (y * y + z * z);
    Rq[1] = q2 * (x * y - w * z);
    Rq[2] = q2 * (x * z + w * y);
    Rq[3] = q2 * (x * y + w * z);
    Rq[4] = 1.0 - q2 * (x * x + z * z);
    Rq[5] = q2 * (y * z - w * x);
    Rq[6] = q2 * (x * z - w * y);
    Rq[7] = q2 * (y * z + w * x);
    Rq[8] = 1.0 - q2 * (x * x + y * y);
    double M[9];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) M[3 * i + j] = Rq[3 * i + j] * (double)sc[j];
    double S3[9];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            S3[3 * i + j] = (M[3 * i] * M[3 * j] + M[3 * i + 1] * M[3 * j + 1]) + M[3 * i + 2] * M[3 * j + 2];
    double Tm[9], Cc[9];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            Tm[3 * i + j] = (Rd[3 * i] * S3[j] + Rd[3 * i + 1] * S3[3 + j]) + Rd[3 * i + 2] * S3[6 + j];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            Cc[3 * i + j] = (Tm[3 * i] * Rd[3 * j] + Tm[3 * i + 1] * Rd[3 * j + 1]) + Tm[3 * i + 2] * Rd[3 * j + 2];

    /* field-of-view clamp of the Jacobian's lateral offset (decision shared with the backward) */
    const double limx = FOV_CLAMP_D * ((0.5 * (double)s->W) / (double)fx);
    const double limy = FOV_CLAMP_D * ((0.5 * (double)s->H) / (double)fy);
    const double iz = 1.0 / tz;
    const double ux = tx * iz, uy = ty * iz;
    r->clip[0] = ux < -limx || ux > limx;
    r->clip[1] = uy < -limy || uy > limy;
    const double uxc = ux < -limx ? -limx : (ux > limx ? limx : ux);
    const double uyc = uy < -limy ? -limy : (uy > limy ? limy : uy);
    const double j00 = (double)fx * iz, j02 = -((double)fx * uxc) * iz;
    const double j11 = (double)fy * iz, j12 = -((double)fy * uyc) * iz;
    const double u00 = j00 * Cc[0] + j02 * Cc[6];
    const double u01 = j00 * Cc[1] + j02 * Cc[7];
    const double u02 = j00 * Cc[2] + j02 * Cc[8];
    const double u11 = j11 * Cc[4] + j12 * Cc[7];
    const double u12 = j11 * Cc[5] + j12 * Cc[8];
    const double ar = u00 * j00 + u02 * j02, cr = u11 * j11 + u12 * j12;
    const double a = ar + DILATION_D;
    const double b = u01 * j11 + u02 * j12;
    const double c = cr + DILATION_D;
    const double det = a * c - b * b;
    if (!(det > 0.0) || !(det <= DBL_MAX) || !(a <= DBL_MAX) || !(c <= DBL_MAX)) return;
    const float a32 = (float)a, b32 = (float)b, c32 = (float)c, d32 = (float)det;
    if (!(d32 > 0.0f) || !(d32 <= FLT_MAX) || !(a32 <= FLT_MAX) || !(c32 <= FLT_MAX)) return;
    /* antialiased mode: the 0.3 px^2 dilation widens the footprint, so opacity is
     * scaled by sqrt(det of the undilated 2D covariance / det of the dilated one),
     * which keeps the integrated weight and depends on depth through the
     * projected covariance (the depth-dependent antialiasing the Proposal's mean
     * score stops gradient through) */
    float opx = op;
    if (s->antialiased) {
        const double det_r = ar * cr - b * b;
        r->comp_ok = det_r > 0.0;
        opx = op * (r->comp_ok ? sqrtf((float)(det_r / det)) : 0.0f);
    }
    /* 3-sigma radius (float32) */
    const float mid = 0.5f * (a32 + c32);
    const float disc = mid * mid - d32;
    const float lam = mid + sqrtf(disc > EIG_FLOOR_F ? disc : EIG_FLOOR_F);
    const float rad = ceilf(3.0f * sqrtf(lam));
    /* projected centre: float64, kept as hi + lo */
    const double mx = (double)fx * ux + (double)cx;
    const double my = (double)fy * uy + (double)cy;
    const float hx = (float)mx, hy = (float)my;
    const float lx = (float)(mx - (double)hx), ly = (float)(my - (double)hy);

    const float fx0 = (hx - rad) * 0.0625f, fx1 = ((hx + rad) + 15.0f) * 0.0625f;
    const float fy0 = (hy - rad) * 0.0625f, fy1 = ((hy + rad) + 15.0f) * 0.0625f;
#define CLAMP_TILE(f, n) (!((f) > 0.0f) ? 0 : ((f) >= (float)(n) ? (n) : (int)(f)))
    int x0 = CLAMP_TILE(fx0, s->TX), x1 = CLAMP_TILE(fx1, s->TX);
    int y0 = CLAMP_TILE(fy0, s->TY), y1 = CLAMP_TILE(fy1, s->TY);
#undef CLAMP_TILE
    if (x1 <= x0 || y1 <= y0) return;

    /* exponent factors (float32) */
    const float s3 = sqrtf(g_hl2e / c32);
    const float s1 = sqrtf((g_hl2e * c32) / d32);
    const float s2 = -((g_hl2e * b32) / d32) / s1;

    /* view direction from the camera centre -R^T t (float32) */
    float ccx = -((R[0] * t[0] + R[3] * t[1]) + R[6] * t[2]);
    float ccy = -((R[1] * t[0] + R[4] * t[1]) + R[7] * t[2]);
    float ccz = -((R[2] * t[0] + R[5] * t[1]) + R[8] * t[2]);
    float dx = mu[0] - ccx, dy = mu[1] - ccy, dz = mu[2] - ccz;
    float len = sqrtf((dx * dx + dy * dy) + dz * dz);
    float il = 1.0f / len;
    float B[16];
    sh_basis32(dx * il, dy * il, dz * il, s->d, B);
    for (int ch = 0; ch < 3; ++ch) {
        float acc = B[0] * sh[ch];
        for (int k = 1; k < s->d; ++k) acc = fmaf(B[k], sh[3 * k + ch], acc);
        float pre = acc + 0.5f;
        r->pre[ch] = pre;
        /* the colour clamp: negative or non-finite colours are clamped to 0 and masked */
        r->clamp_ok[ch] = pre >= 0.0f && pre <= FLT_MAX;
        r->col[ch] = r->clamp_ok[ch] ? pre : 0.0f;
    }
    r->culled = 0;
    r->mx = hx;
    r->my = hy;
    r->mx_lo = lx;
    r->my_lo = ly;
    r->s1 = s1;
    r->s2 = s2;
    r->s3 = s3;
    r->opac = opx;
    r->depth = (float)tz;
    r->radius = rad;
    r->rect[0] = x0;
    r->rect[1] = y0;
    r->rect[2] = x1;
    r->rect[3] = y1;
}

/* float64 values of one (Gaussian, view): same formulas as above, no rounding to float32 */
static void params64_from_inputs(scene* s)
{
    for (int64_t g = 0; g < s->G; ++g) {
        double* prm = s->p64 + 11 * g;
        for (int i = 0; i < 3; ++i) prm[i] = s->means[3 * g + i];
        for (int i = 0; i < 4; ++i) prm[3 + i] = s->quats[4 * g + i];
        for (int i = 0; i < 3; ++i) prm[7 + i] = s->scales[3 * g + i];
        prm[10] = s->opac[g];
    }
}

/* Every float64 intermediate of one (Gaussian, view) projection, kept for the
 * backward: EWA splatting of the 3D covariance R_q S S^T R_q^T through the
 * camera rotation and the perspective Jacobian (evaluated at the centre
 * clamped to 1.3x the half field of view), plus the 0.3 px^2 dilation. */
typedef struct {
    double R[9], t[3], fx, fy, cx, cy;
    double tc[3];          /* camera-space centre */
    double qn, qh[4];      /* quaternion norm and the normalised quaternion (w, x, y, z) */
    double Rq[9], sc[3];   /* rotation of the quaternion, axis scales */
    double M[9];           /* Rq diag(sc) */
    double S3[9], Cc[9];   /* world and camera covariance */
    double uxc, uyc;       /* clamped tan-space centre */
    int clip_x, clip_y;    /* 1 where that clamp is active */
    double Jc[6];          /* perspective Jacobian at the clamped centre, 2x3 row-major */
    double a, b, c, det;   /* dilated 2D covariance [[a, b], [b, c]] and its determinant */
    double ar, cr;         /* undilated diagonal entries (a - 0.3, c - 0.3 before rounding) */
    double dir[3], len;    /* unit view direction from the camera centre, distance */
} fwd64;

static void forward64(const scene* s, int g, int v, fwd64* f)
{
    const double* prm = s->p64 + 11 * (int64_t)g;
    const double* mu = prm;      /* value copies (float32 inputs unless a probe moved them) */
    const double* qi = prm + 3;
    const float* cam = s->cams + 16 * v;
    for (int i = 0; i < 9; ++i) f->R[i] = cam[i];
    for (int i = 0; i < 3; ++i) f->t[i] = cam[9 + i];
    f->fx = cam[12];
    f->fy = cam[13];
    f->cx = cam[14];
    f->cy = cam[15];
    const double* R = f->R;
    for (int i = 0; i < 3; ++i)
        f->tc[i] = R[3 * i] * mu[0] + R[3 * i + 1] * mu[1] + R[3 * i + 2] * mu[2] + f->t[i];
    const double tx = f->tc[0], ty = f->tc[1], tz = f->tc[2];

    f->qn = sqrt(qi[0] * qi[0] + qi[1] * qi[1] + qi[2] * qi[2] + qi[3] * qi[3]);
    for (int i = 0; i < 4; ++i) f->qh[i] = qi[i] / f->qn;
    const double w = f->qh[0], x = f->qh[1], y = f->qh[2], z = f->qh[3];
    double* Rq = f->Rq;
    Rq[0] = 1 - 2 * (y * y + z * z);
    Rq[1] = 2 * (x * y - w * z);
    Rq[2] = 2 * (x * z + w * y);
    Rq[3] = 2 * (x * y + w * z);
    Rq[4] = 1 - 2 * (x * x + z * z);
    Rq[5] = 2 * (y * z - w * x);
    Rq[6] = 2 * (x * z - w * y);
    Rq[7] = 2 * (y * z + w * x);
    Rq[8] = 1 - 2 * (x * x + y * y);
    for (int k = 0; k < 3; ++k) f->sc[k] = prm[7 + k];
    for (int i = 0; i < 3; ++i)
        for (int k = 0; k < 3; ++k) f->M[3 * i + k] = Rq[3 * i + k] * f->sc[k];
    double Tm[9];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            double acc = 0;
            for (int k = 0; k < 3; ++k) acc += Rq[3 * i + k] * f->sc[k] * Rq[3 * j + k] * f->sc[k];
            f->S3[3 * i + j] = acc;
        }
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            double acc = 0;
            for (int k = 0; k < 3; ++k) acc += R[3 * i + k] * f->S3[3 * k + j];
            Tm[3 * i + j] = acc;
        }
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            double acc = 0;
            for (int k = 0; k < 3; ++k) acc += Tm[3 * i + k] * R[3 * j + k];
            f->Cc[3 * i + j] = acc;
        }
    const double limx = 1.3 * (0.5 * s->W / f->fx), limy = 1.3 * (0.5 * s->H / f->fy);
    const double ux = tx / tz, uy = ty / tz;
    /* the clamp state is the record's decision, frozen (it equals this test at the unperturbed inputs:
     * the same float64 operations) */
    const rec32* r32 = &s->r32[(int64_t)v * s->G + g];
    f->clip_x = r32->clip[0];
    f->clip_y = r32->clip[1];
    f->uxc = f->clip_x ? (ux < 0.0 ? -limx : limx) : ux;
    f->uyc = f->clip_y ? (uy < 0.0 ? -limy : limy) : uy;
    double* Jc = f->Jc;
    Jc[0] = f->fx / tz;
    Jc[1] = 0;
    Jc[2] = -f->fx * f->uxc / tz;
    Jc[3] = 0;
    Jc[4] = f->fy / tz;
    Jc[5] = -f->fy * f->uyc / tz;
    double S2[4] = {0, 0, 0, 0};
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) {
            double acc = 0;
            for (int k = 0; k < 3; ++k)
                for (int l = 0; l < 3; ++l) acc += Jc[3 * i + k] * f->Cc[3 * k + l] * Jc[3 * j + l];
            S2[2 * i + j] = acc;
        }
    f->ar = S2[0];
    f->cr = S2[3];
    f->a = S2[0] + 0.3;
    f->b = 0.5 * (S2[1] + S2[2]);
    f->c = S2[3] + 0.3;
    f->det = f->a * f->c - f->b * f->b;
    double cc3[3];
    for (int j = 0; j < 3; ++j) cc3[j] = -(R[j] * f->t[0] + R[3 + j] * f->t[1] + R[6 + j] * f->t[2]);
    double dv[3] = {mu[0] - cc3[0], mu[1] - cc3[1], mu[2] - cc3[2]};
    f->len = sqrt(dv[0] * dv[0] + dv[1] * dv[1] + dv[2] * dv[2]);
    for (int j = 0; j < 3; ++j) f->dir[j] = dv[j] / f->len;
}

static void project64(const scene* s, int g, int v, const rec32* r32, rec64* r)
{
    memset(r, 0, sizeof *r);
    const double* sh = s->sh64 + (int64_t)g * s->d * 3;
    r->opac_raw = s->p64[11 * (int64_t)g + 10];
    r->opac = r->opac_raw;
    r->comp = 1.0;
    if (r32->culled) return;
    fwd64 f;
    forward64(s, g, v, &f);
    if (s->antialiased) {
        r->comp = r32->comp_ok ? sqrt((f.ar * f.cr - f.b * f.b) / f.det) : 0.0;
        r->opac = r->opac_raw * r->comp;
    }
    const double tx = f.tc[0], ty = f.tc[1], tz = f.tc[2];
    r->ca = f.c / f.det;
    r->cb = -f.b / f.det;
    r->cc = f.a / f.det;
    r->mx = f.fx * tx / tz + f.cx;
    r->my = f.fy * ty / tz + f.cy;
    /* unclamped pixel-projection Jacobian d pi / d mu = Jp(t) R */
    double Jp[6] = {f.fx / tz, 0, -f.fx * tx / (tz * tz), 0, f.fy / tz, -f.fy * ty / (tz * tz)};
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 3; ++j) {
            double acc = 0;
            for (int k = 0; k < 3; ++k) acc += Jp[3 * i + k] * f.R[3 * k + j];
            r->J[3 * i + j] = acc;
        }
    sh_basis64(f.dir[0], f.dir[1], f.dir[2], s->d, r->B);
    for (int ch = 0; ch < 3; ++ch) {
        double acc = 0.5;
        for (int k = 0; k < s->d; ++k) acc += r->B[k] * sh[3 * k + ch];
        r->col[ch] = r32->clamp_ok[ch] ? acc : 0.0;
    }
}

void* orc_scene_new(int G, int sh_degree, const float* means, const float* quats, const float* scales,
                    const float* opac, const float* sh, int V, const float* cams, int W, int H,
                    float near_plane, float far_plane, const float* bg, int antialiased)
{
    init_constants();
    if (G < 0 || V <= 0 || W <= 0 || H <= 0 || sh_degree < 0 || sh_degree > 3) return NULL;
    scene* s = (scene*)calloc(1, sizeof(scene));
    s->G = G;
    s->d = (sh_degree + 1) * (sh_degree + 1);
    s->V = V;
    s->W = W;
    s->H = H;
    s->TX = (W + TILE - 1) / TILE;
    s->TY = (H + TILE - 1) / TILE;
    s->near_plane = near_plane;
    s->far_plane = far_plane;
    s->antialiased = antialiased != 0;
    for (int i = 0; i < 3; ++i) s->bg[i] = bg[i];
    size_t Gs = (size_t)G;
    s->means = (float*)malloc(sizeof(float) * 3 * Gs + 1);
    s->quats = (float*)malloc(sizeof(float) * 4 * Gs + 1);
    s->scales = (float*)malloc(sizeof(float) * 3 * Gs + 1);
    s->opac = (float*)malloc(sizeof(float) * Gs + 1);
    s->sh = (float*)malloc(sizeof(float) * 3 * s->d * Gs + 1);
    s->sh64 = (double*)malloc(sizeof(double) * 3 * s->d * Gs + 1);
    s->p64 = (double*)malloc(sizeof(double) * 11 * Gs + 1);
    s->cams = (float*)malloc(sizeof(float) * 16 * V);
    memcpy(s->means, means, sizeof(float) * 3 * Gs);
    memcpy(s->quats, quats, sizeof(float) * 4 * Gs);
    memcpy(s->scales, scales, sizeof(float) * 3 * Gs);
    memcpy(s->opac, opac, sizeof(float) * Gs);
    memcpy(s->sh, sh, sizeof(float) * 3 * s->d * Gs);
    for (size_t i = 0; i < 3 * s->d * Gs; ++i) s->sh64[i] = sh[i];
    params64_from_inputs(s);
    memcpy(s->cams, cams, sizeof(float) * 16 * V);
    size_t VG = (size_t)V * Gs;
    s->r32 = (rec32*)malloc(sizeof(rec32) * VG + 1);
    s->r64 = (rec64*)malloc(sizeof(rec64) * VG + 1);
    s->r64_base = (rec64*)malloc(sizeof(rec64) * VG + 1);
    s->slot = (int32_t*)malloc(sizeof(int32_t) * Gs + 1);
    for (size_t i = 0; i < Gs; ++i) s->slot[i] = -1;
#pragma omp parallel for schedule(dynamic, 256)
    for (int64_t i = 0; i < (int64_t)VG; ++i) {
        int v = (int)(i / G), g = (int)(i % G);
        project32(s, g, v, &s->r32[i]);
        project64(s, g, v, &s->r32[i], &s->r64[i]);
    }
    memcpy(s->r64_base, s->r64, sizeof(rec64) * VG);
    return s;
}

void orc_scene_free(void* p)
{
    scene* s = (scene*)p;
    if (!s) return;
    free(s->means); free(s->quats); free(s->scales); free(s->opac); free(s->sh); free(s->sh64); free(s->p64);
    free(s->cams); free(s->r32); free(s->r64); free(s->r64_base); free(s->starts); free(s->ids);
    free(s->slot); free(s->sel); free(s->acc);
    free(s);
}

/* Export the float32 records: per (v, g) 20 floats
 * [culled, mx, my, mx_lo, my_lo, s1, s2, s3, clip bits (x | y << 1), opac, pre r, g, b, depth, radius,
 *  x0, y0, x1, y1, clamp bits] */
void orc_get_records32(const void* p, float* out)
{
    const scene* s = (const scene*)p;
    int64_t VG = (int64_t)s->V * s->G;
    for (int64_t i = 0; i < VG; ++i) {
        const rec32* r = &s->r32[i];
        float* o = out + 20 * i;
        o[0] = (float)r->culled;
        o[1] = r->mx; o[2] = r->my;
        o[3] = r->mx_lo; o[4] = r->my_lo;
        o[5] = r->s1; o[6] = r->s2; o[7] = r->s3;
        o[8] = (float)(r->clip[0] | (r->clip[1] << 1));
        o[9] = r->opac;
        o[10] = r->pre[0]; o[11] = r->pre[1]; o[12] = r->pre[2];
        o[13] = r->depth; o[14] = r->radius;
        o[15] = (float)r->rect[0]; o[16] = (float)r->rect[1];
        o[17] = (float)r->rect[2]; o[18] = (float)r->rect[3];
        o[19] = (float)(r->clamp_ok[0] | (r->clamp_ok[1] << 1) | (r->clamp_ok[2] << 2));
    }
}

/* Export float64 values: per (v, g) 12 doubles [mx, my, ca, cb, cc, opac, col r, g, b, J...] -> 6 + 3 + 6 = 15 */
void orc_get_records64(const void* p, double* out)
{
    const scene* s = (const scene*)p;
    int64_t VG = (int64_t)s->V * s->G;
    for (int64_t i = 0; i < VG; ++i) {
        const rec64* r = &s->r64[i];
        double* o = out + 15 * i;
        o[0] = r->mx; o[1] = r->my; o[2] = r->ca; o[3] = r->cb; o[4] = r->cc; o[5] = r->opac;
        o[6] = r->col[0]; o[7] = r->col[1]; o[8] = r->col[2];
        for (int k = 0; k < 6; ++k) o[9 + k] = r->J[k];
    }
}

/* ----------------------------------------------------------------------------
 * Candidate lists per tile, brute force, ordered by (depth bits, Gaussian id).
 * ------------------------------------------------------------------------- */
static uint32_t fbits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

static int cmp_u64(const void* a, const void* b)
{
    uint64_t x = *(const uint64_t*)a, y = *(const uint64_t*)b;
    return x < y ? -1 : (x > y ? 1 : 0);
}

int64_t orc_build_lists(void* p)
{
    scene* s = (scene*)p;
    int T = s->TX * s->TY;
    int64_t nt = (int64_t)s->V * T;
    int64_t* count = (int64_t*)calloc((size_t)nt + 1, sizeof(int64_t));
    for (int v = 0; v < s->V; ++v)
        for (int g = 0; g < s->G; ++g) {
            const rec32* r = &s->r32[(int64_t)v * s->G + g];
            if (r->culled) continue;
            for (int ty = r->rect[1]; ty < r->rect[3]; ++ty)
                for (int tx = r->rect[0]; tx < r->rect[2]; ++tx) count[(int64_t)v * T + ty * s->TX + tx]++;
        }
    free(s->starts);
    free(s->ids);
    s->starts = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nt + 1));
    s->starts[0] = 0;
    for (int64_t i = 0; i < nt; ++i) s->starts[i + 1] = s->starts[i] + count[i];
    s->n_pairs = s->starts[nt];
    uint64_t* keys = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)s->n_pairs + 1);
    int64_t* fill = count;
    for (int64_t i = 0; i < nt; ++i) fill[i] = s->starts[i];
    for (int v = 0; v < s->V; ++v)
        for (int g = 0; g < s->G; ++g) {
            const rec32* r = &s->r32[(int64_t)v * s->G + g];
            if (r->culled) continue;
            uint64_t key = ((uint64_t)fbits(r->depth) << 32) | (uint32_t)g;
            for (int ty = r->rect[1]; ty < r->rect[3]; ++ty)
                for (int tx = r->rect[0]; tx < r->rect[2]; ++tx) keys[fill[(int64_t)v * T + ty * s->TX + tx]++] = key;
        }
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < nt; ++i)
        qsort(keys + s->starts[i], (size_t)(s->starts[i + 1] - s->starts[i]), sizeof(uint64_t), cmp_u64);
    s->ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)s->n_pairs + 1);
    for (int64_t i = 0; i < s->n_pairs; ++i) s->ids[i] = (int32_t)(keys[i] & 0xffffffffu);
    free(keys);
    free(count);
    return s->n_pairs;
}

void orc_get_lists(const void* p, int64_t* starts, int32_t* ids)
{
    const scene* s = (const scene*)p;
    int64_t nt = (int64_t)s->V * s->TX * s->TY;
    memcpy(starts, s->starts, sizeof(int64_t) * (size_t)(nt + 1));
    memcpy(ids, s->ids, sizeof(int32_t) * (size_t)s->n_pairs);
}

/* One tile's list by scanning every Gaussian of the view (used to pin orc_build_lists). */
int64_t orc_tile_list_scan(const void* p, int64_t tile, int32_t* out)
{
    const scene* s = (const scene*)p;
    int T = s->TX * s->TY;
    int v = (int)(tile / T), t = (int)(tile % T);
    int tx = t % s->TX, ty = t / s->TX;
    int64_t n = 0;
    uint64_t* keys = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)s->G + 1);
    for (int g = 0; g < s->G; ++g) {
        const rec32* r = &s->r32[(int64_t)v * s->G + g];
        if (r->culled) continue;
        if (tx >= r->rect[0] && tx < r->rect[2] && ty >= r->rect[1] && ty < r->rect[3])
            keys[n++] = ((uint64_t)fbits(r->depth) << 32) | (uint32_t)g;
    }
    qsort(keys, (size_t)n, sizeof(uint64_t), cmp_u64);
    for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)(keys[i] & 0xffffffffu);
    free(keys);
    return n;
}

/* ----------------------------------------------------------------------------
 * Per-pixel front-to-back composite, back-to-front suffix, literal score sums.
 * ------------------------------------------------------------------------- */
typedef struct {
    int g;
    double alpha, T, G;  /* float64 values */
    float tT32;          /* float32 transmittance after this contribution */
    int clamped;         /* alpha clamp active (o G >= 0.99 in float32) */
} contrib;

void orc_select(void* p, const int32_t* gids, int n)
{
    scene* s = (scene*)p;
    for (int g = 0; g < s->G; ++g) s->slot[g] = -1;
    free(s->sel);
    free(s->acc);
    if (n < 0) { /* all */
        n = s->G;
        s->sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)n + 1);
        for (int g = 0; g < n; ++g) s->sel[g] = g;
    } else {
        s->sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)n + 1);
        memcpy(s->sel, gids, sizeof(int32_t) * (size_t)n);
    }
    s->n_sel = n;
    for (int i = 0; i < n; ++i) s->slot[s->sel[i]] = i;
    s->acc = (double*)calloc((size_t)n * s->V * nacc(s) + 1, sizeof(double));
}

static void add(double* a, double x)
{
#pragma omp atomic
    *a += x;
}

/* Stage 1 for one pixel (x, y) of view v over its tile list: float32 decisions
 * (distance cut, alpha clamp and floor, transmittance stop), float64 values.
 * Fills the accepted contributions in front-to-back order and returns their
 * count; C gets the colour including the background. */
/* Front-to-back composite of one pixel over its tile's list.  With work != NULL
 * it also counts the pass's work: work[0] = list entries examined up to and
 * including the one at which the pixel stopped (the whole list if it never
 * did), work[1] = those of them past the distance cut. */
static int composite_pixel_counted(const scene* s, int v, int x, int y, const int32_t* list, int64_t L,
                                   contrib* cl, double C[3], float* T32_out, double* T64_out, uint32_t work[2])
{
    /* float32 decisions at tile-relative coordinates: the pixel centre (x - 16 tx) + 1/2 and
     * the entry's centre (mx - 16 tx) + mx_lo, likewise in y */
    const int tx = x / TILE, ty = y / TILE;
    const float tox = (float)(TILE * tx), toy = (float)(TILE * ty);
    const float pxl = (float)(x - TILE * tx) + 0.5f, pyl = (float)(y - TILE * ty) + 0.5f;
    double pxd = x + 0.5, pyd = y + 0.5;
    float T32 = 1.0f;
    double T64 = 1.0;
    int n = 0;
    C[0] = C[1] = C[2] = 0.0;
    for (int64_t k = 0; k < L; ++k) {
        int g = list[k];
        const rec32* r = &s->r32[(int64_t)v * s->G + g];
        float mxt = (r->mx - tox) + r->mx_lo, myt = (r->my - toy) + r->my_lo;
        float dx = pxl - mxt, dy = pyl - myt;
        float u = fmaf(r->s1, dx, r->s2 * dy), w = r->s3 * dy;
        float S = fmaf(u, u, w * w);
        if (work) work[0] = (uint32_t)(k + 1);
        if (!(S <= S_CUTOFF_F)) continue;
        if (work) work[1]++;
        float aG = r->opac * orc_exp2f(-S);
        int clamped = !(aG < ALPHA_MAX_F);
        float a32 = clamped ? ALPHA_MAX_F : aG;
        if (!(a32 >= g_alpha_min)) continue;
        float tT = T32 * (1.0f - a32);
        if (tT < T_MIN_F) break;
        const rec64* q = &s->r64[(int64_t)v * s->G + g];
        double ddx = pxd - q->mx, ddy = pyd - q->my;
        double sig = 0.5 * (q->ca * ddx * ddx + 2.0 * q->cb * ddx * ddy + q->cc * ddy * ddy);
        double G64 = exp(-sig);
        double a64 = clamped ? ALPHA_MAX_D : q->opac * G64;
        for (int ch = 0; ch < 3; ++ch) C[ch] += q->col[ch] * a64 * T64;
        cl[n].g = g;
        cl[n].alpha = a64;
        cl[n].T = T64;
        cl[n].G = G64;
        cl[n].tT32 = tT;
        cl[n].clamped = clamped;
        n++;
        T64 = T64 * (1.0 - a64);
        T32 = tT;
    }
    for (int ch = 0; ch < 3; ++ch) C[ch] += T64 * s->bg[ch];
    *T32_out = T32;
    *T64_out = T64;
    return n;
}

static int composite_pixel(const scene* s, int v, int x, int y, const int32_t* list, int64_t L, contrib* cl,
                           double C[3], float* T32_out, double* T64_out)
{
    return composite_pixel_counted(s, v, x, y, list, L, cl, C, T32_out, T64_out, NULL);
}

/* Work counts of the render pass for every pixel of the given tiles, written at
 * out[2 * pix] (entries examined until the pixel stopped) and out[2 * pix + 1]
 * (those past the distance cut). */
void orc_pixel_work(void* p, const int64_t* tiles, int64_t n_tiles, uint32_t* out)
{
    scene* s = (scene*)p;
    const int T = s->TX * s->TY;
    int64_t maxlen = 0;
    for (int64_t i = 0; i < (int64_t)s->V * T; ++i)
        if (s->starts[i + 1] - s->starts[i] > maxlen) maxlen = s->starts[i + 1] - s->starts[i];
#pragma omp parallel
    {
        contrib* cl = (contrib*)malloc(sizeof(contrib) * (size_t)maxlen + 1);
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < n_tiles; ++it) {
            int64_t tile = tiles[it];
            int v = (int)(tile / T), t = (int)(tile % T);
            int tx = t % s->TX, ty = t / s->TX;
            const int32_t* list = s->ids + s->starts[tile];
            int64_t L = s->starts[tile + 1] - s->starts[tile];
            for (int yy = 0; yy < TILE; ++yy)
                for (int xx = 0; xx < TILE; ++xx) {
                    int x = tx * TILE + xx, y = ty * TILE + yy;
                    if (x >= s->W || y >= s->H) continue;
                    double C[3];
                    float T32;
                    double T64;
                    uint32_t work[2] = {0u, 0u};
                    composite_pixel_counted(s, v, x, y, list, L, cl, C, &T32, &T64, work);
                    int64_t pix = ((int64_t)v * s->H + y) * s->W + x;
                    out[2 * pix] = work[0];
                    out[2 * pix + 1] = work[1];
                }
        }
        free(cl);
    }
}

/* Render (and, with obs != NULL, replay) the pixels of the given tiles.
 * Pixel outputs are written at [v, y, x]; score sums accumulate into the selected slots. */
void orc_render_tiles(void* p, const int64_t* tiles, int64_t n_tiles, const float* obs, float eps,
                      float den_min, double* color, float* T_out, int32_t* n_out, double* T64_out)
{
    scene* s = (scene*)p;
    const int T = s->TX * s->TY;
    const int d = s->d;
    const int na = nacc(s);
    int64_t maxlen = 0;
    for (int64_t i = 0; i < (int64_t)s->V * T; ++i)
        if (s->starts[i + 1] - s->starts[i] > maxlen) maxlen = s->starts[i + 1] - s->starts[i];

#pragma omp parallel
    {
        contrib* cl = (contrib*)malloc(sizeof(contrib) * (size_t)maxlen + 1);
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < n_tiles; ++it) {
            int64_t tile = tiles[it];
            int v = (int)(tile / T), t = (int)(tile % T);
            int tx = t % s->TX, ty = t / s->TX;
            const int32_t* list = s->ids + s->starts[tile];
            int64_t L = s->starts[tile + 1] - s->starts[tile];
            for (int yy = 0; yy < TILE; ++yy)
                for (int xx = 0; xx < TILE; ++xx) {
                    int x = tx * TILE + xx, y = ty * TILE + yy;
                    if (x >= s->W || y >= s->H) continue;
                    double pxd = x + 0.5, pyd = y + 0.5;
                    float T32;
                    double T64;
                    double C[3];
                    int n = composite_pixel(s, v, x, y, list, L, cl, C, &T32, &T64);
                    int64_t pix = ((int64_t)v * s->H + y) * s->W + x;
                    if (color) for (int ch = 0; ch < 3; ++ch) color[3 * pix + ch] = C[ch];
                    if (T_out) T_out[pix] = T32;
                    if (n_out) n_out[pix] = n;
                    if (T64_out) T64_out[pix] = T64;
                    if (!obs) continue;

                    /* residual r = C_hat - C_obs */
                    double rr[3];
                    for (int ch = 0; ch < 3; ++ch) rr[ch] = C[ch] - (double)obs[3 * pix + ch];
                    /* Stage 2: explicit back-to-front suffix */
                    double S[3];
                    for (int ch = 0; ch < 3; ++ch) S[ch] = T64 * s->bg[ch];
                    for (int k = n - 1; k >= 0; --k) {
                        const contrib* c = &cl[k];
                        const rec64* q = &s->r64[(int64_t)v * s->G + c->g];
                        double den = c->T * (1.0 - c->alpha) + (double)eps;
                        double Cp[3];
                        int finite = 1;
                        for (int ch = 0; ch < 3; ++ch) {
                            Cp[ch] = S[ch] / den;
                            if (!isfinite(Cp[ch])) finite = 0;
                        }
                        double w = c->T * c->alpha;
                        for (int ch = 0; ch < 3; ++ch) S[ch] += w * q->col[ch];
                        int sl = s->slot[c->g];
                        if (sl < 0) continue;
                        double rho = 0;
                        for (int ch = 0; ch < 3; ++ch) rho += rr[ch] * (q->col[ch] - Cp[ch]);
                        int Ma = !c->clamped && (c->tT32 >= den_min) && finite;
                        double* A = s->acc + ((int64_t)sl * s->V + v) * na;
                        add(&A[0], w);
                        add(&A[7], 1.0);
                        if (Ma) {
                            /* opacity logit: T alpha (1 - o) rho */
                            double ta = c->T * c->alpha * (1.0 - q->opac_raw) * rho;
                            /* projected centre: T o grad G rho, grad G = G conic (p - mu) */
                            double dx = pxd - q->mx, dy = pyd - q->my;
                            double gx = c->G * (q->ca * dx + q->cb * dy);
                            double gy = c->G * (q->cb * dx + q->cc * dy);
                            double tmx = c->T * q->opac * gx * rho;
                            double tmy = c->T * q->opac * gy * rho;
                            add(&A[1], ta);
                            add(&A[2], tmx);
                            add(&A[3], tmy);
                            add(&A[4], fabs(ta));
                            add(&A[5], fabs(tmx));
                            add(&A[6], fabs(tmy));
                        }
                        if (Ma) {
                            /* Sensitivity sums (test diagnostics, not scores): how far each masked score
                             * term can move when the residual moves by at most 1 per channel (weight
                             * |factor| * |c - C+|_1) and when the suffix moves by at most 1 per channel
                             * (weight |factor| * |r|_1 / den), for the opacity and the two centre terms. */
                            double cd = 0, rn = 0;
                            for (int ch = 0; ch < 3; ++ch) {
                                cd += fabs(q->col[ch] - Cp[ch]);
                                rn += fabs(rr[ch]);
                            }
                            double dx = pxd - q->mx, dy = pyd - q->my;
                            double f3[3] = {c->T * c->alpha * (1.0 - q->opac_raw),
                                            c->T * q->opac * c->G * (q->ca * dx + q->cb * dy),
                                            c->T * q->opac * c->G * (q->cb * dx + q->cc * dy)};
                            double* Sx = &A[NACC_FIXED + 6 * d];
                            for (int j = 0; j < 3; ++j) {
                                add(&Sx[j], fabs(f3[j]) * cd);
                                add(&Sx[3 + j], fabs(f3[j]) * rn / den);
                            }
                            /* and when the projected centre moves by at most 1 along each axis: the
                             * magnitudes of the terms' derivatives in (mx, my), summed over both axes
                             * (g = conic (p - mu), dG/dmu = G g, dg_x/dmx = -ca, dg_x/dmy = -cb) */
                            const double gx = q->ca * dx + q->cb * dy, gy = q->cb * dx + q->cc * dy;
                            const double ag = fabs(gx) + fabs(gy), toGr = c->T * q->opac * c->G * fabs(rho);
                            add(&Sx[6], c->T * (1.0 - q->opac_raw) * fabs(rho) * q->opac * c->G * ag);
                            add(&Sx[7], toGr * (fabs(gx) * ag + fabs(q->ca) + fabs(q->cb)));
                            add(&Sx[8], toGr * (fabs(gy) * ag + fabs(q->cb) + fabs(q->cc)));
                        }
                        const rec32* r = &s->r32[(int64_t)v * s->G + c->g];
                        for (int k2 = 0; k2 < d; ++k2)
                            for (int ch = 0; ch < 3; ++ch) {
                                if (!r->clamp_ok[ch]) continue;
                                double tsh = w * q->B[k2] * rr[ch];
                                add(&A[NACC_FIXED + 3 * k2 + ch], tsh);
                                add(&A[NACC_FIXED + 3 * d + 3 * k2 + ch], fabs(tsh));
                            }
                    }
                }
        }
        free(cl);
    }
}

void orc_get_acc(const void* p, double* out)
{
    const scene* s = (const scene*)p;
    memcpy(out, s->acc, sizeof(double) * (size_t)s->n_sel * s->V * nacc(s));
}

/* ----------------------------------------------------------------------------
 * Token: cross-view weights, pullback, conditioning statistics.
 * ------------------------------------------------------------------------- */
/* eigenvalues of a symmetric 3x3 matrix by cyclic Jacobi rotations, descending */
void orc_eig3(const double* Ain, double* ev)
{
    double a[3][3];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) a[i][j] = Ain[3 * i + j];
    for (int sweep = 0; sweep < 64; ++sweep) {
        double off = a[0][1] * a[0][1] + a[0][2] * a[0][2] + a[1][2] * a[1][2];
        double dia = a[0][0] * a[0][0] + a[1][1] * a[1][1] + a[2][2] * a[2][2];
        if (off <= 1e-34 * dia || off == 0.0) break;
        for (int p = 0; p < 2; ++p)
            for (int q = p + 1; q < 3; ++q) {
                if (a[p][q] == 0.0) continue;
                double theta = (a[q][q] - a[p][p]) / (2.0 * a[p][q]);
                double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
                double c = 1.0 / sqrt(t * t + 1.0), sn = t * c;
                for (int k = 0; k < 3; ++k) { /* columns p, q */
                    double akp = a[k][p], akq = a[k][q];
                    a[k][p] = c * akp - sn * akq;
                    a[k][q] = sn * akp + c * akq;
                }
                for (int k = 0; k < 3; ++k) { /* rows p, q */
                    double apk = a[p][k], aqk = a[q][k];
                    a[p][k] = c * apk - sn * aqk;
                    a[q][k] = sn * apk + c * aqk;
                }
            }
    }
    ev[0] = a[0][0];
    ev[1] = a[1][1];
    ev[2] = a[2][2];
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (ev[j] > ev[i]) {
                double tmp = ev[i];
                ev[i] = ev[j];
                ev[j] = tmp;
            }
}

/* tokens [n_sel][9 + 3d] for the selected Gaussians; optional A matrices [n_sel][9] and q [n_sel][V] */
void orc_tokens(const void* p, double eps, double lambda, double* tok, double* Aout, double* qout)
{
    const scene* s = (const scene*)p;
    const int d = s->d, V = s->V, na = nacc(s);
    const int D = 9 + 3 * d;
#pragma omp parallel for schedule(dynamic, 64)
    for (int i = 0; i < s->n_sel; ++i) {
        int g = s->sel[i];
        const double* acc = s->acc + (int64_t)i * V * na;
        double Q = eps;
        for (int v = 0; v < V; ++v) Q += eps + acc[v * na + 0];
        double b[3] = {0, 0, 0}, sa = 0, A[9] = {0};
        double* z = tok + (int64_t)i * D;
        for (int k = 0; k < 3 * d; ++k) z[4 + k] = 0.0;
        for (int v = 0; v < V; ++v) {
            const double* a = acc + v * na;
            const rec32* r32 = &s->r32[(int64_t)v * s->G + g];
            const rec64* r64 = &s->r64[(int64_t)v * s->G + g];
            double q = eps + a[0];
            double gamma = q / Q;
            if (qout) qout[(int64_t)i * V + v] = q;
            double J[6] = {0, 0, 0, 0, 0, 0};
            if (!r32->culled)
                for (int k = 0; k < 6; ++k) J[k] = r64->J[k];
            double s_alpha = a[1] / q;
            double s_mu[2] = {a[2] / q, a[3] / q};
            for (int j = 0; j < 3; ++j) b[j] += gamma * (J[j] * s_mu[0] + J[3 + j] * s_mu[1]);
            sa += gamma * s_alpha;
            for (int k = 0; k < 3 * d; ++k) z[4 + k] += gamma * (a[NACC_FIXED + k] / q);
            for (int r = 0; r < 3; ++r)
                for (int c = 0; c < 3; ++c) A[3 * r + c] += gamma * (J[r] * J[c] + J[3 + r] * J[3 + c]);
        }
        for (int r = 0; r < 3; ++r) A[4 * r] += lambda;
        double ev[3];
        orc_eig3(A, ev);
        double tr = A[0] + A[4] + A[8];
        z[0] = b[0];
        z[1] = b[1];
        z[2] = b[2];
        z[3] = sa;
        z[4 + 3 * d] = log(Q);
        for (int k = 0; k < 3; ++k) z[5 + 3 * d + k] = ev[k] / (tr + eps);
        z[8 + 3 * d] = log(tr + eps);
        if (Aout)
            for (int k = 0; k < 9; ++k) Aout[(int64_t)i * 9 + k] = A[k];
    }
}

/* ----------------------------------------------------------------------------
 * Scalar / feature attributes: composite and attribution scatter.
 * The render weight of an accepted contribution is w = T alpha (Stage 1 with
 * float32 decisions, float64 values).  A per-Gaussian attribute vector f_g is
 * composited like the colour (the ATSplat summary page renders its per-anchor
 * uncertainty score this way; ReCoSplat's feature channels are rendered the
 * same way):  F(p) = sum_k w_k f_{g_k} + T_final bg.  The attribution scatter
 * sends a per-pixel map m back along the same weights:
 * a_g = sum_v sum_p w_{p,g,v} m(p) (alphaT scatter for m = 1; the mask-channel
 * gain attribution of L2D2-GS for m = the gain map).
 * ------------------------------------------------------------------------- */
void orc_render_features(void* p, const float* feat, int C, const float* bg, double* out)
{
    scene* s = (scene*)p;
    const int T = s->TX * s->TY;
    int64_t maxlen = 0;
    for (int64_t i = 0; i < (int64_t)s->V * T; ++i)
        if (s->starts[i + 1] - s->starts[i] > maxlen) maxlen = s->starts[i + 1] - s->starts[i];
    const int64_t n_tiles = (int64_t)s->V * T;
#pragma omp parallel
    {
        contrib* cl = (contrib*)malloc(sizeof(contrib) * (size_t)maxlen + 1);
#pragma omp for schedule(dynamic, 1)
        for (int64_t tile = 0; tile < n_tiles; ++tile) {
            int v = (int)(tile / T), t = (int)(tile % T);
            int tx = t % s->TX, ty = t / s->TX;
            const int32_t* list = s->ids + s->starts[tile];
            int64_t L = s->starts[tile + 1] - s->starts[tile];
            for (int yy = 0; yy < TILE; ++yy)
                for (int xx = 0; xx < TILE; ++xx) {
                    int x = tx * TILE + xx, y = ty * TILE + yy;
                    if (x >= s->W || y >= s->H) continue;
                    double Cc[3], T64;
                    float T32;
                    int n = composite_pixel(s, v, x, y, list, L, cl, Cc, &T32, &T64);
                    double* o = out + (((int64_t)v * s->H + y) * s->W + x) * C;
                    for (int c = 0; c < C; ++c) o[c] = T64 * (bg ? (double)bg[c] : 0.0);
                    for (int k = 0; k < n; ++k) {
                        const double w = cl[k].T * cl[k].alpha;
                        const float* f = feat + (int64_t)cl[k].g * C;
                        for (int c = 0; c < C; ++c) o[c] += w * (double)f[c];
                    }
                }
        }
        free(cl);
    }
}

void orc_attribute(void* p, const float* map, int C, double* out /* [G][C], zeroed here */)
{
    scene* s = (scene*)p;
    const int T = s->TX * s->TY;
    int64_t maxlen = 0;
    for (int64_t i = 0; i < (int64_t)s->V * T; ++i)
        if (s->starts[i + 1] - s->starts[i] > maxlen) maxlen = s->starts[i + 1] - s->starts[i];
    for (int64_t i = 0; i < (int64_t)s->G * C; ++i) out[i] = 0.0;
    const int64_t n_tiles = (int64_t)s->V * T;
#pragma omp parallel
    {
        contrib* cl = (contrib*)malloc(sizeof(contrib) * (size_t)maxlen + 1);
#pragma omp for schedule(dynamic, 1)
        for (int64_t tile = 0; tile < n_tiles; ++tile) {
            int v = (int)(tile / T), t = (int)(tile % T);
            int tx = t % s->TX, ty = t / s->TX;
            const int32_t* list = s->ids + s->starts[tile];
            int64_t L = s->starts[tile + 1] - s->starts[tile];
            for (int yy = 0; yy < TILE; ++yy)
                for (int xx = 0; xx < TILE; ++xx) {
                    int x = tx * TILE + xx, y = ty * TILE + yy;
                    if (x >= s->W || y >= s->H) continue;
                    double Cc[3], T64;
                    float T32;
                    int n = composite_pixel(s, v, x, y, list, L, cl, Cc, &T32, &T64);
                    const float* m = map + (((int64_t)v * s->H + y) * s->W + x) * C;
                    for (int k = 0; k < n; ++k) {
                        const double w = cl[k].T * cl[k].alpha;
                        for (int c = 0; c < C; ++c) add(&out[(int64_t)cl[k].g * C + c], w * (double)m[c]);
                    }
                }
        }
        free(cl);
    }
}

/* Debug top-K contributor metadata (the Renderer Score Tokens plan, Block 0:
 * "debug top-K only on small tiles"): per pixel, the K accepted contributions
 * with the largest weight w = T alpha, in decreasing weight; equal weights keep
 * list order; unused entries are id -1, weight 0. */
void orc_topk(void* p, int K, int32_t* ids, double* wts)
{
    scene* s = (scene*)p;
    const int T = s->TX * s->TY;
    int64_t maxlen = 0;
    for (int64_t i = 0; i < (int64_t)s->V * T; ++i)
        if (s->starts[i + 1] - s->starts[i] > maxlen) maxlen = s->starts[i + 1] - s->starts[i];
    const int64_t n_tiles = (int64_t)s->V * T;
#pragma omp parallel
    {
        contrib* cl = (contrib*)malloc(sizeof(contrib) * (size_t)maxlen + 1);
        char* used = (char*)malloc((size_t)maxlen + 1);
#pragma omp for schedule(dynamic, 1)
        for (int64_t tile = 0; tile < n_tiles; ++tile) {
            int v = (int)(tile / T), t = (int)(tile % T);
            int tx = t % s->TX, ty = t / s->TX;
            const int32_t* list = s->ids + s->starts[tile];
            int64_t L = s->starts[tile + 1] - s->starts[tile];
            for (int yy = 0; yy < TILE; ++yy)
                for (int xx = 0; xx < TILE; ++xx) {
                    int x = tx * TILE + xx, y = ty * TILE + yy;
                    if (x >= s->W || y >= s->H) continue;
                    double Cc[3], T64;
                    float T32;
                    int n = composite_pixel(s, v, x, y, list, L, cl, Cc, &T32, &T64);
                    int64_t base = (((int64_t)v * s->H + y) * s->W + x) * K;
                    for (int k = 0; k < n; ++k) used[k] = 0;
                    /* selection: K times the largest unused weight, the earliest on ties */
                    for (int r = 0; r < K; ++r) {
                        int best = -1;
                        for (int k = 0; k < n; ++k) {
                            if (used[k]) continue;
                            if (best < 0 || cl[k].T * cl[k].alpha > cl[best].T * cl[best].alpha) best = k;
                        }
                        if (best < 0) {
                            ids[base + r] = -1;
                            wts[base + r] = 0.0;
                        } else {
                            used[best] = 1;
                            ids[base + r] = cl[best].g;
                            wts[base + r] = cl[best].T * cl[best].alpha;
                        }
                    }
                }
        }
        free(used);
        free(cl);
    }
}

/* ----------------------------------------------------------------------------
 * Renderer backward: the vector-Jacobian product of the colour image with an
 * upstream gradient dL/dC_hat, through the composite, the 2D Gaussian, the EWA
 * projection, the quaternion/scale covariance and the SH colour (view
 * direction included), with the float32 decisions frozen.
 * ------------------------------------------------------------------------- */
#define NB2D 9  /* per (Gaussian, view): dL/dmx, dL/dmy, dL/dca, dL/dcb, dL/dcc, dL/do, dL/dcol[3] */

/* d B_k / d(x, y, z) of the SH polynomials of sh_basis64, (x, y, z) taken as
 * independent variables (the unit-norm constraint is applied by the caller) */
static void sh_basis_grad64(double x, double y, double z, int d, double (*dB)[3])
{
    const double* K = g_sh64;
    for (int k = 0; k < d; ++k) dB[k][0] = dB[k][1] = dB[k][2] = 0.0;
    if (d <= 1) return;
    dB[1][1] = K[1];
    dB[2][2] = K[2];
    dB[3][0] = K[3];
    if (d <= 4) return;
    dB[4][0] = K[4] * y;
    dB[4][1] = K[4] * x;
    dB[5][1] = K[5] * z;
    dB[5][2] = K[5] * y;
    dB[6][0] = -2.0 * K[6] * x;
    dB[6][1] = -2.0 * K[6] * y;
    dB[6][2] = 4.0 * K[6] * z;
    dB[7][0] = K[7] * z;
    dB[7][2] = K[7] * x;
    dB[8][0] = 2.0 * K[8] * x;
    dB[8][1] = -2.0 * K[8] * y;
    if (d <= 9) return;
    double xx = x * x, yy = y * y, zz = z * z;
    dB[9][0] = 6.0 * K[9] * x * y;
    dB[9][1] = K[9] * (3.0 * xx - 3.0 * yy);
    dB[10][0] = K[10] * y * z;
    dB[10][1] = K[10] * x * z;
    dB[10][2] = K[10] * x * y;
    dB[11][0] = -2.0 * K[11] * x * y;
    dB[11][1] = K[11] * (4.0 * zz - xx - 3.0 * yy);
    dB[11][2] = 8.0 * K[11] * y * z;
    dB[12][0] = -6.0 * K[12] * x * z;
    dB[12][1] = -6.0 * K[12] * y * z;
    dB[12][2] = K[12] * (6.0 * zz - 3.0 * xx - 3.0 * yy);
    dB[13][0] = K[13] * (4.0 * zz - 3.0 * xx - yy);
    dB[13][1] = -2.0 * K[13] * x * y;
    dB[13][2] = 8.0 * K[13] * x * z;
    dB[14][0] = 2.0 * K[14] * x * z;
    dB[14][1] = -2.0 * K[14] * y * z;
    dB[14][2] = K[14] * (xx - yy);
    dB[15][0] = K[15] * (3.0 * xx - 3.0 * yy);
    dB[15][1] = -6.0 * K[15] * x * y;
}

void orc_sh_basis_grad64(const double* dirs, int64_t n, int d, double* out /* [n][d][3] */)
{
    init_constants();
    for (int64_t i = 0; i < n; ++i)
        sh_basis_grad64(dirs[3 * i], dirs[3 * i + 1], dirs[3 * i + 2], d, (double(*)[3])(out + i * d * 3));
}

/* Image-space gradients: for every pixel of every tile, Stage 1 again, then
 * the contributions back to front with the explicit suffix S (everything
 * composited behind the contribution, background included):
 *   dC/dalpha_k = T_k c_k - S_k / (1 - alpha_k)
 * and, where the alpha clamp is inactive, alpha = o G with
 *   G = exp(-1/2 d^T conic d), d = p - mu2D,
 *   dG/dmu2D = G conic d,  dG/d(ca, cb, cc) = -G (dx^2 / 2, dx dy, dy^2 / 2);
 * the colour gets dC/dc_k = T_k alpha_k.  Sums per (Gaussian, view) into
 * g2d[v*G + g][NB2D]. */
static void backward_image(scene* s, const float* gC, const int64_t* tiles, int64_t n_tiles, double* g2d)
{
    const int T = s->TX * s->TY;
    int64_t maxlen = 0;
    for (int64_t i = 0; i < (int64_t)s->V * T; ++i)
        if (s->starts[i + 1] - s->starts[i] > maxlen) maxlen = s->starts[i + 1] - s->starts[i];
#pragma omp parallel
    {
        contrib* cl = (contrib*)malloc(sizeof(contrib) * (size_t)maxlen + 1);
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < n_tiles; ++it) {
            const int64_t tile = tiles ? tiles[it] : it;
            int v = (int)(tile / T), t = (int)(tile % T);
            int tx = t % s->TX, ty = t / s->TX;
            const int32_t* list = s->ids + s->starts[tile];
            int64_t L = s->starts[tile + 1] - s->starts[tile];
            for (int yy = 0; yy < TILE; ++yy)
                for (int xx = 0; xx < TILE; ++xx) {
                    int x = tx * TILE + xx, y = ty * TILE + yy;
                    if (x >= s->W || y >= s->H) continue;
                    double C[3], T64;
                    float T32;
                    int n = composite_pixel(s, v, x, y, list, L, cl, C, &T32, &T64);
                    int64_t pix = ((int64_t)v * s->H + y) * s->W + x;
                    double gp[3] = {gC[3 * pix], gC[3 * pix + 1], gC[3 * pix + 2]};
                    double S[3];
                    for (int ch = 0; ch < 3; ++ch) S[ch] = T64 * s->bg[ch];
                    for (int k = n - 1; k >= 0; --k) {
                        const contrib* c = &cl[k];
                        const rec64* q = &s->r64[(int64_t)v * s->G + c->g];
                        double* A = g2d + ((int64_t)v * s->G + c->g) * NB2D;
                        double w = c->T * c->alpha;
                        for (int ch = 0; ch < 3; ++ch) add(&A[6 + ch], gp[ch] * w);
                        if (!c->clamped) {
                            double dLda = 0.0;
                            for (int ch = 0; ch < 3; ++ch)
                                dLda += gp[ch] * (c->T * q->col[ch] - S[ch] / (1.0 - c->alpha));
                            double dx = (x + 0.5) - q->mx, dy = (y + 0.5) - q->my;
                            double dLdG = dLda * q->opac;
                            add(&A[5], dLda * c->G);
                            add(&A[0], dLdG * c->G * (q->ca * dx + q->cb * dy));
                            add(&A[1], dLdG * c->G * (q->cb * dx + q->cc * dy));
                            add(&A[2], -0.5 * dLdG * c->G * dx * dx);
                            add(&A[3], -dLdG * c->G * dx * dy);
                            add(&A[4], -0.5 * dLdG * c->G * dy * dy);
                        }
                        for (int ch = 0; ch < 3; ++ch) S[ch] += w * q->col[ch];
                    }
                }
        }
        free(cl);
    }
}

/* Per Gaussian: chain rule from the image-space gradients of every view to the
 * parameters, out[g] = [mean (3), quaternion (4), scale (3), opacity (1),
 * SH (d x 3, channel fastest)]. */
static void backward_params(scene* s, const double* g2d, double* out)
{
    const int d = s->d, NP = 11 + 3 * d;
#pragma omp parallel for schedule(dynamic, 16)
    for (int g = 0; g < s->G; ++g) {
        double* o = out + (int64_t)g * NP;
        for (int i = 0; i < NP; ++i) o[i] = 0.0;
        const double* sh = s->sh64 + (int64_t)g * d * 3;
        for (int v = 0; v < s->V; ++v) {
            const int64_t rid = (int64_t)v * s->G + g;
            if (s->r32[rid].culled) continue;
            const double* A = g2d + rid * NB2D;
            fwd64 f;
            forward64(s, g, v, &f);
            const double tx = f.tc[0], ty = f.tc[1], tz = f.tc[2];
            double gmu[3] = {0, 0, 0}, gt[3] = {0, 0, 0};

            /* opacity: alpha = o comp G, A[5] = dL/d(o comp) */
            const double comp = s->r64[rid].comp, o_raw = s->r64[rid].opac_raw;
            o[10] += comp * A[5];

            /* colour = max(0.5 + sum_k B_k(dir) sh_k, 0), clamp state frozen */
            double gpre[3];
            for (int ch = 0; ch < 3; ++ch) gpre[ch] = s->r32[rid].clamp_ok[ch] ? A[6 + ch] : 0.0;
            double B[16], dB[16][3];
            sh_basis64(f.dir[0], f.dir[1], f.dir[2], d, B);
            sh_basis_grad64(f.dir[0], f.dir[1], f.dir[2], d, dB);
            double gdir[3] = {0, 0, 0};
            for (int k = 0; k < d; ++k) {
                double gB = 0.0;
                for (int ch = 0; ch < 3; ++ch) {
                    o[11 + 3 * k + ch] += B[k] * gpre[ch];
                    /* a clamped channel (also one with non-finite coefficients) has no direction term */
                    if (s->r32[rid].clamp_ok[ch]) gB += sh[3 * k + ch] * gpre[ch];
                }
                for (int j = 0; j < 3; ++j) gdir[j] += gB * dB[k][j];
            }
            /* dir = (mu - camera centre) / len:  d dir / d mu = (I - dir dir^T) / len */
            double dd = gdir[0] * f.dir[0] + gdir[1] * f.dir[1] + gdir[2] * f.dir[2];
            for (int j = 0; j < 3; ++j) gmu[j] += (gdir[j] - f.dir[j] * dd) / f.len;

            /* projected centre: mx = fx tx / tz + cx, my = fy ty / tz + cy */
            gt[0] += A[0] * f.fx / tz;
            gt[1] += A[1] * f.fy / tz;
            gt[2] += -A[0] * f.fx * tx / (tz * tz) - A[1] * f.fy * ty / (tz * tz);

            /* conic (ca, cb, cc) = (c, -b, a) / (a c - b^2) */
            const double a = f.a, b = f.b, c = f.c, D2 = f.det * f.det;
            const double gca = A[2], gcb = A[3], gcc = A[4];
            double ga = (-c * c * gca + b * c * gcb - b * b * gcc) / D2;
            double gb = (2.0 * b * c * gca - (a * c + b * b) * gcb + 2.0 * a * b * gcc) / D2;
            double gc = (-b * b * gca + a * b * gcb - a * a * gcc) / D2;
            if (s->antialiased && comp > 0.0) {
                /* comp = sqrt(det_r / det): d comp = comp (d log det_r - d log det) / 2 */
                const double dr = f.ar * f.cr - b * b, gcomp = o_raw * A[5] * comp;
                ga += gcomp * (0.5 * f.cr / dr - 0.5 * c / f.det);
                gb += gcomp * (-b / dr + b / f.det);
                gc += gcomp * (0.5 * f.ar / dr - 0.5 * a / f.det);
            }
            /* a, b, c are the entries of S2 = Jc Cc Jc^T (+ dilation), b the mean of the two off-diagonals */
            const double G2[4] = {ga, 0.5 * gb, 0.5 * gb, gc};
            /* dL/dCc = Jc^T G2 Jc,  dL/dJc = 2 G2 Jc Cc (G2, Cc symmetric) */
            double GC[9], GJ[6], JCc[6];
            for (int k = 0; k < 3; ++k)
                for (int l = 0; l < 3; ++l) {
                    double acc = 0;
                    for (int i = 0; i < 2; ++i)
                        for (int j = 0; j < 2; ++j) acc += f.Jc[3 * i + k] * G2[2 * i + j] * f.Jc[3 * j + l];
                    GC[3 * k + l] = acc;
                }
            for (int i = 0; i < 2; ++i)
                for (int l = 0; l < 3; ++l) {
                    double acc = 0;
                    for (int k = 0; k < 3; ++k) acc += f.Jc[3 * i + k] * f.Cc[3 * k + l];
                    JCc[3 * i + l] = acc;
                }
            for (int i = 0; i < 2; ++i)
                for (int l = 0; l < 3; ++l) {
                    double acc = 0;
                    for (int j = 0; j < 2; ++j) acc += G2[2 * i + j] * JCc[3 * j + l];
                    GJ[3 * i + l] = 2.0 * acc;
                }
            /* Jc = [[fx/tz, 0, -fx uxc/tz], [0, fy/tz, -fy uyc/tz]], uxc = tx/tz unless clamped */
            gt[2] += -GJ[0] * f.fx / (tz * tz) - GJ[4] * f.fy / (tz * tz);
            if (f.clip_x) {
                gt[2] += GJ[2] * f.fx * f.uxc / (tz * tz);
            } else {
                gt[0] += -GJ[2] * f.fx / (tz * tz);
                gt[2] += GJ[2] * 2.0 * f.fx * tx / (tz * tz * tz);
            }
            if (f.clip_y) {
                gt[2] += GJ[5] * f.fy * f.uyc / (tz * tz);
            } else {
                gt[1] += -GJ[5] * f.fy / (tz * tz);
                gt[2] += GJ[5] * 2.0 * f.fy * ty / (tz * tz * tz);
            }
            /* t = R mu + t0 */
            for (int j = 0; j < 3; ++j) gmu[j] += f.R[j] * gt[0] + f.R[3 + j] * gt[1] + f.R[6 + j] * gt[2];
            for (int j = 0; j < 3; ++j) o[j] += gmu[j];

            /* Cc = R S3 R^T:  dL/dS3 = R^T GC R */
            double GS[9], tmp[9];
            for (int i = 0; i < 3; ++i)
                for (int l = 0; l < 3; ++l) {
                    double acc = 0;
                    for (int k = 0; k < 3; ++k) acc += f.R[3 * k + i] * GC[3 * k + l];
                    tmp[3 * i + l] = acc;
                }
            for (int i = 0; i < 3; ++i)
                for (int j = 0; j < 3; ++j) {
                    double acc = 0;
                    for (int l = 0; l < 3; ++l) acc += tmp[3 * i + l] * f.R[3 * l + j];
                    GS[3 * i + j] = acc;
                }
            /* S3 = M M^T:  dL/dM = (GS + GS^T) M */
            double GM[9];
            for (int i = 0; i < 3; ++i)
                for (int k = 0; k < 3; ++k) {
                    double acc = 0;
                    for (int j = 0; j < 3; ++j) acc += (GS[3 * i + j] + GS[3 * j + i]) * f.M[3 * j + k];
                    GM[3 * i + k] = acc;
                }
            /* M = Rq diag(sc) */
            double GR[9];
            for (int k = 0; k < 3; ++k) {
                double acc = 0;
                for (int i = 0; i < 3; ++i) acc += GM[3 * i + k] * f.Rq[3 * i + k];
                o[7 + k] += acc;
            }
            for (int i = 0; i < 3; ++i)
                for (int k = 0; k < 3; ++k) GR[3 * i + k] = GM[3 * i + k] * f.sc[k];
            /* Rq of the unit quaternion (w, x, y, z), entry by entry */
            const double w = f.qh[0], x = f.qh[1], y = f.qh[2], z = f.qh[3];
            double gq[4];
            gq[0] = 2.0 * (-z * GR[1] + y * GR[2] + z * GR[3] - x * GR[5] - y * GR[6] + x * GR[7]);
            gq[1] = 2.0 * (y * GR[1] + z * GR[2] + y * GR[3] - 2.0 * x * GR[4] - w * GR[5] + z * GR[6] + w * GR[7] -
                           2.0 * x * GR[8]);
            gq[2] = 2.0 * (-2.0 * y * GR[0] + x * GR[1] + w * GR[2] + x * GR[3] + z * GR[5] - w * GR[6] + z * GR[7] -
                           2.0 * y * GR[8]);
            gq[3] = 2.0 * (-2.0 * z * GR[0] - w * GR[1] + x * GR[2] + w * GR[3] - 2.0 * z * GR[4] + y * GR[5] +
                           x * GR[6] + y * GR[7]);
            /* normalisation q -> q / |q| */
            double qg = 0;
            for (int i = 0; i < 4; ++i) qg += f.qh[i] * gq[i];
            for (int i = 0; i < 4; ++i) o[3 + i] += (gq[i] - f.qh[i] * qg) / f.qn;
        }
    }
}

/* Full backward: out [G][11 + 3 d]; g2d (optional) receives the image-space
 * sums [V*G][NB2D] (record index v*G + g).  With tiles != NULL only those
 * tiles' pixels are walked: the result is complete for every Gaussian whose
 * tile rectangles (in every view) lie inside them.  Needs the lists. */
void orc_backward(void* p, const float* gC, const int64_t* tiles, int64_t n_tiles, double* out, double* g2d_out)
{
    scene* s = (scene*)p;
    double* g2d = (double*)calloc((size_t)s->V * s->G * NB2D + 1, sizeof(double));
    if (!tiles) n_tiles = (int64_t)s->V * s->TX * s->TY;
    backward_image(s, gC, tiles, n_tiles, g2d);
    backward_params(s, g2d, out);
    if (g2d_out) memcpy(g2d_out, g2d, sizeof(double) * (size_t)s->V * s->G * NB2D);
    free(g2d);
}

/* ----------------------------------------------------------------------------
 * Value probes for finite differences (float32 decisions stay frozen).
 * ------------------------------------------------------------------------- */
void orc_values_reset(void* p)
{
    scene* s = (scene*)p;
    memcpy(s->r64, s->r64_base, sizeof(rec64) * (size_t)s->V * s->G);
    for (size_t i = 0; i < (size_t)3 * s->d * s->G; ++i) s->sh64[i] = s->sh[i];
    params64_from_inputs(s);
}

/* move every parameter of Gaussian g (mean 3, quaternion 4, scale 3, opacity 1):
 * all its float64 values are recomputed, the float32 decisions stay frozen */
void orc_set_params64(void* p, int g, const double* prm)
{
    scene* s = (scene*)p;
    memcpy(s->p64 + 11 * (int64_t)g, prm, sizeof(double) * 11);
    for (int v = 0; v < s->V; ++v) {
        const int64_t i = (int64_t)v * s->G + g;
        project64(s, g, v, &s->r32[i], &s->r64[i]);
    }
}

void orc_set_opacity64(void* p, int g, double o)
{
    scene* s = (scene*)p;
    s->p64[11 * (int64_t)g + 10] = o;
    for (int v = 0; v < s->V; ++v) {
        rec64* r = &s->r64[(int64_t)v * s->G + g];
        r->opac_raw = o;
        r->opac = o * r->comp;
    }
}

void orc_set_sh64(void* p, int g, int k, int ch, double value)
{
    scene* s = (scene*)p;
    s->sh64[((int64_t)g * s->d + k) * 3 + ch] = value;
    const double* sh = s->sh64 + (int64_t)g * s->d * 3;
    for (int v = 0; v < s->V; ++v) {
        rec64* r = &s->r64[(int64_t)v * s->G + g];
        const rec32* r32 = &s->r32[(int64_t)v * s->G + g];
        if (r32->culled) continue;
        for (int c = 0; c < 3; ++c) {
            double acc = 0.5;
            for (int kk = 0; kk < s->d; ++kk) acc += r->B[kk] * sh[3 * kk + c];
            r->col[c] = r32->clamp_ok[c] ? acc : 0.0;
        }
    }
}

void orc_set_mean2d64(void* p, int g, int v, double mx, double my)
{
    scene* s = (scene*)p;
    rec64* r = &s->r64[(int64_t)v * s->G + g];
    r->mx = mx;
    r->my = my;
}

/* move the 3D mean; only the projected centres follow (covariance and colour frozen) */
void orc_set_mean3d64(void* p, int g, const double* mu)
{
    scene* s = (scene*)p;
    for (int v = 0; v < s->V; ++v) {
        const float* cam = s->cams + 16 * v;
        double t[3];
        for (int i = 0; i < 3; ++i)
            t[i] = cam[3 * i] * mu[0] + (double)cam[3 * i + 1] * mu[1] + (double)cam[3 * i + 2] * mu[2] + cam[9 + i];
        rec64* r = &s->r64[(int64_t)v * s->G + g];
        r->mx = cam[12] * t[0] / t[2] + cam[14];
        r->my = cam[13] * t[1] / t[2] + cam[15];
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads used by the oracle's parallel loops from now on (timing only). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
