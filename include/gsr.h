/*
 * gsr.h -- C ABI of the MI355X (gfx950) Gaussian-splat renderer with analytic
 * score replay.
 *
 * The method is the one of the page "Research Proposal: Renderer Score Tokens
 * for Recurrent Gaussian Splatting":
 *   Stage 1 (section "Two-Stage Algorithm", Stage 1: Standard Render): tile
 *     binning and contributor sorting, front-to-back compositing giving the
 *     rendered colour, the final transmittance and the contributor count; the
 *     tile bins and sorted contributor indices stay inside the renderer
 *     workspace and are never exposed as a per-pixel contributor tensor.
 *   Stage 2 (Stage 2: Analytic Score Replay, suffix equation and masks): a
 *     second traversal of the same bins in the same order that recovers the
 *     suffix composite behind each contribution and accumulates per-Gaussian
 *     scores, emitting only fixed-dimensional tokens.
 *   Scores and tokens: section "Exact Score Operators" (opacity-logit score,
 *     SH score, projected-centre mean score, projection Jacobian, cross-view
 *     weight, covector pullback, conditioning matrix statistics, appearance
 *     aggregation) and "Final Token and Updater" (token layout, dimension
 *     9 + 3 d_SH).
 *
 * Calling sequence, all on one stream:  gs_project -> gs_bin_sort -> gs_render
 * [-> gs_score_replay] [-> gs_backward] [-> gs_render_features] [-> gs_attribute].  Each call returns a status and never aborts.
 *
 * Memory: every array argument is a DEVICE pointer unless marked "host".
 * The caller owns every buffer (inputs, outputs and the workspace); the
 * library never allocates or frees device memory.  Input pointers given to
 * gs_project are borrowed until gs_score_replay (or the next gs_project)
 * returns: the replay re-reads means and opacities.
 *
 * Errors: a call that returns anything but GS_OK has launched no work when the
 * error is GS_ERR_INVALID_ARGUMENT or GS_ERR_STATE; gs_last_error() gives a
 * thread-local message for the last failure on the calling thread.
 *
 * Threading: a context is used from one thread and one stream at a time.
 */
#ifndef GSR_H
#define GSR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GSR_API __attribute__((visibility("default")))

typedef enum {
    GS_OK = 0,
    GS_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, bad size, unsupported degree */
    GS_ERR_WORKSPACE_TOO_SMALL = 2, /* more (tile, Gaussian) pairs than the workspace holds */
    GS_ERR_STATE = 3,              /* call out of order (e.g. render before bin_sort) */
    GS_ERR_HIP = 4,                /* a HIP runtime call failed; see gs_last_error() */
    GS_ERR_UNSUPPORTED = 5         /* size beyond the implementation limits */
} gs_status;

/* Limits of this implementation. */
#define GS_MAX_VIEWS 32
/* Size of the device array gs_render_score_noalloc works in (one per GPU). */
#define GS_NOALLOC_SCRATCH_BYTES (64u << 20)
#define GS_TILE 16

/* Scene: n Gaussians, parameters already activated.
 *   means      [n,3]    world-space centres
 *   quats      [n,4]    rotation quaternions (w, x, y, z); normalised inside
 *   scales     [n,3]    positive axis scales (already exp-activated)
 *   opacities  [n]      opacity o = sigmoid(a) in [0, 1]
 *   sh         [n,d,3]  SH coefficients, d = (sh_degree + 1)^2, channel fastest
 * All float32, contiguous, 4-byte aligned device arrays.  Non-finite values are
 * not an error: the affected (Gaussian, view) pairs are culled or masked. */
typedef struct {
    const float* means;
    const float* quats;
    const float* scales;
    const float* opacities;
    const float* sh;
    int64_t n;
    int32_t sh_degree; /* 0..3 */
} gs_gaussians;

/* Pinhole camera (host memory): x_cam = R x_world + t (R row-major), pixel
 * u = fx x/z + cx, v = fy y/z + cy; the pixel (i, j) centre is (i + 0.5, j + 0.5). */
typedef struct {
    float R[9];
    float t[3];
    float fx, fy, cx, cy;
} gs_camera;

/* Problem sizes fixed for the lifetime of a context. */
typedef struct {
    int64_t n_gaussians;
    int32_t sh_degree;  /* 0..3 */
    int32_t n_views;    /* 1..GS_MAX_VIEWS, all views share width x height */
    int32_t width;
    int32_t height;
    uint64_t max_pairs; /* capacity for (tile, Gaussian) pairs, 1 .. 2^32 - 2^16 */
} gs_dims;

/* Numerical parameters (the pages name these constants but give no values).
 *   eps        epsilon of the suffix denominator, the support q and the
 *              cross-view weight (default 1e-6)
 *   den_min    a contribution whose suffix denominator T(1-alpha) is below
 *              this is masked out of the opacity and mean scores (default 1e-3)
 *   lambda     ridge of the conditioning matrix A = lambda I + ... (default 1)
 *   near_plane, far_plane   depth culling range (defaults 0.01, 1e10)
 *   background colour added behind the last contributor (default 0)
 *   antialiased  0 (default) or 1: opacity-compensated 2D filter -- the 0.3 px^2
 *              dilation is kept and each (Gaussian, view) opacity is scaled by
 *              sqrt(det S / det(S + 0.3 I)) (S the undilated projected
 *              covariance; 0 when det S <= 0), so a footprint keeps the
 *              integrated weight of the undilated Gaussian.  The score replay's
 *              opacity score keeps the Gaussian's own o in (1 - o); gs_backward
 *              differentiates the compensation too. */
typedef struct {
    float eps;
    float den_min;
    float lambda;
    float near_plane;
    float far_plane;
    float background[3];
    int32_t antialiased;
} gs_params;

typedef struct gs_context gs_context;

/* Fill *out with the defaults above.  Never fails for a non-null pointer. */
GSR_API gs_status gs_default_params(gs_params* out);

/* Bytes of device workspace a context with these sizes needs (host-only call). */
GSR_API gs_status gs_workspace_size(const gs_dims* dims, size_t* bytes_out);

/* Create a context over caller-owned device memory `workspace` (>= the size
 * above, 256-byte aligned).  The context itself is host memory. */
GSR_API gs_status gs_context_create(const gs_dims* dims, void* workspace, size_t workspace_bytes,
                            gs_context** out);
GSR_API gs_status gs_context_destroy(gs_context* ctx);

/* Preprocess every (Gaussian, view).  Follows the page "Research Proposal:
 * Renderer Score Tokens for Recurrent Gaussian Splatting", Two-Stage Algorithm,
 * Stage 1 (Standard Render: project the Gaussians, evaluate their colours),
 * with the projection conventions of the ATSplat summary page (section
 * 前置知识: EWA covariance projection, SH colour): EWA projection of the 3D
 * covariance to the image (+0.3 px^2 dilation), inverse 2D covariance as
 * exponent factors, 3-sigma radius and tile rectangle, depth, SH colour along
 * the view direction (+0.5, clamped at 0, clamp state kept for the SH score).
 *   scene   device arrays of scene->n Gaussians (layouts in gs_gaussians), read
 *           only; they must stay valid until the last call that reads them
 *           (gs_score_replay and gs_backward read means and opacities again)
 *   cams    host array [n_views], copied into the context
 *   params  host struct, copied (gs_default_params gives the defaults)
 * Asynchronous on `stream`.  Errors: GS_ERR_INVALID_ARGUMENT (null or
 * misaligned pointers, n or sh_degree not those of the context, invalid params,
 * a camera whose focal lengths are not > 0 -- then nothing in the context
 * changes); GS_ERR_HIP on a launch failure. */
GSR_API gs_status gs_project(gs_context* ctx, const gs_gaussians* scene, const gs_camera* cams,
                     const gs_params* params, hipStream_t stream);

/* Tile binning and contributor sorting.  Follows the Proposal page's
 * Two-Stage Algorithm, Stage 1 (tile binning and per-tile depth order of the
 * standard render, which the score replay re-traverses unchanged): order the
 * (Gaussian, view) records by depth, emit one (tile, Gaussian) pair per
 * covered tile, stable-sort the pairs by tile and build per-tile ranges; the
 * lists and ranges stay in the workspace.  Waits on the host for the pair
 * count (polling a pinned host word the context allocates on its first call,
 * while the GPU sorts; written to *n_pairs_out, which may be null).  Errors:
 * GS_ERR_STATE before gs_project; GS_ERR_WORKSPACE_TOO_SMALL (with the count)
 * when it exceeds max_pairs -- the caller then creates a larger context and
 * starts again from gs_project; GS_ERR_HIP on a launch or stream failure. */
GSR_API gs_status gs_bin_sort(gs_context* ctx, hipStream_t stream, uint64_t* n_pairs_out);

/* Front-to-back compositing per 16x16 tile.  Follows the Proposal page's
 * Two-Stage Algorithm, Stage 1 (Standard Render: rendered colour, final
 * transmittance and contributor count per pixel), with the alpha rules of its
 * Exact Score Operators section (alpha = o G clamped at 0.99, contributions
 * below 1/255 skipped, a pixel stops before its transmittance falls below
 * 1e-4).  Outputs are caller-owned device arrays (any may be null):
 *   color      [n_views, height, width, 3] rendered colour incl. background
 *   T_final    [n_views, height, width]    final transmittance
 *   n_contrib  [n_views, height, width]    accepted contributions (int32)
 * The rendered colour is also kept in the workspace for gs_score_replay, with
 * one byte per processed list entry marking the 8x8 pixel blocks in which some
 * pixel's state changed there (the replay walks only those entries).
 * Scheduling: the render records each tile's work (list entries processed)
 * and the traversals that follow it (replay, backward, features, attribution)
 * take the tiles longest first; the next gs_render on the same context starts
 * from that order too (the first takes the tiles in index order).  The order
 * changes only how the work packs onto the GPU: every tile is fully computed
 * and all outputs are identical whatever the order.  Errors: GS_ERR_STATE
 * before gs_bin_sort; GS_ERR_INVALID_ARGUMENT for a misaligned output;
 * GS_ERR_HIP on a launch failure. */
GSR_API gs_status gs_render(gs_context* ctx, float* color, float* T_final, int32_t* n_contrib,
                    hipStream_t stream);

/* Analytic score replay.  Follows the Proposal page's Two-Stage Algorithm,
 * Stage 2 (Analytic Score Replay: re-traverse the same lists, residual, prefix
 * and suffix composites, masks), its Exact Score Operators (the mean, opacity
 * and SH scores, the cross-view weights and the conditioning matrix) and its
 * Final Token section.  `observed` is a caller-owned device array
 * [n_views, height, width, 3] (float32); `tokens` a caller-owned device array
 * [n, 9 + 3 d] (may be null only when n = 0).  Computes the residual
 * r = C_hat - C, the suffix C+ = (C_hat - P - T alpha c) /
 * (T (1 - alpha) + eps), masked per-Gaussian partial scores, cross-view
 * aggregation and the token
 *   tokens [n, 9 + 3 d] = [ b_mu (3), s_alpha (1), s_SH (3 d, index k*3 + channel),
 *                           log Q (1), eig(A) / (tr A + eps) (3, descending),
 *                           log(tr A + eps) (1) ]
 * with Q = eps + sum_v q_gv the cross-view support. */
/* Errors: GS_ERR_STATE before gs_render; GS_ERR_INVALID_ARGUMENT for null or
 * misaligned arrays; GS_ERR_HIP on a launch failure. */
GSR_API gs_status gs_score_replay(gs_context* ctx, const float* observed, float* tokens, hipStream_t stream);

/* The whole path -- gs_project, gs_bin_sort, gs_render, gs_score_replay --
 * in one call that allocates nothing, for callers that cannot allocate device
 * or pinned memory (tight serving loops, harnesses that forbid allocation).
 * It takes the same inputs and writes the same outputs as that sequence
 * (`color`, `T_final`, `n_contrib` may be null; `tokens` [n, 9 + 3 d] may be
 * null only when n = 0), with a context on the host stack and, as workspace,
 * a file-scope device array of GS_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU
 * the library runs on holds until the process ends.  The pair count is read
 * back with a copy into host stack memory (the call synchronises `stream`).
 * Problems whose workspace does not fit -- the records of n x n_views, or the
 * (tile, Gaussian) pairs the binning finds -- return
 * GS_ERR_WORKSPACE_TOO_SMALL with the sizes in gs_last_error(); the outputs
 * are then not written.  Every call on a GPU uses that GPU's one array, so
 * calls that overlap on one GPU (several threads or streams) race; the array
 * keeps the last call's contents, and the call clears what it needs cleared. */
GSR_API gs_status gs_render_score_noalloc(const gs_gaussians* scene, const gs_camera* cams, int32_t n_views,
                                          int32_t width, int32_t height, const gs_params* params,
                                          const float* observed, float* color, float* T_final, int32_t* n_contrib,
                                          float* tokens, hipStream_t stream);

/* Gradients of a scalar loss with respect to the scene parameters, laid out
 * like the gs_gaussians arrays they belong to (float32 device arrays, written,
 * not accumulated; a null member is skipped):
 *   means [n,3], quats [n,4] (of the quaternion as given, before its
 *   normalisation), scales [n,3], opacities [n], sh [n,d,3]. */
typedef struct {
    float* means;
    float* quats;
    float* scales;
    float* opacities;
    float* sh;
} gs_gaussian_grads;

/* Renderer backward: the vector-Jacobian product of the rendered colour with
 * `grad_color` = dL/dC_hat [n_views, height, width, 3] (float32 device), i.e.
 * the exact gradient of the colour image of gs_render through the
 * front-to-back composite, the 2D Gaussian, the EWA projection (covariance
 * Jacobian at the field-of-view-clamped centre, 0.3 px^2 dilation), the
 * covariance R_q diag(s)^2 R_q^T of the normalised quaternion and the scales,
 * and the SH colour including its dependence on the view direction, with the
 * render's float32 decisions held fixed (contributor sets and early stop,
 * alpha clamp at 0.99 -- a clamped contribution passes no gradient to
 * opacity or shape --, colour clamp at 0, field-of-view clamp).  The forward
 * is Stage 1 of the page "Research Proposal: Renderer Score Tokens for
 * Recurrent Gaussian Splatting" ("Two-Stage Algorithm", Standard Render) with
 * the 3DGS primitive of the ATSplat summary page ("前置知识: 3DGS").
 * Traverses the same tile bins and order as gs_render (valid after gs_render,
 * before or after gs_score_replay), reading the scene arrays given to
 * gs_project.  Asynchronous on `stream`; uses the workspace's partial and
 * per-record sum areas, so it must not overlap gs_score_replay on the same
 * context. */
GSR_API gs_status gs_backward(gs_context* ctx, const float* grad_color, const gs_gaussian_grads* grads,
                              hipStream_t stream);

/* Feature composite: per-Gaussian attribute vectors `features` [n, n_channels]
 * (float32 device, view-independent) composited with the render's weights,
 *   out[v, y, x, c] = sum_k T_k alpha_k features[g_k, c] + T_final * background[c]
 * into `out` [n_views, height, width, n_channels] (float32 device) -- the same
 * contributors, order and float32 decisions as the colour of gs_render.  The
 * ATSplat summary page ("核心方法": the uncertainty score rendered as a scalar
 * attribute by alpha compositing) and ReCoSplat's render-and-compare module
 * (9 learned feature channels rendered with the RGB) use this operation.
 * `background` is a host array of n_channels floats, or null for zeros.
 * n_channels >= 1 (slices of 16 channels are composited per launch).  Valid
 * after gs_render; asynchronous on `stream`. */
GSR_API gs_status gs_render_features(gs_context* ctx, const float* features, int32_t n_channels,
                                     const float* background, float* out, hipStream_t stream);

/* Attribution scatter: a per-pixel map `pixel_map` [n_views, height, width,
 * n_channels] (float32 device) sent back to the Gaussians along the render's
 * weights,
 *   out[g, c] = sum over views v and pixels p of T alpha (p, g, v) * pixel_map[v, p, c]
 * into `out` [n, n_channels] (float32 device, written).  The transpose of
 * gs_render_features: the alphaT scatter (map = 1) and the scalar-attribution
 * baselines of the Renderer Score Tokens plan (an error + coverage token for
 * map = (|r|^2, 1)), and the mask-channel gain attribution of the L2D2-GS
 * summary (map = the 2D gain).  n_channels >= 1 (passes of 8 channels).  Valid
 * after gs_render; uses the workspace's partial and per-record sum areas, so it
 * must not overlap gs_score_replay / gs_backward on the same context. */
GSR_API gs_status gs_attribute(gs_context* ctx, const float* pixel_map, int32_t n_channels, float* out,
                               hipStream_t stream);

GSR_API const char* gs_status_string(gs_status s);
GSR_API const char* gs_last_error(void);

/* ---- diagnostics used by the test-suite ---------------------------------- */

/* The float32 exponential used by every alpha decision: out[i] = 2^in[i],
 * valid for in[i] in [-8, 0.5] (device arrays of n floats). */
GSR_API gs_status gs_debug_exp2(const float* in, float* out, int64_t n, hipStream_t stream);

/* Copy an internal workspace array into the caller's device buffer `dst`
 * (`bytes` must be at least the array size; the call fails otherwise):
 *   GS_EXPORT_RECORDS   after gs_project:  [4, n_views*n, 4] float32, planes
 *       {mx, my, s1, s2}, {s3, opacity, pre_r, pre_g},
 *       {pre_b, <entry box: two binary16 half-widths, x low>, mx_lo, my_lo},
 *       {<x0 | y0 << 16>, <x1 | y1 << 16>, -, -} (tile rectangle
 *       [x0, x1) x [y0, y1)), record index v*n + g; the projected centre is
 *       (mx + mx_lo, my + my_lo) and the Gaussian weight at offset
 *       (dx, dy) = pixel - centre is 2^-((s1 dx + s2 dy)^2 + (s3 dy)^2); culled
 *       records are all zero
 *   GS_EXPORT_DEPTH_KEYS after gs_project: [n_views*n] uint32 depth bits
 *       (0xffffffff when culled)
 *   GS_EXPORT_SORTED_IDS after gs_bin_sort: [n_pairs] uint32 Gaussian index
 *   GS_EXPORT_RANGES    after gs_bin_sort: [n_views*tiles] x 2 uint32 [start, end)
 *   GS_EXPORT_PIXEL_STATS after gs_render: [n_views*height*width] x 2 uint32:
 *       list entries evaluated before the pixel stopped, and how many of those
 *       passed the distance cut (exponent >= -8) -- the work counts of the pass,
 *       counted on export by a pass over the same lists with the render's
 *       decisions (the render itself keeps no such counts)
 */
typedef enum {
    GS_EXPORT_RECORDS = 1,
    GS_EXPORT_DEPTH_KEYS = 2,
    GS_EXPORT_SORTED_IDS = 3,
    GS_EXPORT_RANGES = 4,
    GS_EXPORT_PIXEL_STATS = 5
} gs_export_kind;
GSR_API gs_status gs_debug_export(gs_context* ctx, int32_t kind, void* dst, size_t bytes, hipStream_t stream);

/* Debug top-K contributor metadata (the Renderer Score Tokens plan, Block 0,
 * which enables it on small tiles only): per pixel the k accepted contributions
 * of largest weight T alpha, in decreasing weight (equal weights in list order),
 *   ids     [n_views, height, width, k] int32 Gaussian index, -1 where unused
 *   weights [n_views, height, width, k] float32 T alpha, 0 where unused
 * (device arrays).  1 <= k <= 16.  Valid after gs_render.  Costs a traversal
 * and 8 k bytes per pixel: a diagnostic, not part of the path. */
GSR_API gs_status gs_debug_topk(gs_context* ctx, int32_t k, int32_t* ids, float* weights, hipStream_t stream);

/* Per-stage timing with HIP events recorded on the caller's stream around each
 * stage's launches (events are created by the library on first use and kept
 * until gs_context_destroy).  gs_profile_read waits for the recorded events,
 * writes the milliseconds and launch counts accumulated since the previous read
 * for the first min(n_stages, GS_NUM_STAGES) stages into the host arrays ms and
 * calls (n_stages entries each), and resets every stage's totals. */
typedef enum {
    GS_STAGE_PROJECT = 0,
    GS_STAGE_DEPTH_SORT = 1,
    GS_STAGE_SCAN = 2,
    GS_STAGE_EMIT = 3,
    GS_STAGE_TILE_SORT = 4,
    GS_STAGE_RANGES = 5,             /* tile ranges set on their own: only without records (else the pair emission sets them) */
    GS_STAGE_RENDER = 6,
    GS_STAGE_REPLAY = 7,
    GS_STAGE_FINALIZE = 8,
    GS_STAGE_BACKWARD = 9,          /* gs_backward traversal */
    GS_STAGE_BACKWARD_FINALIZE = 10, /* gs_backward slot gather and per-Gaussian chain rule */
    GS_STAGE_FEATURES = 11,          /* gs_render_features */
    GS_STAGE_ATTRIBUTE = 12,         /* gs_attribute (traversal, gather, sum over views) */
    GS_NUM_STAGES = 13
} gs_stage;
/* gs_profile_enable: every stage (enable != 0) or none.  gs_profile_stages:
 * only the stages whose bit (1 << stage) is set in stage_mask; each timed stage
 * costs two event records on the stream (a few microseconds of idle GPU at its
 * boundaries), so a caller timing the whole path selects the stages it needs.
 * A bit at or above GS_NUM_STAGES is GS_ERR_INVALID_ARGUMENT. */
GSR_API gs_status gs_profile_enable(gs_context* ctx, int32_t enable);
GSR_API gs_status gs_profile_stages(gs_context* ctx, uint32_t stage_mask);
GSR_API gs_status gs_profile_read(gs_context* ctx, double* ms, int64_t* calls, int32_t n_stages);

#ifdef __cplusplus
}
#endif

#endif /* GSR_H */
