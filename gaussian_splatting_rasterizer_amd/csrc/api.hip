// api.hip -- the C ABI declared in include/gsr.h.
//
// Host code only: argument validation, workspace carve-up, state checks and
// kernel launches on the caller's stream.  No device memory is allocated or
// freed here (a context holds one pinned host word for the pair count); the
// only host/device synchronisation is the read of that count in gs_bin_sort.
#include <sched.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "gsr_internal.hpp"

using namespace gsr;

namespace {

thread_local char g_err[512] = "";

gs_status fail(gs_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

gs_status hip_fail(hipError_t e, const char* where) {
    return fail(GS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

enum State { kCreated = 0, kProjected = 1, kBinned = 2, kRendered = 3 };

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int bits_for(uint64_t n) {  // bits needed to represent values 0..n-1
    int b = 0;
    while (b < 64 && (1ull << b) < n) ++b;
    return b;
}

constexpr int64_t kBlockItems = 4096;  // items per scan block (radix blocks are larger)
constexpr uint64_t kCountPending = ~0ull;  // the pinned pair-count word before the slot scan writes it

}  // namespace

// Per-stage HIP-event timers (host objects; no device memory).
struct StageTimer {
    struct Rec {
        int stage;
        hipEvent_t a, b;
    };
    uint32_t mask = 0u;  // bit s: stage s is timed
    std::vector<hipEvent_t> pool;
    std::vector<Rec> pending;
    double ms[GS_NUM_STAGES] = {};
    int64_t calls[GS_NUM_STAGES] = {};
    hipEvent_t open_ev = nullptr;

    hipEvent_t take() {
        if (pool.empty()) {
            hipEvent_t e = nullptr;
            // timing only: no system-scope fence (cache write-back) at the record, which would idle the GPU
            // between the stages and count that write-back in the stage's time
            if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
            return e;
        }
        hipEvent_t e = pool.back();
        pool.pop_back();
        return e;
    }
    void begin(int stage, hipStream_t st) {
        if (open_ev) pool.push_back(open_ev);  // a stage left open by an early error return
        open_ev = nullptr;
        if (!((mask >> stage) & 1u)) return;
        open_ev = take();
        if (open_ev) (void)hipEventRecord(open_ev, st);
    }
    void end(int stage, hipStream_t st) {
        if (!open_ev) return;  // begin left it unopened: the stage is not timed
        hipEvent_t e = take();
        if (!e) return;
        (void)hipEventRecord(e, st);
        pending.push_back({stage, open_ev, e});
        open_ev = nullptr;
        if (pending.size() > 4096) fold();
    }
    void fold() {
        for (const Rec& r : pending) {
            float t = 0.0f;
            (void)hipEventSynchronize(r.b);
            if (hipEventElapsedTime(&t, r.a, r.b) == hipSuccess) {
                ms[r.stage] += t;
                calls[r.stage] += 1;
            }
            pool.push_back(r.a);
            pool.push_back(r.b);
        }
        pending.clear();
    }
    void destroy() {
        fold();
        for (hipEvent_t e : pool) (void)hipEventDestroy(e);
        pool.clear();
        if (open_ev) (void)hipEventDestroy(open_ev);
        open_ev = nullptr;
    }
};

struct gs_context {
    Sizes s;
    Workspace ws;
    int state;
    gs_gaussians scene;
    CamPack cams;
    gs_params params;
    uint64_t n_pairs;
    const uint32_t* sorted_g;     // Gaussian of each pair in (tile, depth, id) order (set by gs_bin_sort)
    StageTimer timer;
    uint32_t epoch;               // last radix pass epoch; 0 = look-back words not cleared yet
    uint64_t* host_count;         // pinned host word receiving the pair count (allocated on first use)
    uint64_t* host_count_dev;     // its device address: the slot scan writes the count there itself
    bool packed_fresh;            // gs_project left the packed rectangles that the next depth sort reads
    bool order_valid;             // tile_order holds the order a render of this context measured
    uint32_t scan_epoch;          // last single-pass scan tag; 0 = its tile words not cleared yet
    uint32_t scan_ticket_base;    // scan tickets handed out since they were cleared
};

namespace gsr {

Sizes make_sizes(const gs_dims& d) {
    Sizes s;
    s.G = d.n_gaussians;
    s.d = (d.sh_degree + 1) * (d.sh_degree + 1);
    s.V = d.n_views;
    s.W = d.width;
    s.H = d.height;
    s.TX = (d.width + kTile - 1) / kTile;
    s.TY = (d.height + kTile - 1) / kTile;
    s.T = s.TX * s.TY;
    s.VG = (int64_t)s.V * s.G;
    s.max_pairs = d.max_pairs;
    const int64_t nmax = s.VG > (int64_t)s.max_pairs ? s.VG : (int64_t)s.max_pairs;
    // look-back rows for the largest of: the tiles of the largest sort, those of a small sort in half tiles,
    // those of a tiny sort in quarter tiles
    const int64_t nsmall = nmax < kSmallSortKeys ? nmax : kSmallSortKeys;
    const int64_t ntiny = nmax < kTinySortKeys ? nmax : kTinySortKeys;
    const int64_t tiles_large = (nmax + kSortTile - 1) / kSortTile, tiles_small = (nsmall + kSmallSortTile - 1) / kSmallSortTile,
                  tiles_tiny = (ntiny + kTinySortTile - 1) / kTinySortTile;
    s.sort_tiles_cap = tiles_large > tiles_small ? tiles_large : tiles_small;
    if (tiles_tiny > s.sort_tiles_cap) s.sort_tiles_cap = tiles_tiny;
    s.scan_blocks_cap = (s.VG + kBlockItems - 1) / kBlockItems + 1;
    return s;
}

size_t carve_workspace(const Sizes& s, char* base, Workspace* ws) {
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        off = (off + 255) & ~(size_t)255;
        char* p = base ? base + off : nullptr;
        off += bytes;
        return p;
    };
    const size_t VG = (size_t)s.VG, P = (size_t)s.max_pairs;
    const size_t tiles = (size_t)s.V * s.T, pixels = (size_t)s.V * s.W * s.H;
    ws->rec0 = (float4*)take(16 * VG);
    ws->rec1 = (float4*)take(16 * VG);
    ws->rec2 = (float4*)take(16 * VG);
    ws->rect = (uint2*)take(8 * VG);
    ws->depth_key = (uint32_t*)take(4 * VG);
    ws->tiles_touched = (uint32_t*)take(4 * VG);
    ws->slot_base = (uint32_t*)take(4 * VG);
    ws->dkey_b = (uint32_t*)take(4 * VG);
    ws->drid_a = (uint32_t*)take(4 * VG);
    ws->drid_b = (uint32_t*)take(4 * VG);
    ws->rect_sorted = (uint2*)take(8 * VG);
    ws->tt_sorted = (uint32_t*)take(4 * VG);
    ws->offsets = (uint32_t*)take(4 * VG);
    ws->pay_a = (uint32_t*)take(4 * VG);
    ws->pay_b = (uint32_t*)take(4 * VG);
    ws->scan_blocks = (uint64_t*)take(8 * (size_t)s.scan_blocks_cap);
    ws->scan_total = (uint64_t*)take(8 * 4);
    ws->lookback = (uint64_t*)take(8 * 256 * (size_t)s.sort_tiles_cap);
    ws->sort_ctl = (uint32_t*)take(4 * (size_t)kSortCtlWords);
    ws->sort_part = (uint32_t*)take(4 * (size_t)kSortPartBlocks * kSortMaxPasses * 256);
    ws->pkey_emit = (uint32_t*)take(4 * P);
    ws->pkey_b = (uint32_t*)take(4 * P);
    ws->pkey_c = (uint32_t*)take(4 * P);
    ws->pval_a = (uint32_t*)take(4 * P);
    ws->pval_b = (uint32_t*)take(4 * P);
    ws->pair_g = (uint32_t*)take(4 * P);
    ws->ranges = (uint2*)take(8 * tiles);
    ws->tile_work = (uint32_t*)take(4 * tiles);
    ws->tile_order = (uint32_t*)take(4 * tiles);
    ws->partials = (float4*)take(48 * P);
    ws->gv_sums = (float4*)take(48 * VG);
    ws->rec_masks = (uint64_t*)take(16 * ((VG + 63) / 64));
    ws->pixel = (float4*)take(16 * pixels);
    ws->pixel_stats = (uint2*)take(8 * pixels);
    ws->events = (uint8_t*)take(P);
    ws->slot_bits = (uint32_t*)take(4 * ((P + 31) / 32));
    return (off + 255) & ~(size_t)255;
}

}  // namespace gsr

namespace {

// The depth sort carries the tile rectangles through its passes, packed to 32 bits, for tile grids of at most
// 256 x 256 and more than kTinySortKeys records; it gathers them by record in its last pass otherwise (too wide to
// pack, or so few records that a pass is latency-bound and the carry's second reorder costs more than the
// gather: 68 against 72 us for the depth sort of the 311,296-record 512x960 compact scene, while the gather costs
// 0.38 against 0.29 ms for the 7.3 M records of the 8-view 256x448 step).
bool carries_packed_rects(const gsr::Sizes& s) { return s.TX <= 256 && s.TY <= 256 && s.VG > gsr::kTinySortKeys; }

gs_status check_dims(const gs_dims* d) {
    if (!d) return fail(GS_ERR_INVALID_ARGUMENT, "dims is null");
    if (d->n_gaussians < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n_gaussians < 0");
    if (d->sh_degree < 0 || d->sh_degree > 3) return fail(GS_ERR_INVALID_ARGUMENT, "sh_degree must be 0..3");
    if (d->n_views < 1) return fail(GS_ERR_INVALID_ARGUMENT, "n_views must be >= 1");
    if (d->n_views > GS_MAX_VIEWS) return fail(GS_ERR_UNSUPPORTED, "n_views > %d", GS_MAX_VIEWS);
    if (d->width <= 0 || d->height <= 0) return fail(GS_ERR_INVALID_ARGUMENT, "image size must be positive");
    if (d->width > 65535 * 16 || d->height > 65535 * 16) return fail(GS_ERR_UNSUPPORTED, "image too large");
    if (d->max_pairs < 1) return fail(GS_ERR_INVALID_ARGUMENT, "max_pairs must be >= 1");
    // pair indices are u32 and the per-tile loops step past the list end by one batch
    if (d->max_pairs > (1ull << 32) - (1ull << 16)) return fail(GS_ERR_UNSUPPORTED, "max_pairs must be <= 2^32 - 2^16");
    const uint64_t VG = (uint64_t)d->n_gaussians * (uint64_t)d->n_views;
    if (VG >= (1ull << 32)) return fail(GS_ERR_UNSUPPORTED, "n_gaussians * n_views must be < 2^32");
    const uint64_t TX = (d->width + 15) / 16, TY = (d->height + 15) / 16;
    if (TX * TY * (uint64_t)d->n_views >= (1ull << 31)) return fail(GS_ERR_UNSUPPORTED, "too many tiles");
    return GS_OK;
}

}  // namespace

extern "C" {

gs_status gs_default_params(gs_params* out) {
    if (!out) return fail(GS_ERR_INVALID_ARGUMENT, "params is null");
    out->eps = 1e-6f;
    out->den_min = 1e-3f;
    out->lambda = 1.0f;
    out->near_plane = 0.01f;
    out->far_plane = 1e10f;
    out->background[0] = out->background[1] = out->background[2] = 0.0f;
    out->antialiased = 0;
    return GS_OK;
}

gs_status gs_workspace_size(const gs_dims* dims, size_t* bytes_out) {
    gs_status st = check_dims(dims);
    if (st != GS_OK) return st;
    if (!bytes_out) return fail(GS_ERR_INVALID_ARGUMENT, "bytes_out is null");
    Sizes s = make_sizes(*dims);
    Workspace ws;
    *bytes_out = carve_workspace(s, nullptr, &ws);
    return GS_OK;
}

gs_status gs_context_create(const gs_dims* dims, void* workspace, size_t workspace_bytes, gs_context** out) {
    gs_status st = check_dims(dims);
    if (st != GS_OK) return st;
    if (!out) return fail(GS_ERR_INVALID_ARGUMENT, "out is null");
    if (!workspace) return fail(GS_ERR_INVALID_ARGUMENT, "workspace is null");
    if (!aligned(workspace, 256)) return fail(GS_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    Sizes s = make_sizes(*dims);
    Workspace ws;
    const size_t need = carve_workspace(s, nullptr, &ws);
    if (workspace_bytes < need)
        return fail(GS_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    gs_context* c = new (std::nothrow) gs_context();
    if (!c) return fail(GS_ERR_INVALID_ARGUMENT, "out of host memory");
    c->s = s;
    carve_workspace(s, (char*)workspace, &c->ws);
    c->state = kCreated;
    *out = c;
    return GS_OK;
}

gs_status gs_context_destroy(gs_context* ctx) {
    if (ctx) {
        ctx->timer.destroy();
        if (ctx->host_count) (void)hipHostFree(ctx->host_count);
    }
    delete ctx;
    return GS_OK;
}

gs_status gs_project(gs_context* ctx, const gs_gaussians* sc, const gs_camera* cams, const gs_params* params,
                     hipStream_t stream) {
    if (!ctx) return fail(GS_ERR_INVALID_ARGUMENT, "context is null");
    if (!sc || !cams || !params) return fail(GS_ERR_INVALID_ARGUMENT, "null scene, cameras or params");
    const Sizes& s = ctx->s;
    if (sc->n != s.G) return fail(GS_ERR_INVALID_ARGUMENT, "scene has %lld Gaussians, context %lld",
                                  (long long)sc->n, (long long)s.G);
    if ((sc->sh_degree + 1) * (sc->sh_degree + 1) != s.d)
        return fail(GS_ERR_INVALID_ARGUMENT, "scene SH degree differs from the context");
    if (s.G > 0) {
        const void* ptrs[5] = {sc->means, sc->quats, sc->scales, sc->opacities, sc->sh};
        for (const void* p : ptrs) {
            if (!p) return fail(GS_ERR_INVALID_ARGUMENT, "null Gaussian parameter pointer");
            if (!aligned(p, 4)) return fail(GS_ERR_INVALID_ARGUMENT, "misaligned Gaussian parameter pointer");
        }
    }
    if (!(params->eps >= 0.0f) || !(params->den_min >= 0.0f) || !(params->lambda >= 0.0f) ||
        !(params->near_plane > 0.0f) || !(params->far_plane > params->near_plane) ||
        (params->antialiased != 0 && params->antialiased != 1))
        return fail(GS_ERR_INVALID_ARGUMENT, "invalid params");
    // every camera is validated before the context changes, so a rejected call leaves it as it was
    CamPack cp;
    for (int v = 0; v < s.V; ++v) {
        const gs_camera& c = cams[v];
        if (!(c.fx > 0.0f) || !(c.fy > 0.0f)) return fail(GS_ERR_INVALID_ARGUMENT, "focal lengths must be > 0");
        for (int k = 0; k < 9; ++k) cp.c[v][k] = c.R[k];
        for (int k = 0; k < 3; ++k) cp.c[v][9 + k] = c.t[k];
        cp.c[v][12] = c.fx;
        cp.c[v][13] = c.fy;
        cp.c[v][14] = c.cx;
        cp.c[v][15] = c.cy;
        // the same float64 operations preprocess would otherwise repeat for every Gaussian (IEEE division)
        cp.lim[v][0] = kFovClamp * ((0.5 * (double)s.W) / (double)c.fx);
        cp.lim[v][1] = kFovClamp * ((0.5 * (double)s.H) / (double)c.fy);
    }
    ctx->cams = cp;
    ctx->scene = *sc;
    ctx->params = *params;
    ctx->state = kCreated;
    ctx->timer.begin(GS_STAGE_PROJECT, stream);
    // the depth sort's first pass reads the rectangles packed by preprocess (into the depth-ordered tile counts'
    // array, which the sort's last pass writes only afterwards) when it carries them
    const bool packable = carries_packed_rects(s);
    hipError_t e = launch_project(*sc, ctx->cams, s, params->near_plane, params->far_plane, params->antialiased,
                                  packable ? ctx->ws.tt_sorted : nullptr, ctx->ws, stream);
    if (e != hipSuccess) return hip_fail(e, "project");
    ctx->packed_fresh = packable;
    ctx->timer.end(GS_STAGE_PROJECT, stream);
    ctx->state = kProjected;
    return GS_OK;
}

}  // extern "C"

namespace {

// Binning and sorting.  With `count_by_copy` the pair count is read back with a copy into host
// stack memory after the depth sort is queued (nothing allocated: the no-allocation path); otherwise
// the slot scan writes it into the context's mapped pinned word and the host polls an event.
gs_status bin_sort_impl(gs_context* ctx, hipStream_t stream, uint64_t* n_pairs_out, bool count_by_copy) {
    if (!ctx) return fail(GS_ERR_INVALID_ARGUMENT, "context is null");
    if (ctx->state < kProjected) return fail(GS_ERR_STATE, "gs_bin_sort before gs_project");
    const Sizes& s = ctx->s;
    Workspace& ws = ctx->ws;
    hipError_t e;
    StageTimer& tm = ctx->timer;
    // look-back words: cleared on the first sort of the context and before the epoch wraps
    if (ctx->epoch == 0 || ctx->epoch > kEpochLimit) {
        e = launch_fill_u32(reinterpret_cast<uint32_t*>(ws.lookback), 2 * 256 * s.sort_tiles_cap, 0u, stream);
        if (e != hipSuccess) return hip_fail(e, "look-back clear");
        ctx->epoch = 0;
    }
    if (!count_by_copy && !ctx->host_count) {
        e = hipHostMalloc((void**)&ctx->host_count, 64, hipHostMallocMapped | hipHostMallocCoherent);
        if (e != hipSuccess) {
            ctx->host_count = nullptr;
            return hip_fail(e, "pinned count word");
        }
        e = hipHostGetDevicePointer((void**)&ctx->host_count_dev, ctx->host_count, 0);
        if (e != hipSuccess) return hip_fail(e, "pinned count word address");
    }
    // the pinned word holds kCountPending until the slot scan writes the count into it
    if (!count_by_copy) *(volatile uint64_t*)ctx->host_count = kCountPending;
    const SortScratch sort_scratch{ws.lookback, ws.sort_ctl, ws.sort_part};
    // (scan_total[3] holds the scans' ticket counter)
    ScanState scan_state{ws.scan_blocks, s.scan_blocks_cap, reinterpret_cast<uint32_t*>(ws.scan_total + 3),
                         &ctx->scan_epoch, &ctx->scan_ticket_base};
    // 0. slot bases of the replay's partials: tile counts scanned in record order
    tm.begin(GS_STAGE_DEPTH_SORT, stream);
    // the pair count is this scan's total (the same tile counts as the depth-ordered scan below): the scan
    // writes it into pinned host memory too, and the host waits for it only after the sort and the second scan
    // are queued, so that the GPU has work while the host waits
    e = launch_scan_u32(ws.tiles_touched, s.VG, ws.slot_base, scan_state, ws.scan_total + 1, stream, false,
                        count_by_copy ? nullptr : ctx->host_count_dev);
    if (e != hipSuccess) return hip_fail(e, "slot scan");
    // 1. depth sort of the records (four 8-bit passes; keys ping-pong through offsets, which the
    //    scan rewrites next); the tile rectangles ride along (packed, or gathered by the last pass), and
    //    the last pass writes rectangles and tile counts in depth order but no keys
    uint32_t* rid_sorted = nullptr;
    const bool packable = carries_packed_rects(s);
    // (a second sort after one gs_project packs on load: the first sort's last pass overwrote the packed form)
    // for such grids the last pass leaves the packed rectangles (in depth order) in tt_sorted, from which the
    // offsets scan and emit take the tile counts and rectangles
    const RectSort rs{ws.rect, ws.rect_sorted, ws.tt_sorted, packable ? ws.pay_a : nullptr,
                      packable ? ws.pay_b : nullptr, packable && ctx->packed_fresh ? ws.tt_sorted : nullptr, packable};
    ctx->packed_fresh = false;
    e = launch_radix_sort(ws.depth_key, nullptr, s.VG, 32, ws.dkey_b, ws.offsets, ws.drid_a, ws.drid_b, &rs, nullptr,
                          false, 0, sort_scratch, &ctx->epoch, stream, nullptr, &rid_sorted);
    if (e != hipSuccess) return hip_fail(e, "depth sort");
    tm.end(GS_STAGE_DEPTH_SORT, stream);
    // 2. pair offsets in depth order
    tm.begin(GS_STAGE_SCAN, stream);
    e = launch_scan_u32(ws.tt_sorted, s.VG, ws.offsets, scan_state, ws.scan_total, stream, packable);
    if (e != hipSuccess) return hip_fail(e, "scan");
    tm.end(GS_STAGE_SCAN, stream);
    uint64_t total = 0;
    if (count_by_copy) {
        e = hipMemcpyAsync(&total, ws.scan_total + 1, sizeof total, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e, "pair count copy");
    } else {
        // wait for the pair count by polling the pinned word (no event in the stream, so no gap between the
        // kernels), yielding the core between polls; a stream that fails or drains without writing it ends
        // the wait with an error
        for (;;) {
            total = *(volatile uint64_t*)ctx->host_count;
            if (total != kCountPending) break;
            e = hipStreamQuery(stream);
            if (e == hipSuccess) {
                total = *(volatile uint64_t*)ctx->host_count;
                if (total == kCountPending) return fail(GS_ERR_HIP, "the slot scan did not write the pair count");
                break;
            }
            if (e != hipErrorNotReady) return hip_fail(e, "pair count wait");
            sched_yield();
        }
    }
    if (n_pairs_out) *n_pairs_out = total;
    ctx->n_pairs = total;
    if (total > s.max_pairs) {
        ctx->state = kCreated;
        return fail(GS_ERR_WORKSPACE_TOO_SMALL, "%llu pairs exceed max_pairs %llu", (unsigned long long)total,
                    (unsigned long long)s.max_pairs);
    }
    // 3. emit pairs in depth order, counting the tile sort's digits on the way (the histogram rows and the
    //    ranges are cleared first), 4. stable sort by tile with the ranges, 5. empty ranges
    const int64_t tiles = (int64_t)s.V * s.T;
    const RadixDigits td = radix_digits(bits_for((uint64_t)tiles));
    // when a tile id and a Gaussian index fit one 32-bit word together, the pairs are sorted as such words
    const int gbits = bits_for((uint64_t)s.G) > 0 ? bits_for((uint64_t)s.G) : 1;
    const int packed_gbits = td.bits + gbits <= 32 ? gbits : 0;
    // the ranges start as {~0u, 0} (set by the emission, or here when there is no record to emit): a tile the
    // last pass never sees keeps start > end, an empty range for every traversal (they loop while start < end;
    // the ranges export turns it into {0, 0}).  The depth sort left the histogram rows the emission adds the
    // tile sort's digit counts into at zero.
    if (s.VG == 0) {
        tm.begin(GS_STAGE_RANGES, stream);
        e = launch_ranges_init(ws.ranges, tiles, nullptr, stream);
        if (e != hipSuccess) return hip_fail(e, "ranges init");
        tm.end(GS_STAGE_RANGES, stream);
    }
    tm.begin(GS_STAGE_EMIT, stream);
    e = launch_emit(s, ws, rid_sorted, &td, packed_gbits, packable, stream);
    if (e != hipSuccess) return hip_fail(e, "emit");
    tm.end(GS_STAGE_EMIT, stream);
    uint32_t* sorted_g = nullptr;
    // the last pass of the tile sort records every tile's [start, end) (sorted keys are not kept)
    tm.begin(GS_STAGE_TILE_SORT, stream);
    e = launch_radix_sort(ws.pkey_emit, packed_gbits > 0 ? nullptr : ws.pair_g, (int64_t)total, td.bits, ws.pkey_b,
                          ws.pkey_c, ws.pval_a, ws.pval_b, nullptr, ws.ranges, true, packed_gbits, sort_scratch,
                          &ctx->epoch, stream, nullptr, &sorted_g);
    if (e != hipSuccess) return hip_fail(e, "tile sort");
    tm.end(GS_STAGE_TILE_SORT, stream);
    ctx->sorted_g = sorted_g;
    ctx->state = kBinned;
    return GS_OK;
}

}  // namespace

extern "C" {

gs_status gs_bin_sort(gs_context* ctx, hipStream_t stream, uint64_t* n_pairs_out) {
    return bin_sort_impl(ctx, stream, n_pairs_out, false);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The path without any allocation: the workspace is a file-scope device array
// (one per GPU, held until the process ends) and the context lives on the stack.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = (size_t)GS_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this GPU's copy of `scratch`, looked up once per device with that device
// current (the array's name is a host-side stand-in, not a device address).
gs_status scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(GS_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "scratch address");
        if (!ptr || !aligned(ptr, 256)) return fail(GS_ERR_HIP, "scratch address is null or misaligned");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GS_OK;
}

}  // namespace

extern "C" {

gs_status gs_render_score_noalloc(const gs_gaussians* scene, const gs_camera* cams, int32_t n_views, int32_t width,
                                  int32_t height, const gs_params* params, const float* observed, float* color,
                                  float* T_final, int32_t* n_contrib, float* tokens, hipStream_t stream) {
    if (!scene || !cams || !params || !observed) return fail(GS_ERR_INVALID_ARGUMENT, "null argument");
    gs_dims d;
    d.n_gaussians = scene->n;
    d.sh_degree = scene->sh_degree;
    d.n_views = n_views;
    d.width = width;
    d.height = height;
    d.max_pairs = 1;
    gs_status st = check_dims(&d);
    if (st != GS_OK) return st;
    // the largest pair capacity whose workspace fits the scratch array (the workspace grows linearly in it)
    Workspace probe;
    const size_t base = carve_workspace(make_sizes(d), nullptr, &probe);
    d.max_pairs = 1025;
    const size_t per_1024 = carve_workspace(make_sizes(d), nullptr, &probe) - base;
    if (base > kScratchBytes)
        return fail(GS_ERR_WORKSPACE_TOO_SMALL,
                    "gs_render_score_noalloc: %lld Gaussians x %d views of %dx%d need %zu bytes before any pair, "
                    "the scratch array holds %zu", (long long)scene->n, n_views, width, height, base, kScratchBytes);
    uint64_t cap = 1 + (uint64_t)((kScratchBytes - base) / (per_1024 + 1)) * 1024;
    if (cap > (1ull << 32) - (1ull << 16)) cap = (1ull << 32) - (1ull << 16);
    for (;;) {
        d.max_pairs = cap;
        if (carve_workspace(make_sizes(d), nullptr, &probe) <= kScratchBytes || cap <= 1) break;
        cap = cap > 1024 ? cap - 1024 : 1;
    }
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != GS_OK) return st;
    // a context on the stack: no timers, no pinned word, no events (the pair count is copied back)
    gs_context ctx{};
    ctx.s = make_sizes(d);
    carve_workspace(ctx.s, (char*)ws, &ctx.ws);
    ctx.state = kCreated;
    ctx.epoch = 0;  // clears the look-back words: the previous call's contents are not trusted
    st = gs_project(&ctx, scene, cams, params, stream);
    if (st != GS_OK) return st;
    uint64_t n_pairs = 0;
    st = bin_sort_impl(&ctx, stream, &n_pairs, true);
    if (st == GS_ERR_WORKSPACE_TOO_SMALL)
        return fail(GS_ERR_WORKSPACE_TOO_SMALL,
                    "gs_render_score_noalloc: %llu (tile, Gaussian) pairs exceed the %llu the %zu-byte scratch array "
                    "holds for this problem", (unsigned long long)n_pairs, (unsigned long long)cap, kScratchBytes);
    if (st != GS_OK) return st;
    st = gs_render(&ctx, color, T_final, n_contrib, stream);
    if (st != GS_OK) return st;
    return gs_score_replay(&ctx, observed, tokens, stream);
}

gs_status gs_render(gs_context* ctx, float* color, float* T_final, int32_t* n_contrib, hipStream_t stream) {
    if (!ctx) return fail(GS_ERR_INVALID_ARGUMENT, "context is null");
    if (ctx->state < kBinned) return fail(GS_ERR_STATE, "gs_render before gs_bin_sort");
    if ((color && !aligned(color, 4)) || (T_final && !aligned(T_final, 4)) || (n_contrib && !aligned(n_contrib, 4)))
        return fail(GS_ERR_INVALID_ARGUMENT, "misaligned output pointer");
    ctx->timer.begin(GS_STAGE_RENDER, stream);
    hipError_t e = launch_render(ctx->s, ctx->ws, ctx->sorted_g, ctx->n_pairs, ctx->params.background, color,
                                 T_final, n_contrib, stream, ctx->order_valid);
    if (e != hipSuccess) return hip_fail(e, "render");
    ctx->order_valid = true;
    ctx->timer.end(GS_STAGE_RENDER, stream);
    ctx->state = kRendered;
    return GS_OK;
}

gs_status gs_score_replay(gs_context* ctx, const float* observed, float* tokens, hipStream_t stream) {
    if (!ctx) return fail(GS_ERR_INVALID_ARGUMENT, "context is null");
    if (ctx->state < kRendered) return fail(GS_ERR_STATE, "gs_score_replay before gs_render");
    if (!observed || (!tokens && ctx->s.G > 0)) return fail(GS_ERR_INVALID_ARGUMENT, "null observed or tokens");
    if (!aligned(observed, 4) || !aligned(tokens, 4)) return fail(GS_ERR_INVALID_ARGUMENT, "misaligned pointer");
    ctx->timer.begin(GS_STAGE_REPLAY, stream);
    hipError_t e = launch_replay(ctx->s, ctx->ws, ctx->sorted_g, observed, ctx->params.eps, ctx->params.den_min,
                                 stream);
    if (e != hipSuccess) return hip_fail(e, "replay");
    ctx->timer.end(GS_STAGE_REPLAY, stream);
    ctx->timer.begin(GS_STAGE_FINALIZE, stream);
    if (!tokens_gather(ctx->s)) {  // (otherwise the token kernel sums each record's slots itself)
        e = launch_gather_slots(ctx->s, ctx->ws, 2, stream);
        if (e != hipSuccess) return hip_fail(e, "gather");
    }
    e = launch_tokens(ctx->scene, ctx->cams, ctx->s, ctx->ws, ctx->params.eps, ctx->params.lambda, tokens, stream);
    if (e != hipSuccess) return hip_fail(e, "tokens");
    ctx->timer.end(GS_STAGE_FINALIZE, stream);
    return GS_OK;
}

gs_status gs_backward(gs_context* ctx, const float* grad_color, const gs_gaussian_grads* grads, hipStream_t stream) {
    if (!ctx) return fail(GS_ERR_INVALID_ARGUMENT, "context is null");
    if (ctx->state < kRendered) return fail(GS_ERR_STATE, "gs_backward before gs_render");
    if (!grad_color || !grads) return fail(GS_ERR_INVALID_ARGUMENT, "null grad_color or grads");
    if (!aligned(grad_color, 4)) return fail(GS_ERR_INVALID_ARGUMENT, "misaligned grad_color");
    const float* outs[5] = {grads->means, grads->quats, grads->scales, grads->opacities, grads->sh};
    for (const float* p : outs)
        if (p && !aligned(p, 4)) return fail(GS_ERR_INVALID_ARGUMENT, "misaligned gradient pointer");
    ctx->timer.begin(GS_STAGE_BACKWARD, stream);
    hipError_t e = launch_backward(ctx->s, ctx->ws, ctx->sorted_g, grad_color, stream);
    if (e != hipSuccess) return hip_fail(e, "backward");
    ctx->timer.end(GS_STAGE_BACKWARD, stream);
    ctx->timer.begin(GS_STAGE_BACKWARD_FINALIZE, stream);
    e = launch_gather_slots(ctx->s, ctx->ws, 3, stream);
    if (e != hipSuccess) return hip_fail(e, "backward gather");
    e = launch_backward_finalize(ctx->scene, ctx->cams, ctx->s, ctx->ws, ctx->params.antialiased, *grads, stream);
    if (e != hipSuccess) return hip_fail(e, "gradients");
    ctx->timer.end(GS_STAGE_BACKWARD_FINALIZE, stream);
    return GS_OK;
}

gs_status gs_render_features(gs_context* ctx, const float* features, int32_t n_channels, const float* background,
                             float* out, hipStream_t stream) {
    if (!ctx) return fail(GS_ERR_INVALID_ARGUMENT, "context is null");
    if (ctx->state < kRendered) return fail(GS_ERR_STATE, "gs_render_features before gs_render");
    if (n_channels < 1) return fail(GS_ERR_INVALID_ARGUMENT, "n_channels must be >= 1");
    if ((ctx->s.G > 0 && !features) || !out) return fail(GS_ERR_INVALID_ARGUMENT, "null features or out");
    if ((features && !aligned(features, 4)) || !aligned(out, 4))
        return fail(GS_ERR_INVALID_ARGUMENT, "misaligned pointer");
    ctx->timer.begin(GS_STAGE_FEATURES, stream);
    hipError_t e = launch_render_features(ctx->s, ctx->ws, ctx->sorted_g, features, n_channels, background, out,
                                          stream);
    if (e != hipSuccess) return hip_fail(e, "feature composite");
    ctx->timer.end(GS_STAGE_FEATURES, stream);
    return GS_OK;
}

gs_status gs_attribute(gs_context* ctx, const float* pixel_map, int32_t n_channels, float* out, hipStream_t stream) {
    if (!ctx) return fail(GS_ERR_INVALID_ARGUMENT, "context is null");
    if (ctx->state < kRendered) return fail(GS_ERR_STATE, "gs_attribute before gs_render");
    if (n_channels < 1) return fail(GS_ERR_INVALID_ARGUMENT, "n_channels must be >= 1");
    if (!pixel_map || (ctx->s.G > 0 && !out)) return fail(GS_ERR_INVALID_ARGUMENT, "null pixel_map or out");
    if (!aligned(pixel_map, 4) || (out && !aligned(out, 4))) return fail(GS_ERR_INVALID_ARGUMENT, "misaligned pointer");
    ctx->timer.begin(GS_STAGE_ATTRIBUTE, stream);
    hipError_t e = launch_attribute(ctx->s, ctx->ws, ctx->sorted_g, pixel_map, n_channels, out, stream);
    if (e != hipSuccess) return hip_fail(e, "attribution");
    ctx->timer.end(GS_STAGE_ATTRIBUTE, stream);
    return GS_OK;
}

gs_status gs_debug_topk(gs_context* ctx, int32_t k, int32_t* ids, float* weights, hipStream_t stream) {
    if (!ctx) return fail(GS_ERR_INVALID_ARGUMENT, "context is null");
    if (ctx->state < kRendered) return fail(GS_ERR_STATE, "gs_debug_topk before gs_render");
    if (k < 1 || k > 16) return fail(GS_ERR_INVALID_ARGUMENT, "k must be 1..16");
    if (!ids || !weights) return fail(GS_ERR_INVALID_ARGUMENT, "null ids or weights");
    if (!aligned(ids, 4) || !aligned(weights, 4)) return fail(GS_ERR_INVALID_ARGUMENT, "misaligned pointer");
    hipError_t e = launch_topk(ctx->s, ctx->ws, ctx->sorted_g, k, ids, weights, stream);
    if (e != hipSuccess) return hip_fail(e, "top-k");
    return GS_OK;
}

const char* gs_status_string(gs_status s) {
    switch (s) {
        case GS_OK: return "GS_OK";
        case GS_ERR_INVALID_ARGUMENT: return "GS_ERR_INVALID_ARGUMENT";
        case GS_ERR_WORKSPACE_TOO_SMALL: return "GS_ERR_WORKSPACE_TOO_SMALL";
        case GS_ERR_STATE: return "GS_ERR_STATE";
        case GS_ERR_HIP: return "GS_ERR_HIP";
        case GS_ERR_UNSUPPORTED: return "GS_ERR_UNSUPPORTED";
    }
    return "GS_ERR_UNKNOWN";
}

const char* gs_last_error(void) { return g_err; }

gs_status gs_debug_exp2(const float* in, float* out, int64_t n, hipStream_t stream) {
    if (n < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n < 0");
    if (n > 0 && (!in || !out)) return fail(GS_ERR_INVALID_ARGUMENT, "null pointer");
    hipError_t e = launch_exp2(in, out, n, stream);
    if (e != hipSuccess) return hip_fail(e, "exp2");
    return GS_OK;
}

gs_status gs_debug_export(gs_context* ctx, int32_t kind, void* dst, size_t bytes, hipStream_t stream) {
    if (!ctx || !dst) return fail(GS_ERR_INVALID_ARGUMENT, "null context or destination");
    const Sizes& s = ctx->s;
    const Workspace& ws = ctx->ws;
    const size_t VG = (size_t)s.VG;
    hipError_t e = hipSuccess;
    switch (kind) {
        case GS_EXPORT_RECORDS: {
            if (ctx->state < kProjected) return fail(GS_ERR_STATE, "records exist after gs_project");
            if (bytes < 64 * VG) return fail(GS_ERR_INVALID_ARGUMENT, "destination too small");
            char* d = (char*)dst;
            e = hipMemcpyAsync(d, ws.rec0, 16 * VG, hipMemcpyDeviceToDevice, stream);
            if (e == hipSuccess) e = hipMemcpyAsync(d + 16 * VG, ws.rec1, 16 * VG, hipMemcpyDeviceToDevice, stream);
            if (e == hipSuccess) e = hipMemcpyAsync(d + 32 * VG, ws.rec2, 16 * VG, hipMemcpyDeviceToDevice, stream);
            // fourth plane {rect lo, rect hi, -, -}
            if (e == hipSuccess && VG > 0)
                e = hipMemcpy2DAsync(d + 48 * VG, 16, ws.rect, 8, 8, VG, hipMemcpyDeviceToDevice, stream);
            break;
        }
        case GS_EXPORT_DEPTH_KEYS:
            if (ctx->state < kProjected) return fail(GS_ERR_STATE, "depth keys exist after gs_project");
            if (bytes < 4 * VG) return fail(GS_ERR_INVALID_ARGUMENT, "destination too small");
            e = hipMemcpyAsync(dst, ws.depth_key, 4 * VG, hipMemcpyDeviceToDevice, stream);
            break;
        case GS_EXPORT_SORTED_IDS:
            if (ctx->state < kBinned) return fail(GS_ERR_STATE, "lists exist after gs_bin_sort");
            if (bytes < 4 * (size_t)ctx->n_pairs) return fail(GS_ERR_INVALID_ARGUMENT, "destination too small");
            if (ctx->n_pairs)
                e = hipMemcpyAsync(dst, ctx->sorted_g, 4 * (size_t)ctx->n_pairs, hipMemcpyDeviceToDevice, stream);
            break;
        case GS_EXPORT_RANGES: {
            const size_t tiles = (size_t)s.V * s.T;
            if (ctx->state < kBinned) return fail(GS_ERR_STATE, "ranges exist after gs_bin_sort");
            if (bytes < 8 * tiles) return fail(GS_ERR_INVALID_ARGUMENT, "destination too small");
            e = launch_ranges_export(ws.ranges, (uint2*)dst, (int64_t)tiles, stream);
            break;
        }
        case GS_EXPORT_PIXEL_STATS: {
            const size_t pixels = (size_t)s.V * s.W * s.H;
            if (ctx->state < kRendered) return fail(GS_ERR_STATE, "pixel stats exist after gs_render");
            if (bytes < 8 * pixels) return fail(GS_ERR_INVALID_ARGUMENT, "destination too small");
            // counted by a statistics pass over the same lists with the render's decisions
            e = launch_render_stats(s, ws, ctx->sorted_g, stream);
            if (e == hipSuccess) e = hipMemcpyAsync(dst, ws.pixel_stats, 8 * pixels, hipMemcpyDeviceToDevice, stream);
            break;
        }
        default:
            return fail(GS_ERR_INVALID_ARGUMENT, "unknown export kind %d", kind);
    }
    if (e != hipSuccess) return hip_fail(e, "export copy");
    return GS_OK;
}

gs_status gs_profile_enable(gs_context* ctx, int32_t enable) {
    return gs_profile_stages(ctx, enable != 0 ? (1u << GS_NUM_STAGES) - 1u : 0u);
}

gs_status gs_profile_stages(gs_context* ctx, uint32_t stage_mask) {
    if (!ctx) return fail(GS_ERR_INVALID_ARGUMENT, "context is null");
    if (stage_mask >> GS_NUM_STAGES) return fail(GS_ERR_INVALID_ARGUMENT, "stage mask 0x%x names no stage", stage_mask);
    ctx->timer.mask = stage_mask;
    return GS_OK;
}

gs_status gs_profile_read(gs_context* ctx, double* ms, int64_t* calls, int32_t n_stages) {
    if (!ctx || !ms || !calls) return fail(GS_ERR_INVALID_ARGUMENT, "null argument");
    if (n_stages < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n_stages < 0");
    ctx->timer.fold();
    for (int i = 0; i < GS_NUM_STAGES; ++i) {
        if (i < n_stages) {
            ms[i] = ctx->timer.ms[i];
            calls[i] = ctx->timer.calls[i];
        }
        ctx->timer.ms[i] = 0.0;
        ctx->timer.calls[i] = 0;
    }
    return GS_OK;
}

}  // extern "C"
