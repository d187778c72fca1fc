// render.hip -- front-to-back compositing per 16x16 tile on gfx950.
//
// Stage 1 of the Renderer Score Tokens proposal ("Two-Stage Algorithm",
// Standard Render): rendered colour, final transmittance and contributor count
// per pixel, over the depth-ordered tile lists built by the binning pass.
//
// One 256-thread block per tile; the four wave64s each own an 8x8 pixel
// quadrant, so a wave's lanes stay spatially coherent and a wave whose 64
// pixels are all saturated stops.  Batches of 256 list entries are gathered
// (one per thread) into LDS -- centre relative to the tile, exponent factors,
// opacity, clamped colour -- and the gathering thread decides which quadrants
// the entry can reach: its conservative box must meet the quadrant's pixel
// centres, and so must the region of its ellipse where the float32 alpha test
// can pass (its minimum over the quadrant's rectangle, with error margins).  Each wave compacts, in list order, the entries that can
// reach its quadrant, then walks only those with broadcast LDS reads.  Both
// tests are conservative for the float32 evaluation, so the skipped entries are
// exactly ones every pixel of the quadrant would have skipped.  Alpha decisions use the float32 canonical order and the
// specified exponential; the colour is accumulated with fused multiply-adds.
// For every entry it processes, the render also leaves one byte whose bit w
// says whether any pixel of wave w contributed or saturated there: the replay
// walks only those entries, since at every other one no pixel's state changes.
//
// The statistics variant (STATS) evaluates every list entry, takes the same
// decisions, and writes only, per pixel, the list entries examined up to the
// one at which the pixel stopped and how many of them passed the distance cut
// (the plain algorithm's work counts); it runs when those counts are exported,
// so the render itself carries no bookkeeping for them.
#include "gsr_internal.hpp"

namespace gsr {

constexpr int kRenderBatch = 256;
constexpr int kRenderAhead = 3;  // list entries whose geometry is evaluated in one round

template <bool STATS>
__global__ __launch_bounds__(256) void k_render(const uint2* __restrict__ ranges, const uint32_t* __restrict__ sorted_g,
                                                const float4* __restrict__ rec0, const float4* __restrict__ rec1,
                                                const float4* __restrict__ rec2, int64_t G, int T, int TX, int W, int H,
                                                float bg0, float bg1, float bg2, float* __restrict__ color,
                                                float* __restrict__ T_out, int32_t* __restrict__ n_out,
                                                float4* __restrict__ pixel, uint2* __restrict__ pixel_stats,
                                                uint8_t* __restrict__ events, uint32_t* __restrict__ slot_bits,
                                                int64_t n_slot_words, uint32_t* __restrict__ tile_work,
                                                const uint32_t* __restrict__ prev_order) {
    // clear the replay's written-slot bits (a grid-stride share per block)
    if constexpr (!STATS) {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_slot_words;
             i += (int64_t)gridDim.x * blockDim.x)
            slot_bits[i] = 0u;
    }
    // an entry's staged vectors sit at the same byte offset (16 j, kept in the wave's list) of each array
    __shared__ float4 s0[kRenderBatch];   // {tile-relative centre (2), s1, s2}
    __shared__ float4 s1[kRenderBatch];   // {s3, opacity, colour r, colour g}
    __shared__ float4 s2[kRenderBatch];   // {colour b, unused}
    __shared__ uint8_t squad[kRenderBatch];  // bit q: some pixel of quadrant q may pass the entry's alpha test
    __shared__ uint16_t slist[4][kRenderBatch];
    __shared__ uint8_t s_ev[4][kRenderBatch];  // per wave: some pixel contributed or saturated at the entry
    // the same per position of the wave's list (laid out like the list, so both share one address)
    __shared__ uint16_t s_evk[4][kRenderBatch];

    // tiles in the order the previous render of this context measured (longest first), or the natural order;
    // the order only changes how the blocks pack onto the GPU, never a result
    const int tile = prev_order ? (int)prev_order[blockIdx.x] : (int)blockIdx.x;
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
    // pixel-centre range of this wave's 8x8 quadrant, tile-relative
    const uint2 rg = ranges[tile];
    const int64_t vG = (int64_t)v * G;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    float Tr = 1.0f;
    float h0 = 0.f, h1 = 0.f, h2 = 0.f;
    int n = 0;
    uint32_t n_near = 0;          // entries past the distance cut
    uint32_t stop = 0xffffffffu;  // list index at which the pixel saturated
    bool done = !inside;

    uint32_t prev_base = 0;
    int prev_cnt = 0;
    uint32_t base = rg.x;
    for (;; base += kRenderBatch) {
        const int live = __syncthreads_count(!done);
        // the previous batch's event bits (every wave finished it at the barrier above)
        if (!STATS && (int)threadIdx.x < prev_cnt)
            events[prev_base + threadIdx.x] = (uint8_t)(s_ev[0][threadIdx.x] | (s_ev[1][threadIdx.x] << 1) |
                                                        (s_ev[2][threadIdx.x] << 2) | (s_ev[3][threadIdx.x] << 3));
        if (base >= rg.y || live == 0) break;
#pragma unroll
        for (int w = 0; w < 4; ++w) s_ev[w][threadIdx.x] = 0;
        const uint32_t i = base + threadIdx.x;
        if (i < rg.y) {
            const int64_t rid = vG + sorted_g[i];
            const float4 a = rec0[rid];
            const float4 b = rec1[rid];
            const float4 c = rec2[rid];
            const float mxt = tile_centre(a.x, c.z, tx), myt = tile_centre(a.y, c.w, ty);
            s0[threadIdx.x] = make_float4(mxt, myt, a.z, a.w);
            s1[threadIdx.x] = make_float4(b.x, b.y, clamp_colour(b.z), clamp_colour(b.w));
            s2[threadIdx.x] = make_float4(clamp_colour(c.x), 0.0f, 0.0f, 0.0f);
            if constexpr (!STATS) {
                // the quadrants the entry can reach: its box first, then the exact test of its ellipse against
                // the quadrant's pixel-centre rectangle (tile-relative)
                const float4 bx = entry_box_unpack(mxt, myt, __float_as_uint(c.y));
                const EntryConic kq = entry_conic_from_box(a.z, a.w, b.x, __float_as_uint(c.y));
                uint32_t qm = 0u;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float x0 = (float)((q & 1) * 8) + 0.5f, x1 = x0 + 7.0f;
                    const float y0 = (float)((q >> 1) * 8) + 0.5f, y1 = y0 + 7.0f;
                    if (bx.x <= x1 && bx.y >= x0 && bx.z <= y1 && bx.w >= y0 &&
                        ellipse_meets_rect(mxt, myt, kq, x0, x1, y0, y1))
                        qm |= 1u << q;
                }
                squad[threadIdx.x] = (uint8_t)qm;
            }
        }
        __syncthreads();
        const int cnt = (int)min((uint32_t)kRenderBatch, rg.y - base);
        if (__ballot(!done) != 0ull) {
            // this wave's entries, in list order: those whose box meets the quadrant
            int nw = 0;
            for (int c = 0; c < cnt; c += 64) {
                const int j = c + lane;
                bool hit = false;
                if (j < cnt) {
                    // the statistics pass evaluates every entry, so its distance-cut count is the plain
                    // algorithm's (the skipped entries fail the alpha test at every pixel of the quadrant, so
                    // the decisions are the same)
                    hit = STATS || ((squad[j] >> wave) & 1u);
                }
                const uint64_t m = __ballot(hit);
                if (hit) {
                    const int pos = nw + __popcll(m & lt_mask);
                    slist[wave][pos] = (uint16_t)(j * sizeof(float4));
                    s_evk[wave][pos] = 0;
                }
                nw += __popcll(m);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // one entry's geometry (no state): the exponent, alpha and the colour
            struct Geo {
                float S, alpha, cr, cg, cb;
            };
            auto geo = [&](uint32_t off) {
                const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(s0) + off);
                const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(s1) + off);
                // evaluated in every lane; the decisions below mask lanes that are done or beyond the cut
                const float dx = px - a.x, dy = py - a.y;
                Geo g;
                g.S = quad_S(a.z, a.w, b.x, dx, dy);
                const float aG = b.y * exp2_spec(-g.S);
                g.alpha = aG < kAlphaMax ? aG : kAlphaMax;
                g.cr = b.z;
                g.cg = b.w;
                g.cb = reinterpret_cast<const float4*>(reinterpret_cast<const char*>(s2) + off)->x;
                return g;
            };
            // the entry at list position k: its decisions on the lane's state, and the state update; false once
            // every pixel of the wave is done
            auto apply = [&](int k, uint32_t off, const Geo& g) {
                const bool near = !done && g.S <= kSCutoff;
                const bool pass = near && g.alpha >= kAlphaMin;
                const float tT = Tr * (1.0f - g.alpha);
                const bool sat = pass && tT < kTMin;
                const bool contrib = pass != sat;  // (sat implies pass: a mask difference, no second compare)
                if constexpr (STATS) {
                    n_near += near ? 1u : 0u;
                    if (sat) stop = base + off / (uint32_t)sizeof(float4);
                }
                done = done || sat;
                if constexpr (!STATS) {
                    // branch-free: lanes without a contribution add zero
                    const float w = contrib ? g.alpha * Tr : 0.0f;
                    h0 = __builtin_fmaf(g.cr, w, h0);
                    h1 = __builtin_fmaf(g.cg, w, h1);
                    h2 = __builtin_fmaf(g.cb, w, h2);
                    n += contrib ? 1 : 0;
                }
                Tr = contrib ? tT : Tr;
                if (!STATS && pass) s_evk[wave][k] = 1;  // contributed or saturated (every such lane writes the same)
                return __ballot(!done) != 0ull;
            };
            // kRenderAhead entries per round: their geometry, which needs no state, is evaluated together, and
            // their decisions follow in list order (3 measured fastest: 2 leaves latency exposed, 4 adds
            // registers without gain)
            bool live = true;
            for (int k = 0; k < nw && live; k += kRenderAhead) {
                uint32_t o[kRenderAhead];
                Geo g[kRenderAhead];
#pragma unroll
                for (int u = 0; u < kRenderAhead; ++u) {
                    o[u] = slist[wave][min(k + u, nw - 1)];
                    g[u] = geo(o[u]);
                }
#pragma unroll
                for (int u = 0; u < kRenderAhead; ++u)
                    if (live && k + u < nw) live = apply(k + u, o[u], g[u]);
            }
            if constexpr (!STATS) {
                // the events by list position, moved to the entries they name
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                for (int k = lane; k < nw; k += 64)
                    if (s_evk[wave][k]) s_ev[wave][slist[wave][k] / sizeof(float4)] = 1;
            }
        }
        prev_base = base;
        prev_cnt = cnt;
    }
    if constexpr (STATS) {
        if (inside) {
            const int64_t pix = ((int64_t)v * H + pyi) * W + pxi;
            pixel_stats[pix] =
                make_uint2(stop != 0xffffffffu ? stop - rg.x + 1u : (rg.y > rg.x ? rg.y - rg.x : 0u), n_near);
        }
        return;
    }
    // the work of this tile, for the order of the traversals that follow: entries processed until done
    if (threadIdx.x == 0) tile_work[tile] = rg.y > rg.x ? (base < rg.y ? base : rg.y) - rg.x : 0u;
    if (!inside) return;
    const float o0 = __builtin_fmaf(Tr, bg0, h0), o1 = __builtin_fmaf(Tr, bg1, h1), o2 = __builtin_fmaf(Tr, bg2, h2);
    const int64_t pix = ((int64_t)v * H + pyi) * W + pxi;
    if (color) {
        color[3 * pix] = o0;
        color[3 * pix + 1] = o1;
        color[3 * pix + 2] = o2;
    }
    if (T_out) T_out[pix] = Tr;
    if (n_out) n_out[pix] = n;
    pixel[pix] = make_float4(o0, o1, o2, Tr);
}

hipError_t launch_render(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, uint64_t n_pairs,
                         const float bg[3], float* color, float* T_final, int32_t* n_contrib, hipStream_t st,
                         bool prev_order_valid) {
    const int64_t tiles = (int64_t)s.V * s.T;
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_render<false>, dim3((unsigned)tiles), dim3(256), 0, st, ws.ranges, sorted_g, ws.rec0,
                       ws.rec1, ws.rec2, s.G, s.T, s.TX, s.W, s.H, bg[0], bg[1], bg[2], color, T_final, n_contrib,
                       ws.pixel, nullptr, ws.events, ws.slot_bits, (int64_t)((n_pairs + 31) / 32), ws.tile_work,
                       prev_order_valid ? ws.tile_order : nullptr);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_tile_order(ws.tile_work, tiles, ws.tile_order, st);
}

hipError_t launch_render_stats(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, hipStream_t st) {
    const int64_t tiles = (int64_t)s.V * s.T;
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_render<true>, dim3((unsigned)tiles), dim3(256), 0, st, ws.ranges, sorted_g, ws.rec0,
                       ws.rec1, ws.rec2, s.G, s.T, s.TX, s.W, s.H, 0.0f, 0.0f, 0.0f, nullptr, nullptr, nullptr,
                       nullptr, ws.pixel_stats, nullptr, nullptr, (int64_t)0, nullptr, nullptr);
    return hipGetLastError();
}

}  // namespace gsr
