// render.hip -- front-to-back compositing per 16x16 tile on gfx950.
//
// Stage 1 of the Renderer Score Tokens proposal ("Two-Stage Algorithm",
// Standard Render): rendered colour, final transmittance and contributor count
// per pixel, over the depth-ordered tile lists built by the binning pass.
//
// One 256-thread block per tile; the four wave64s each own an 8x8 pixel
// quadrant, so a wave's lanes stay spatially coherent and a wave whose 64
// pixels are all saturated stops.  Batches of 256 list entries are gathered
// (one per thread) into LDS -- centre, exponent coefficients, opacity, clamped
// colour, and a conservative box of the pixels the entry can reach -- and each
// wave compacts, in list order, the entries whose box meets its quadrant, then
// walks only those with broadcast LDS reads.  The box is conservative for the
// float32 evaluation, so the skipped entries are exactly ones every pixel of
// the quadrant would have skipped.  Alpha decisions use the float32 canonical order and the
// specified exponential; the prefix colour is accumulated with compensated
// (Kahan) summation so that the replay can recover the suffix accurately.
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

template <bool STATS>
__global__ __launch_bounds__(256) void k_render(const uint2* __restrict__ ranges, const uint32_t* __restrict__ sorted_g,
                                                const float4* __restrict__ rec0, const float4* __restrict__ rec1,
                                                const float2* __restrict__ rec2, int64_t G, int T, int TX, int W, int H,
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
    __shared__ float4 s0[kRenderBatch];   // {mx, my, qa, qb}
    __shared__ float4 s1[kRenderBatch];   // {qc, opacity, colour r, colour g}
    __shared__ float s2[kRenderBatch];    // colour b
    __shared__ float4 sbox[kRenderBatch]; // conservative box of the pixels the entry can reach
    __shared__ uint8_t slist[4][kRenderBatch];
    __shared__ uint8_t s_ev[4][kRenderBatch];  // per wave: some pixel contributed or saturated at the entry

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
    const float px = (float)pxi + 0.5f, py = (float)pyi + 0.5f;
    // pixel-centre range of this wave's 8x8 quadrant
    const float qx0 = (float)qx + 0.5f, qx1 = (float)qx + 7.5f, qy0 = (float)qy + 0.5f, qy1 = (float)qy + 7.5f;
    const uint2 rg = ranges[tile];
    const int64_t vG = (int64_t)v * G;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    float Tr = 1.0f;
    float h0 = 0.f, h1 = 0.f, h2 = 0.f, c0 = 0.f, c1 = 0.f, c2 = 0.f;
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
            const float2 c = rec2[rid];
            s0[threadIdx.x] = a;
            s1[threadIdx.x] = make_float4(b.x, b.y, clamp_colour(b.z), clamp_colour(b.w));
            s2[threadIdx.x] = clamp_colour(c.x);
            sbox[threadIdx.x] = entry_box_unpack(a.x, a.y, __float_as_uint(c.y));
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
                    const float4 bx = sbox[j];
                    hit = STATS || (bx.x <= qx1 && bx.y >= qx0 && bx.z <= qy1 && bx.w >= qy0);
                }
                const uint64_t m = __ballot(hit);
                if (hit) slist[wave][nw + __popcll(m & lt_mask)] = (uint8_t)j;
                nw += __popcll(m);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            for (int k = 0; k < nw; ++k) {
                const int j = slist[wave][k];
                const float4 a = s0[j];
                const float4 b = s1[j];
                // evaluated in every lane; the decisions below mask lanes that are done or beyond the cut
                const float dx = px - a.x, dy = py - a.y;
                const float e = __builtin_fmaf(dx, __builtin_fmaf(a.z, dx, a.w * dy), (b.x * dy) * dy);
                const bool near = !done && e >= kECutoff;
                const float aG = b.y * exp2_spec(e);
                const float alpha = aG < kAlphaMax ? aG : kAlphaMax;
                const bool pass = near && alpha >= kAlphaMin;
                const float tT = Tr * (1.0f - alpha);
                const bool sat = pass && tT < kTMin;
                const bool contrib = pass && !sat;
                if constexpr (STATS) {
                    n_near += near ? 1u : 0u;
                    if (sat) stop = base + (uint32_t)j;
                }
                done = done || sat;
                if (contrib) {
                    if constexpr (!STATS) {
                        const float w = alpha * Tr;
                        kahan_add(h0, c0, b.z * w);
                        kahan_add(h1, c1, b.w * w);
                        kahan_add(h2, c2, s2[j] * w);
                        ++n;
                    }
                    Tr = tT;
                }
                if (!STATS && pass) s_ev[wave][j] = 1;  // contributed or saturated (every such lane writes the same byte)
                if (__ballot(!done) == 0ull) break;
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
    kahan_add(h0, c0, Tr * bg0);
    kahan_add(h1, c1, Tr * bg1);
    kahan_add(h2, c2, Tr * bg2);
    const float o0 = h0 - c0, o1 = h1 - c1, o2 = h2 - c2;
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
