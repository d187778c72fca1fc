// attributes.hip -- per-Gaussian attributes composited with the render weights,
// and per-pixel maps scattered back along them, on gfx950.
//
// The render weight of an accepted contribution is w = T alpha (Stage 1 of the
// Renderer Score Tokens proposal, "Two-Stage Algorithm": the same tiles, lists,
// order and float32 decisions as the render).
//   * Feature composite: F(p) = sum_k w_k f_{g_k} + T_final bg.  The ATSplat
//     summary page renders its per-anchor uncertainty score as such a scalar
//     attribute; ReCoSplat's render-and-compare conditioning adds 9 learned
//     feature channels rendered the same way.
//   * Attribution scatter: a_g = sum_v sum_p w_{p,g,v} m(p) for a per-pixel map
//     m: the alphaT scatter for m = 1, an error + coverage token for
//     m = (|r|^2, 1), L2D2-GS's gain attribution through a mask channel for m =
//     the gain map.  It is the transpose of the composite (the gradient of
//     <m, F> with respect to the features).
//
// Both walk, per wave, only the entries at which the render flagged an event
// for that wave (every other entry changes no pixel of the wave), exactly as
// the score replay does; a wave's list ends at its last event, so the walk
// does not test for the wave being done.  The composite keeps NC channel accumulators per
// pixel (channel slices of at most 16 per launch); the scatter reduces eight
// channels per pass over the wave (the replay's reduce-scatter), stores one
// 32-byte partial per event pair at the pair's slot, and the slot gather and a
// per-Gaussian sum over views finish it.
#include "gsr_internal.hpp"

namespace gsr {

constexpr int kAttrBatch = 128;

template <int NC>
__global__ __launch_bounds__(256) void k_render_features(const uint2* __restrict__ ranges,
                                                         const uint32_t* __restrict__ sorted_g,
                                                         const float4* __restrict__ rec0,
                                                         const float4* __restrict__ rec1,
                                                         const float4* __restrict__ rec2, int64_t G, int T, int TX,
                                                         int W, int H, const uint8_t* __restrict__ events,
                                                         const float* __restrict__ feat, int C, int c0, int nc,
                                                         FeatBg bg, float* __restrict__ out,
                                                         const uint32_t* __restrict__ tile_order,
                                                         const uint32_t* __restrict__ tile_work) {
    __shared__ float4 s0[kAttrBatch];
    __shared__ float2 s1[kAttrBatch];
    __shared__ float sf[kAttrBatch][NC];
    __shared__ uint32_t s_gid[kAttrBatch];
    __shared__ uint8_t s_evb[kAttrBatch];
    __shared__ uint8_t slist[4][kAttrBatch];

    const int tile = (int)tile_order[blockIdx.x];
    const int v = tile / T;
    const int t = tile - v * T;
    const int ty = t / TX, tx = t - ty * TX;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pxi = tx * kTile + (wave & 1) * 8 + (lane & 7);
    const int pyi = ty * kTile + (wave >> 1) * 8 + (lane >> 3);
    const bool inside = pxi < W && pyi < H;
    // pixel centre relative to the tile origin (entry centres are staged tile-relative too)
    const float px = (float)(pxi - tx * kTile) + 0.5f, py = (float)(pyi - ty * kTile) + 0.5f;
    const uint2 rg = ranges[tile];
    // the entries the render processed (every event lies there); an empty range ({~0u, 0}) has none
    const uint32_t rend = rg.x + min(tile_work[tile], rg.y > rg.x ? rg.y - rg.x : 0u);
    const int64_t vG = (int64_t)v * G;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    float acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.0f;
    float Tr = 1.0f;
    bool done = !inside;

    for (uint32_t base = rg.x; base < rend; base += kAttrBatch) {
        if (__syncthreads_count(!done) == 0) break;
        const uint32_t i = base + threadIdx.x;
        if (threadIdx.x < kAttrBatch && i < rend) {
            const uint32_t g = sorted_g[i];
            const int64_t rid = vG + g;
            const float4 a = rec0[rid];
            const float4 c = rec2[rid];
            s0[threadIdx.x] = make_float4(tile_centre(a.x, c.z, tx), tile_centre(a.y, c.w, ty), a.z, a.w);
            const float4 b = rec1[rid];
            s1[threadIdx.x] = make_float2(b.x, b.y);
            s_evb[threadIdx.x] = events[i];
            s_gid[threadIdx.x] = g;
        }
        const int cnt = (int)min((uint32_t)kAttrBatch, rend - base);
        __syncthreads();
        // the staged entries' channels, one float per thread in row-major order: consecutive threads write
        // consecutive LDS words (no bank conflicts) and read each Gaussian's channels as one contiguous run
        for (int f = threadIdx.x; f < cnt * NC; f += 256) {
            const int j = f / NC, c = f % NC;
            sf[j][c] = c < nc ? feat[(int64_t)s_gid[j] * C + c0 + c] : 0.0f;
        }
        __syncthreads();
        if (__ballot(!done) != 0ull) {
            int nw = 0;
            for (int c = 0; c < cnt; c += 64) {
                const int j = c + lane;
                const bool hit = j < cnt && ((s_evb[j] >> wave) & 1u);
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
                const float2 b = s1[j];
                const float dx = px - a.x, dy = py - a.y;
                const float S = quad_S(a.z, a.w, b.x, dx, dy);
                const bool near = !done && S <= kSCutoff;
                const float aG = b.y * exp2_spec(-S);
                const float alpha = !(aG < kAlphaMax) ? kAlphaMax : aG;
                const bool pass = near && alpha >= kAlphaMin;
                const float tT = Tr * (1.0f - alpha);
                const bool sat = pass && tT < kTMin;
                const bool contrib = pass != sat;  // (sat implies pass: a mask difference, no second compare)
                done = done || sat;
                const float w = contrib ? alpha * Tr : 0.0f;
#pragma unroll
                for (int c = 0; c < NC; ++c) acc[c] = __builtin_fmaf(w, sf[j][c], acc[c]);
                Tr = contrib ? tT : Tr;
            }
        }
        __syncthreads();
    }
    if (!inside) return;
    float* o = out + (((int64_t)v * H + pyi) * W + pxi) * C + c0;
#pragma unroll
    for (int c = 0; c < NC; ++c)
        if (c < nc) o[c] = __builtin_fmaf(Tr, bg.v[c], acc[c]);
}

hipError_t launch_render_features(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, const float* feat,
                                  int C, const float* bg_host, float* out, hipStream_t st) {
    const int64_t tiles = (int64_t)s.V * s.T;
    if (tiles == 0) return hipSuccess;
    for (int c0 = 0; c0 < C; c0 += 16) {
        const int nc = C - c0 < 16 ? C - c0 : 16;
        FeatBg bg;
        for (int c = 0; c < 16; ++c) bg.v[c] = (bg_host && c < nc) ? bg_host[c0 + c] : 0.0f;
#define GSR_LAUNCH_FEAT(NN)                                                                                       \
    hipLaunchKernelGGL(k_render_features<NN>, dim3((unsigned)tiles), dim3(256), 0, st, ws.ranges, sorted_g,       \
                       ws.rec0, ws.rec1, ws.rec2, s.G, s.T, s.TX, s.W, s.H, ws.events, feat, C, c0, nc, bg, out,      \
                       ws.tile_order, ws.tile_work)
        if (nc <= 4) GSR_LAUNCH_FEAT(4);
        else if (nc <= 8) GSR_LAUNCH_FEAT(8);
        else GSR_LAUNCH_FEAT(16);
#undef GSR_LAUNCH_FEAT
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Attribution scatter of up to eight channels per pass.
__global__ __launch_bounds__(256) void k_attribute(const uint2* __restrict__ ranges,
                                                   const uint32_t* __restrict__ sorted_g,
                                                   const uint32_t* __restrict__ slot_base,
                                                   const float4* __restrict__ rec0, const float4* __restrict__ rec1,
                                                   const float4* __restrict__ rec2,
                                                   const uint2* __restrict__ rect, int64_t G, int T, int TX, int W,
                                                   int H, const uint8_t* __restrict__ events,
                                                   const float* __restrict__ map, int C, int c0, int nc,
                                                   float4* __restrict__ partials, uint32_t* __restrict__ slot_bits,
                                                   const uint32_t* __restrict__ tile_order,
                                                   const uint32_t* __restrict__ tile_work) {
    __shared__ float4 s0[kAttrBatch];
    __shared__ float2 s1[kAttrBatch];
    __shared__ uint8_t s_evb[kAttrBatch];
    __shared__ uint32_t s_slot[kAttrBatch];
    __shared__ uint8_t slist[4][kAttrBatch];
    __shared__ __align__(16) float sp[4][kAttrBatch][8];

    const int tile = (int)tile_order[blockIdx.x];
    const int v = tile / T;
    const int t = tile - v * T;
    const int ty = t / TX, tx = t - ty * TX;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pxi = tx * kTile + (wave & 1) * 8 + (lane & 7);
    const int pyi = ty * kTile + (wave >> 1) * 8 + (lane >> 3);
    const bool inside = pxi < W && pyi < H;
    // pixel centre relative to the tile origin (entry centres are staged tile-relative too)
    const float px = (float)(pxi - tx * kTile) + 0.5f, py = (float)(pyi - ty * kTile) + 0.5f;
    const uint2 rg = ranges[tile];
    // the entries the render processed (every event lies there); an empty range ({~0u, 0}) has none
    const uint32_t rend = rg.x + min(tile_work[tile], rg.y > rg.x ? rg.y - rg.x : 0u);
    const int64_t vG = (int64_t)v * G;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    float m[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) m[c] = 0.0f;
    if (inside) {
        const float* mp = map + (((int64_t)v * H + pyi) * W + pxi) * C + c0;
#pragma unroll
        for (int c = 0; c < 8; ++c)
            if (c < nc) m[c] = mp[c];
    }
    float Tr = 1.0f;
    bool done = !inside;

    for (uint32_t base = rg.x; base < rend; base += kAttrBatch) {
        if (__syncthreads_count(!done) == 0) break;
        const uint32_t i = base + threadIdx.x;
        if (threadIdx.x < kAttrBatch && i < rend) {
            const int64_t rid = vG + sorted_g[i];
            const float4 a = rec0[rid];
            const float4 c = rec2[rid];
            s0[threadIdx.x] = make_float4(tile_centre(a.x, c.z, tx), tile_centre(a.y, c.w, ty), a.z, a.w);
            const float4 b = rec1[rid];
            s1[threadIdx.x] = make_float2(b.x, b.y);
            s_evb[threadIdx.x] = events[i];
            const uint2 rc = rect[rid];
            const uint32_t x0 = rc.x & 0xffffu, y0 = rc.x >> 16, wx = (rc.y & 0xffffu) - x0;
            s_slot[threadIdx.x] = slot_base[rid] + ((uint32_t)ty - y0) * wx + ((uint32_t)tx - x0);
        }
        const int cnt = (int)min((uint32_t)kAttrBatch, rend - base);
        for (int e = lane; e < cnt * 8; e += 64) (&sp[wave][0][0])[e] = 0.0f;
        __syncthreads();
        if (__ballot(!done) != 0ull) {
            int nw = 0;
            for (int c = 0; c < cnt; c += 64) {
                const int j = c + lane;
                const bool hit = j < cnt && ((s_evb[j] >> wave) & 1u);
                const uint64_t mk = __ballot(hit);
                if (hit) slist[wave][nw + __popcll(mk & lt_mask)] = (uint8_t)j;
                nw += __popcll(mk);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // one entry: the decisions and state updates of every lane, and its weight (every listed entry has
            // a contribution or saturation in some lane of the wave)
            auto step = [&](int j) {
                const float4 a = s0[j];
                const float2 b = s1[j];
                const float dx = px - a.x, dy = py - a.y;
                const float S = quad_S(a.z, a.w, b.x, dx, dy);
                const bool near = !done && S <= kSCutoff;
                const float aG = b.y * exp2_spec(-S);
                const float alpha = !(aG < kAlphaMax) ? kAlphaMax : aG;
                const bool pass = near && alpha >= kAlphaMin;
                const float tT = Tr * (1.0f - alpha);
                const bool sat = pass && tT < kTMin;
                const bool contrib = pass != sat;  // (sat implies pass: a mask difference, no second compare)
                done = done || sat;
                const float w = contrib ? alpha * Tr : 0.0f;
                Tr = contrib ? tT : Tr;
                return w;
            };
            auto reduce = [&](float w) {
                float x[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) x[c] = w * m[c];
                return wave_reduce8(x, lane);
            };
            // two entries per round: the two wave reductions, independent of each other, run interleaved
            int k = 0;
            for (; k + 1 < nw; k += 2) {
                const int j0 = slist[wave][k], j1 = slist[wave][k + 1];
                const float w0 = step(j0);
                const float w1 = step(j1);
                const float red0 = reduce(w0), red1 = reduce(w1);
                if ((lane & 7) == 0) {
                    sp[wave][j0][lane >> 3] = red0;
                    sp[wave][j1][lane >> 3] = red1;
                }
            }
            if (k < nw) {
                const int j0 = slist[wave][k];
                const float red0 = reduce(step(j0));
                if ((lane & 7) == 0) sp[wave][j0][lane >> 3] = red0;
            }
        }
        __syncthreads();
        // one 32-byte partial per entry at which some wave had an event, flagged in the slot bits
        if (threadIdx.x < 2 * cnt && s_evb[threadIdx.x >> 1] != 0) {
            const int j = threadIdx.x >> 1, h = threadIdx.x & 1;
            float4 acc = *reinterpret_cast<const float4*>(&sp[0][j][4 * h]);
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                const float4 q = *reinterpret_cast<const float4*>(&sp[w][j][4 * h]);
                acc.x += q.x;
                acc.y += q.y;
                acc.z += q.z;
                acc.w += q.w;
            }
            const uint32_t slot = s_slot[j];
            partials[2 * (int64_t)slot + h] = acc;
            if (h == 0) atomicOr(&slot_bits[slot >> 5], 1u << (slot & 31u));
        }
    }
}

// Per Gaussian: the sum over views of its records' gathered sums (eight channels).
__global__ __launch_bounds__(256) void k_sum_views(int64_t G, int V, const uint64_t* __restrict__ rec_masks,
                                                   const float4* __restrict__ gv_sums, int C, int c0, int nc,
                                                   float* __restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= G) return;
    float a[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) a[c] = 0.0f;
    for (int v = 0; v < V; ++v) {
        const int64_t rid = (int64_t)v * G + g;
        if (!((rec_masks[2 * (rid >> 6) + 1] >> (rid & 63)) & 1ull)) continue;
        const float4 p = gv_sums[2 * rid], q = gv_sums[2 * rid + 1];
        a[0] += p.x;
        a[1] += p.y;
        a[2] += p.z;
        a[3] += p.w;
        a[4] += q.x;
        a[5] += q.y;
        a[6] += q.z;
        a[7] += q.w;
    }
    float* o = out + g * C + c0;
#pragma unroll
    for (int c = 0; c < 8; ++c)
        if (c < nc) o[c] = a[c];
}

hipError_t launch_attribute(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, const float* map, int C,
                            float* out, hipStream_t st) {
    const int64_t tiles = (int64_t)s.V * s.T;
    for (int c0 = 0; c0 < C; c0 += 8) {
        const int nc = C - c0 < 8 ? C - c0 : 8;
        if (tiles > 0)
            hipLaunchKernelGGL(k_attribute, dim3((unsigned)tiles), dim3(256), 0, st, ws.ranges, sorted_g,
                               ws.slot_base, ws.rec0, ws.rec1, ws.rec2, ws.rect, s.G, s.T, s.TX, s.W, s.H, ws.events,
                               map, C,
                               c0, nc, ws.partials, ws.slot_bits, ws.tile_order, ws.tile_work);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_gather_slots(s, ws, 2, st);
        if (e != hipSuccess) return e;
        if (s.G > 0)
            hipLaunchKernelGGL(k_sum_views, dim3((unsigned)((s.G + 255) / 256)), dim3(256), 0, st, s.G, s.V,
                               ws.rec_masks, ws.gv_sums, C, c0, nc, out);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Debug top-K contributor metadata: per pixel the K accepted contributions with
// the largest weight w = T alpha, in decreasing weight (a new weight passes only
// strictly smaller ones, so equal weights keep list order); unused entries are
// id -1, weight 0.  Sorted insertion into K register slots per pixel.
template <int K>
__global__ __launch_bounds__(256) void k_topk(const uint2* __restrict__ ranges, const uint32_t* __restrict__ sorted_g,
                                              const float4* __restrict__ rec0, const float4* __restrict__ rec1,
                                              const float4* __restrict__ rec2, int64_t G, int T, int TX, int W, int H,
                                              const uint8_t* __restrict__ events, int k_out,
                                              int32_t* __restrict__ ids_out, float* __restrict__ w_out,
                                              const uint32_t* __restrict__ tile_work) {
    __shared__ float4 s0[kAttrBatch];
    __shared__ float2 s1[kAttrBatch];
    __shared__ uint32_t s_g[kAttrBatch];
    __shared__ uint8_t s_evb[kAttrBatch];
    __shared__ uint8_t slist[4][kAttrBatch];

    const int tile = blockIdx.x;
    const int v = tile / T;
    const int t = tile - v * T;
    const int ty = t / TX, tx = t - ty * TX;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pxi = tx * kTile + (wave & 1) * 8 + (lane & 7);
    const int pyi = ty * kTile + (wave >> 1) * 8 + (lane >> 3);
    const bool inside = pxi < W && pyi < H;
    // pixel centre relative to the tile origin (entry centres are staged tile-relative too)
    const float px = (float)(pxi - tx * kTile) + 0.5f, py = (float)(pyi - ty * kTile) + 0.5f;
    const uint2 rg = ranges[tile];
    // the entries the render processed (every event lies there); an empty range ({~0u, 0}) has none
    const uint32_t rend = rg.x + min(tile_work[tile], rg.y > rg.x ? rg.y - rg.x : 0u);
    const int64_t vG = (int64_t)v * G;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    float tw[K];
    int32_t tid[K];
#pragma unroll
    for (int q = 0; q < K; ++q) {
        tw[q] = 0.0f;
        tid[q] = -1;
    }
    float Tr = 1.0f;
    bool done = !inside;

    for (uint32_t base = rg.x; base < rend; base += kAttrBatch) {
        if (__syncthreads_count(!done) == 0) break;
        const uint32_t i = base + threadIdx.x;
        if (threadIdx.x < kAttrBatch && i < rend) {
            const uint32_t g = sorted_g[i];
            const float4 a = rec0[vG + g];
            const float4 c = rec2[vG + g];
            s0[threadIdx.x] = make_float4(tile_centre(a.x, c.z, tx), tile_centre(a.y, c.w, ty), a.z, a.w);
            const float4 b = rec1[vG + g];
            s1[threadIdx.x] = make_float2(b.x, b.y);
            s_g[threadIdx.x] = g;
            s_evb[threadIdx.x] = events[i];
        }
        const int cnt = (int)min((uint32_t)kAttrBatch, rend - base);
        __syncthreads();
        if (__ballot(!done) != 0ull) {
            int nw = 0;
            for (int c = 0; c < cnt; c += 64) {
                const int j = c + lane;
                const bool hit = j < cnt && ((s_evb[j] >> wave) & 1u);
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
                const float2 b = s1[j];
                const float dx = px - a.x, dy = py - a.y;
                const float S = quad_S(a.z, a.w, b.x, dx, dy);
                const bool near = !done && S <= kSCutoff;
                const float aG = b.y * exp2_spec(-S);
                const float alpha = !(aG < kAlphaMax) ? kAlphaMax : aG;
                const bool pass = near && alpha >= kAlphaMin;
                const float tT = Tr * (1.0f - alpha);
                const bool sat = pass && tT < kTMin;
                const bool contrib = pass != sat;  // (sat implies pass: a mask difference, no second compare)
                done = done || sat;
                if (contrib && alpha * Tr > tw[K - 1]) {
                    float cw = alpha * Tr;
                    int32_t ci = (int32_t)s_g[j];
#pragma unroll
                    for (int q = 0; q < K; ++q) {
                        if (cw > tw[q]) {
                            const float sw = tw[q];
                            const int32_t si = tid[q];
                            tw[q] = cw;
                            tid[q] = ci;
                            cw = sw;
                            ci = si;
                        }
                    }
                }
                Tr = contrib ? tT : Tr;
            }
        }
        __syncthreads();
    }
    if (!inside) return;
    const int64_t o = (((int64_t)v * H + pyi) * W + pxi) * k_out;
#pragma unroll
    for (int q = 0; q < K; ++q)
        if (q < k_out) {
            ids_out[o + q] = tid[q];
            w_out[o + q] = tw[q];
        }
}

hipError_t launch_topk(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, int k, int32_t* ids, float* w,
                       hipStream_t st) {
    const int64_t tiles = (int64_t)s.V * s.T;
    if (tiles == 0) return hipSuccess;
#define GSR_LAUNCH_TOPK(KK)                                                                                       \
    hipLaunchKernelGGL(k_topk<KK>, dim3((unsigned)tiles), dim3(256), 0, st, ws.ranges, sorted_g, ws.rec0, ws.rec1, \
                       ws.rec2, s.G, s.T, s.TX, s.W, s.H, ws.events, k, ids, w, ws.tile_work)
    if (k <= 4) GSR_LAUNCH_TOPK(4);
    else if (k <= 8) GSR_LAUNCH_TOPK(8);
    else GSR_LAUNCH_TOPK(16);
#undef GSR_LAUNCH_TOPK
    return hipGetLastError();
}

}  // namespace gsr
