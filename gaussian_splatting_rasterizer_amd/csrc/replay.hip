// replay.hip -- analytic score replay and token assembly on gfx950.
//
// Stage 2 of the Renderer Score Tokens proposal ("Two-Stage Algorithm",
// Analytic Score Replay) and the "Exact Score Operators" / "Final Token".
//
// k_replay: the same tiles, lists, order and float32 decisions as the render.
// Each pixel re-walks its list keeping the transmittance T and, for every
// contribution, forms
//     S   = C_hat - P - T alpha c                     (suffix times T(1-alpha))
//     C+  = S / (T (1 - alpha) + eps)                 (suffix equation)
//     rho = <r, c - C+>,  r = C_hat - C_obs            (residual-suffix contrast)
//     w   = T alpha                                   (visibility weight)
//     M   = [o G < 0.99] and [T (1 - alpha) >= den_min]   (mask)
// The suffix enters rho only through <r, S>, so each pixel keeps that scalar,
// q = <r, C_hat - P>: it starts at <r, C_hat> and every contribution takes
// w <r, c> off it (one fused multiply-add per entry instead of three).
// and the seven per-pixel partials (the eighth slot of a stored partial is zero)
//     W += w, U_a += M w rho, U_mu += M w rho (p - mu), U_c += w r;
// the pair's partial then gets the conic applied to U_mu and the colour clamp
// mask applied to U_c (both constant over the pair).
// These suffice for every score block: with M set, alpha = o G, so
// T o grad_mu G rho = conic (p - mu) w rho and T alpha (1 - o) rho = (1 - o) w rho;
// the colour clamp mask and the SH basis are constant over a (Gaussian, view).
// The 64 lanes of a wave are reduced with a reduce-scatter built on the
// gfx950 lane permutations (permlane32/16 swaps, DPP row rotations) that leaves
// lane l holding component l >> 3 summed over the wave, only when some lane
// contributed; the four waves
// meet in LDS and one 32-byte partial per (tile, Gaussian) pair is stored with
// plain stores -- no atomics, so the result is deterministic.  The partial's
// slot is the record's slot base (a scan of tile counts in record order) plus
// the tile's row-major index in the record's rectangle, so one Gaussian's
// slots are contiguous per view and adjacent Gaussians' slots are adjacent.
// Only pairs at which some wave had an event are written (every other pair's
// partial is zero), and each written slot sets its bit in slot_bits.
//
// k_gather_slots: per record (record order), the sums of the pairs the replay
// wrote, stored only for records with such a pair; plus, per 64 records, a
// mask of the records that are live (not culled) and one of those reached.
// k_tokens: one thread per Gaussian; each view's terms in float32, their sums
// over the views, 1/Q and the eigenvalues in float64:
//     q_v = eps + W_v,  Q = eps + sum_v q_v,  gamma_v = q_v / Q
//     b_mu = sum_v gamma_v J_v^T s_mu_v = (1/Q) sum_v J_v^T (conic_v U_mu_v)
//     s_a  = (1/Q) sum_v (1 - o) U_a_v,   s_SH = (1/Q) sum_v M_color (B_v (x) U_c_v)
//     A    = lambda I + (1/Q) sum_v q_v J_v^T J_v
// with J_v the unclamped pixel-projection Jacobian, eigenvalues of A by the
// closed-form trigonometric solution for symmetric 3x3 matrices (descending),
// and writes z = [b_mu, s_a, s_SH, log Q, eig/(tr A + eps), log(tr A + eps)].
#include "gsr_internal.hpp"

namespace gsr {

// Entries staged per batch: 128 (about 25 KB of LDS, six blocks per CU) measured ahead of 96 (eight blocks per
// CU; the 512x960 compact scene 146 -> 143 us) and of 64, fewer barriers per tile outweighing the fewer blocks.
constexpr int kReplayBatch = 128;
static_assert(2 * kReplayBatch <= 256, "two flush threads per staged entry");

__global__ __launch_bounds__(256) void k_replay(const uint2* __restrict__ ranges, const uint32_t* __restrict__ sorted_g,
                                                const uint32_t* __restrict__ slot_base,
                                                const float4* __restrict__ rec0, const float4* __restrict__ rec1,
                                                const float4* __restrict__ rec2, const uint2* __restrict__ rect,
                                                int64_t G, int T, int TX, int W, int H, const float4* __restrict__ pixel, const float* __restrict__ observed,
                                                const uint8_t* __restrict__ events, float eps, float den_min,
                                                float4* __restrict__ partials, uint32_t* __restrict__ slot_bits,
                                                const uint32_t* __restrict__ tile_order,
                                                const uint32_t* __restrict__ tile_work) {
    // an entry's three staged vectors sit at the same byte offset of three arrays, so one offset (16 j,
    // kept in the wave's list) addresses all of them
    __shared__ float4 s0[kReplayBatch];        // {tile-relative centre (2), s1, s2}
    __shared__ float4 s1[kReplayBatch];        // {s3, opacity, colour r, colour g}
    __shared__ float4 s2[kReplayBatch];        // {colour b, unused}
    __shared__ uint8_t s_evb[kReplayBatch];    // event bits of each staged entry (bit w: wave w)
    __shared__ uint32_t s_slot[kReplayBatch];  // partial slot of each staged pair
    __shared__ uint8_t s_mask[kReplayBatch];   // colour clamp mask bits (pre-clamp colour finite and >= 0), r g b
    __shared__ uint32_t slist[4][kReplayBatch];
    __shared__ __align__(16) float sp[4][kReplayBatch][8];

    const int tile = (int)tile_order[blockIdx.x];
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
    const uint2 rg = ranges[tile];
    // the entries the render processed (every event lies there: past them the event bytes are not this frame's,
    // and a wave whose pixels are all done would leave its partial rows unwritten for one it names); an empty
    // range ({~0u, 0}) has none
    const uint32_t rend = rg.x + min(tile_work[tile], rg.y > rg.x ? rg.y - rg.x : 0u);
    const int64_t vG = (int64_t)v * G;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    float Ch0 = 0.f, Ch1 = 0.f, Ch2 = 0.f, r0 = 0.f, r1 = 0.f, r2 = 0.f;
    if (inside) {
        const int64_t pix = ((int64_t)v * H + pyi) * W + pxi;
        const float4 c = pixel[pix];
        Ch0 = c.x;
        Ch1 = c.y;
        Ch2 = c.z;
        r0 = Ch0 - observed[3 * pix];
        r1 = Ch1 - observed[3 * pix + 1];
        r2 = Ch2 - observed[3 * pix + 2];
    }
    float Tr = 1.0f;
    // <r, S> with S the suffix composite times the transmittance in front of it (C_hat minus the prefix colour)
    float q = __builtin_fmaf(r2, Ch2, __builtin_fmaf(r1, Ch1, r0 * Ch0));
    bool done = !inside;

    uint32_t base = rg.x;
    for (; base < rend; base += kReplayBatch) {
        if (__syncthreads_count(!done) == 0) break;
        const uint32_t i = base + threadIdx.x;
        if (threadIdx.x < kReplayBatch && i < rend) {
            const int64_t rid = vG + sorted_g[i];
            const float4 a = rec0[rid];
            const float4 b = rec1[rid];
            const float4 c = rec2[rid];
            const uint2 rc = rect[rid];
            s0[threadIdx.x] = make_float4(tile_centre(a.x, c.z, tx), tile_centre(a.y, c.w, ty), a.z, a.w);
            s1[threadIdx.x] = make_float4(b.x, b.y, clamp_colour(b.z), clamp_colour(b.w));
            s2[threadIdx.x] = make_float4(clamp_colour(c.x), 0.0f, 0.0f, 0.0f);
            s_evb[threadIdx.x] = events[i];
            // slot of this (tile, Gaussian) pair: the record's slot base + row-major tile index
            const uint32_t x0 = rc.x & 0xffffu, y0 = rc.x >> 16, wx = (rc.y & 0xffffu) - x0;
            s_slot[threadIdx.x] = slot_base[rid] + ((uint32_t)ty - y0) * wx + ((uint32_t)tx - x0);
            s_mask[threadIdx.x] = (uint8_t)((colour_ok(b.z) ? 1u : 0u) | (colour_ok(b.w) ? 2u : 0u) | (colour_ok(c.x) ? 4u : 0u));
        }
        const int cnt = (int)min((uint32_t)kReplayBatch, rend - base);
        // (a wave writes the partial row of every entry it walks; the flush reads only those rows)
        __syncthreads();
        if (__ballot(!done) != 0ull) {
            int nw = 0;
            for (int c = 0; c < cnt; c += 64) {
                const int j = c + lane;
                const bool hit = j < cnt && ((s_evb[j] >> wave) & 1u);
                const uint64_t m = __ballot(hit);
                if (hit) slist[wave][nw + __popcll(m & lt_mask)] = (uint32_t)(j * sizeof(float4));
                nw += __popcll(m);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // one entry: the float32 decisions and the state updates of every lane, and the eight values
            // whose wave sums are the entry's partial row
            auto step = [&](uint32_t off, float (&x)[8]) {
                const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(s0) + off);
                const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(s1) + off);
                const float cbl = reinterpret_cast<const float4*>(reinterpret_cast<const char*>(s2) + off)->x;
                // evaluated in every lane; the decisions mask lanes that are done or beyond the cut
                const float dx = px - a.x, dy = py - a.y;
                const float S = quad_S(a.z, a.w, b.x, dx, dy);
                const bool near = !done && S <= kSCutoff;
                const float aG = b.y * exp2_spec(-S);
                const bool clamped = !(aG < kAlphaMax);
                const float alpha = clamped ? kAlphaMax : aG;
                const bool pass = near && alpha >= kAlphaMin;
                const float tT = Tr * (1.0f - alpha);
                const bool sat = pass && tT < kTMin;
                const bool contrib = pass != sat;  // (sat implies pass: a mask difference, no second compare)
                done = done || sat;
                // some lane of the wave contributes or saturates at every listed entry (a wave's list ends
                // at its last such entry), so the partials are formed without testing for a contribution
                const float cr = b.z, cg = b.w;
                const float w = contrib ? alpha * Tr : 0.0f;
                const float rc = __builtin_fmaf(r2, cbl, __builtin_fmaf(r1, cg, r0 * cr));
                // <r, S> behind this entry: the prefix now includes it (lanes without a contribution
                // subtract zero)
                q = __builtin_fmaf(-w, rc, q);
                const float inv_den = __builtin_amdgcn_rcpf(tT + eps);
                // rho = <r, c - S / den> = <r, c> - <r, S> / den
                const float rho = __builtin_fmaf(-q, inv_den, rc);
                const float mw = (contrib && !clamped && tT >= den_min) ? w * rho : 0.0f;
                // the eighth component is never read (the flush stores zero there): rho, a value that
                // dies here, fills it without a register move
                x[0] = w;
                x[1] = mw;
                x[2] = mw * dx;
                x[3] = mw * dy;
                x[4] = w * r0;
                x[5] = w * r1;
                x[6] = w * r2;
                x[7] = rho;
                Tr = contrib ? tT : Tr;
            };
            // every lane of a group of eight holds its component's sum: all store (the same value to the
            // same word), so no lane mask is set up for the store
            // (sp[wave][j][lane >> 3]: rows of 32 bytes, so the row's byte offset is 2 off)
            char* spw = reinterpret_cast<char*>(&sp[wave][0][0]) + 4 * (lane >> 3);
            // two entries per round: the second entry's decisions follow the first's state updates, and the
            // two wave reductions, independent of each other, run interleaved
            int k = 0;
            for (; k + 1 < nw; k += 2) {
                const uint32_t o0 = slist[wave][k], o1 = slist[wave][k + 1];
                float x0[8], x1[8];
                step(o0, x0);
                step(o1, x1);
                const float red0 = wave_reduce8(x0, lane);
                const float red1 = wave_reduce8(x1, lane);
                *reinterpret_cast<float*>(spw + 2 * o0) = red0;
                *reinterpret_cast<float*>(spw + 2 * o1) = red1;
            }
            if (k < nw) {
                const uint32_t o0 = slist[wave][k];
                float x0[8];
                step(o0, x0);
                *reinterpret_cast<float*>(spw + 2 * o0) = wave_reduce8(x0, lane);
            }
        }
        __syncthreads();
        // one partial per entry at which some wave had an event (every other entry's partial is zero),
        // flagged in the slot bits for the gather
        if (threadIdx.x < 2 * cnt && s_evb[threadIdx.x >> 1] != 0) {
            const int j = threadIdx.x >> 1, h = threadIdx.x & 1;
            const uint32_t evb = s_evb[j];
            // the rows of the waves that walked the entry (every other wave's share is zero)
            float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if (!((evb >> w) & 1u)) continue;
                const float4 q = *reinterpret_cast<const float4*>(&sp[w][j][4 * h]);
                acc.x += q.x;
                acc.y += q.y;
                acc.z += q.z;
                acc.w += q.w;
            }
            // per pair: the conic applied to U_mu (from the exponent factors, k conic = L L^T) and the
            // colour clamp mask applied to U_c
            if (h == 0) {
                // (values only: no decision is taken on them)
                const float f1 = s0[j].z, f2 = s0[j].w, f3 = s1[j].x;
                const float ca = (f1 * f1) * kInvHalfLog2e, cb = (f1 * f2) * kInvHalfLog2e,
                            cc = __builtin_fmaf(f2, f2, f3 * f3) * kInvHalfLog2e;
                acc = make_float4(acc.x, acc.y, ca * acc.z + cb * acc.w, cb * acc.z + cc * acc.w);
            } else {
                const uint32_t m = s_mask[j];
                acc = make_float4(m & 1u ? acc.x : 0.0f, m & 2u ? acc.y : 0.0f, m & 4u ? acc.z : 0.0f, 0.0f);
            }
            const uint32_t slot = s_slot[j];
            partials[2 * (int64_t)slot + h] = acc;
            if (h == 0) atomicOr(&slot_bits[slot >> 5], 1u << (slot & 31u));
        }
    }
}

hipError_t launch_replay(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, const float* observed,
                         float eps, float den_min, hipStream_t st) {
    const int64_t tiles = (int64_t)s.V * s.T;
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_replay, dim3((unsigned)tiles), dim3(256), 0, st, ws.ranges, sorted_g,
                       ws.slot_base, ws.rec0, ws.rec1,
                       ws.rec2, ws.rect, s.G, s.T, s.TX, s.W, s.H, ws.pixel, observed, ws.events, eps, den_min,
                       ws.partials, ws.slot_bits, ws.tile_order, ws.tile_work);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// finalize
// ---------------------------------------------------------------------------
__device__ void sym3_eigen_desc(const double A[6] /* a00 a01 a02 a11 a12 a22 */, double ev[3]) {
#pragma clang fp contract(fast)
    const double a00 = A[0], a01 = A[1], a02 = A[2], a11 = A[3], a12 = A[4], a22 = A[5];
    const double p1 = a01 * a01 + a02 * a02 + a12 * a12;
    const double q = (a00 + a11 + a22) / 3.0;
    double e0, e1, e2;
    if (p1 == 0.0) {
        e0 = a00;
        e1 = a11;
        e2 = a22;
    } else {
        const double b00 = a00 - q, b11 = a11 - q, b22 = a22 - q;
        const double p2 = b00 * b00 + b11 * b11 + b22 * b22 + 2.0 * p1;
        const double p = sqrt(p2 / 6.0);
        const double ip = 1.0 / p;
        const double c00 = b00 * ip, c11 = b11 * ip, c22 = b22 * ip;
        const double c01 = a01 * ip, c02 = a02 * ip, c12 = a12 * ip;
        double r = 0.5 * (c00 * (c11 * c22 - c12 * c12) - c01 * (c01 * c22 - c12 * c02) +
                          c02 * (c01 * c12 - c11 * c02));
        r = r < -1.0 ? -1.0 : (r > 1.0 ? 1.0 : r);
        const double phi = acos(r) / 3.0;
        double sn, cs;
        sincos(phi, &sn, &cs);
        e0 = q + 2.0 * p * cs;
        // cos(phi + 2 pi / 3) = -cos(phi) / 2 - sin(phi) sqrt(3) / 2
        e2 = q - p * (cs + 1.7320508075688772935 * sn);
        e1 = 3.0 * q - e0 - e2;
    }
    // sort descending
    double t;
    if (e0 < e1) { t = e0; e0 = e1; e1 = t; }
    if (e1 < e2) { t = e1; e1 = e2; e2 = t; }
    if (e0 < e1) { t = e0; e0 = e1; e1 = t; }
    ev[0] = e0;
    ev[1] = e1;
    ev[2] = e2;
}

// Per (view, Gaussian) record, in record order: the sums of the partials the
// replay (or the backward traversal) wrote at the record's slots.  A record's
// slots [slot_base, slot_base + tile count) are contiguous, consecutive
// records' slots are adjacent, and the traversal set a bit for every slot it
// wrote.
constexpr int kGatherThreads = 256;

// NQ float4 per slot and per record: 2 for the score replay, 3 for the backward.
// Each thread takes kGatherRecs records 64 apart (a wave covers kGatherRecs
// runs of 64; one run per wave measured fastest: more waves, shorter chains of
// dependent loads per wave).  Per record a lane reads the bit words of its
// range (the first three together) and decides whether any slot
// was written; the ballot over one record index of the wave is then exactly that
// run's live and reached mask words.  The few reached records are summed by the
// whole wave, one record at a time: lane l takes slots l, l + 64, ... of the
// record, loads the partials of the set bits, and a fixed-order wave reduction
// leaves the sums in eight lanes, which store them together.  A record's loads
// are thus one round of independent loads instead of a chain of one per slot.
// Where most records are reached (single views with every Gaussian visible) a
// run with more than kGatherDenseRun reached records is summed lane per
// record instead, each lane keeping four slots' loads in flight.
constexpr int kGatherRecs = 1;
// A run with more reached records than this is summed lane per record instead.
constexpr int kGatherDenseRun = 8;
// Slots whose loads a lane keeps in flight at once in that dense case.
constexpr int kGatherInFlight = 4;

__device__ __forceinline__ uint32_t bit_range_mask(int32_t lo, int32_t hi) {  // bits [lo, hi) of a word, clipped
    lo = lo < 0 ? 0 : lo;
    hi = hi > 32 ? 32 : hi;
    if (hi <= lo) return 0u;
    return (hi >= 32 ? ~0u : ((1u << hi) - 1u)) & ~((1u << lo) - 1u);
}

template <int NQ>
__global__ __launch_bounds__(kGatherThreads) void k_gather_slots(int64_t VG,
                                                                 const uint32_t* __restrict__ tiles_touched,
                                                                 const uint32_t* __restrict__ slot_base,
                                                                 const uint32_t* __restrict__ slot_bits,
                                                                 const float4* __restrict__ partials,
                                                                 float4* __restrict__ gv_sums,
                                                                 uint64_t* __restrict__ rec_masks) {
    static_assert(NQ == 2 || NQ == 3, "two or three float4 per slot");
    const int lane = threadIdx.x & 63;
    const int64_t wbase =
        ((int64_t)blockIdx.x * (kGatherThreads / 64) + (threadIdx.x >> 6)) * (64 * kGatherRecs);
    if (wbase >= VG) return;  // the whole wave is past the end
    uint32_t tt[kGatherRecs], sa[kGatherRecs], b0[kGatherRecs], b1[kGatherRecs], b2[kGatherRecs];
#pragma unroll
    for (int j = 0; j < kGatherRecs; ++j) {
        const int64_t rid = wbase + 64 * j + lane;
        tt[j] = rid < VG ? tiles_touched[rid] : 0u;  // culled records touch no tile
        sa[j] = rid < VG ? slot_base[rid] : 0u;
    }
    // the first three bit words of each record's range (a word past the range reads as zero)
#pragma unroll
    for (int j = 0; j < kGatherRecs; ++j) {
        const uint32_t nwords = tt[j] ? ((sa[j] + tt[j] - 1u) >> 5) - (sa[j] >> 5) + 1u : 0u;
        b0[j] = nwords >= 1u ? slot_bits[sa[j] >> 5] : 0u;
        b1[j] = nwords >= 2u ? slot_bits[(sa[j] >> 5) + 1u] : 0u;
        b2[j] = nwords >= 3u ? slot_bits[(sa[j] >> 5) + 2u] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kGatherRecs; ++j) {
        const int64_t run = wbase + 64 * j;
        const bool live = tt[j] != 0u;
        // word k of the range holds bits [lo - 32 k, lo - 32 k + tt) of the record's slots
        const int32_t lo = (int32_t)(sa[j] & 31u), hi = lo + (int32_t)tt[j];
        b0[j] &= bit_range_mask(lo, hi);
        b1[j] &= bit_range_mask(lo - 32, hi - 32);
        b2[j] &= bit_range_mask(lo - 64, hi - 64);
        bool reached = (b0[j] | b1[j] | b2[j]) != 0u;
        if (!reached && hi > 96) {  // a range of more than three words: read on until a set bit
            for (uint32_t w = (sa[j] >> 5) + 3u; w <= (sa[j] + tt[j] - 1u) >> 5 && !reached; ++w) {
                const int32_t k = (int32_t)(w - (sa[j] >> 5));
                reached = (slot_bits[w] & bit_range_mask(lo - 32 * k, hi - 32 * k)) != 0u;
            }
        }
        const uint64_t live_mask = __ballot(live);
        uint64_t reached_mask = __ballot(reached);
        if (lane == 0 && run < VG) {
            rec_masks[2 * (run >> 6)] = live_mask;
            rec_masks[2 * (run >> 6) + 1] = reached_mask;
        }
        if (__popcll(reached_mask) > kGatherDenseRun) {
            // many reached records in this run: each lane sums its own record's flagged slots, four
            // slots' loads in flight at a time
            if (reached) {
                float4 acc[NQ];
#pragma unroll
                for (int q = 0; q < NQ; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
                const uint32_t w0 = sa[j] >> 5, wlast = (sa[j] + tt[j] - 1u) >> 5;
                const int32_t lo = (int32_t)(sa[j] & 31u), hi = lo + (int32_t)tt[j];
                uint32_t bits = b0[j];
                uint32_t w = w0;
                for (;;) {
                    int64_t sl[kGatherInFlight];
#pragma unroll
                    for (int u = 0; u < kGatherInFlight; ++u) {
                        while (bits == 0u && w < wlast) {
                            ++w;
                            const int32_t k = (int32_t)(w - w0);
                            bits = k == 1 ? b1[j] : k == 2 ? b2[j]
                                                           : slot_bits[w] & bit_range_mask(lo - 32 * k, hi - 32 * k);
                        }
                        sl[u] = -1;
                        if (bits) {
                            sl[u] = (int64_t)w * 32 + __builtin_ctz(bits);
                            bits &= bits - 1u;
                        }
                    }
                    float4 p[kGatherInFlight][NQ];
#pragma unroll
                    for (int u = 0; u < kGatherInFlight; ++u)
#pragma unroll
                        for (int q = 0; q < NQ; ++q)
                            p[u][q] = sl[u] >= 0 ? partials[NQ * sl[u] + q] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                    for (int u = 0; u < kGatherInFlight; ++u)
#pragma unroll
                        for (int q = 0; q < NQ; ++q) {
                            acc[q].x += p[u][q].x;
                            acc[q].y += p[u][q].y;
                            acc[q].z += p[u][q].z;
                            acc[q].w += p[u][q].w;
                        }
                    if (sl[kGatherInFlight - 1] < 0) break;
                }
#pragma unroll
                for (int q = 0; q < NQ; ++q) gv_sums[NQ * (run + lane) + q] = acc[q];
            }
            continue;
        }
        // few reached records: the wave sums each reached record of this run
        while (reached_mask) {
            const int src = __builtin_ctzll(reached_mask);
            reached_mask &= reached_mask - 1ull;
            const uint32_t r_sa = __builtin_amdgcn_readlane(sa[j], src);
            const uint32_t r_tt = __builtin_amdgcn_readlane(tt[j], src);
            const uint32_t r_b0 = __builtin_amdgcn_readlane(b0[j], src);
            const uint32_t r_b1 = __builtin_amdgcn_readlane(b1[j], src);
            const uint32_t r_b2 = __builtin_amdgcn_readlane(b2[j], src);
            const uint32_t r_lo = r_sa & 31u;
            float4 acc[NQ];
#pragma unroll
            for (int q = 0; q < NQ; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
            for (uint32_t o0 = 0; o0 < r_tt; o0 += 64u) {
                const uint32_t o = o0 + (uint32_t)lane;  // slot offset within the record
                bool set = false;
                if (o < r_tt) {
                    const uint32_t ob = r_lo + o, wi = ob >> 5;
                    const uint32_t word = wi == 0u ? r_b0 : wi == 1u ? r_b1 : wi == 2u ? r_b2
                                                                                      : slot_bits[(r_sa >> 5) + wi];
                    set = ((word >> (ob & 31u)) & 1u) != 0u;
                }
                if (set) {
                    const int64_t slot = (int64_t)(r_sa + o);
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        const float4 p = partials[NQ * slot + q];
                        acc[q].x += p.x;
                        acc[q].y += p.y;
                        acc[q].z += p.z;
                        acc[q].w += p.w;
                    }
                }
            }
            float* out = reinterpret_cast<float*>(gv_sums + NQ * (run + src));
            const float x0[8] = {acc[0].x, acc[0].y, acc[0].z, acc[0].w, acc[1].x, acc[1].y, acc[1].z, acc[1].w};
            const float s0 = wave_reduce8(x0, lane);
            if ((lane & 7) == 0) out[lane >> 3] = s0;
            if constexpr (NQ == 3) {
                const float x1[8] = {acc[2].x, acc[2].y, acc[2].z, acc[2].w, 0.f, 0.f, 0.f, 0.f};
                const float s1 = wave_reduce8(x1, lane);
                if ((lane & 7) == 0 && lane < 32) out[8 + (lane >> 3)] = s1;
            }
        }
    }
}

hipError_t launch_gather_slots(const Sizes& s, const Workspace& ws, int nq, hipStream_t st) {
    if (s.VG == 0) return hipSuccess;
    const int64_t per_block = (int64_t)kGatherThreads * kGatherRecs;
    const dim3 grid((unsigned)((s.VG + per_block - 1) / per_block)), block(kGatherThreads);
    if (nq == 3)
        hipLaunchKernelGGL(k_gather_slots<3>, grid, block, 0, st, s.VG, ws.tiles_touched, ws.slot_base,
                           ws.slot_bits, ws.partials, ws.gv_sums, ws.rec_masks);
    else
        hipLaunchKernelGGL(k_gather_slots<2>, grid, block, 0, st, s.VG, ws.tiles_touched, ws.slot_base,
                           ws.slot_bits, ws.partials, ws.gv_sums, ws.rec_masks);
    return hipGetLastError();
}

// One thread per Gaussian: cross-view aggregation and the token.  Each wave
// stages the tokens of half its lanes at a time in LDS and stores them as one
// coalesced span (half a wave's tokens take 32 * DT floats, so the staging
// leaves room for the waves the registers allow).  With GATHER (one view: a
// Gaussian is one record) the thread also sums its record's flagged slots
// itself, in slot order with kGatherInFlight slots' loads in flight, instead of
// reading the sums k_gather_slots left (no separate launch, no sums through
// memory): for up to kTokGatherMaxG Gaussians (measured: the 512x960 compact
// scene's finalize 50 -> 36 us; on 5.9M Gaussians, where the token stores bound
// the kernel, the gather's load chains cost 297 -> 356 us).
constexpr int kTokThreads = 128;
constexpr int64_t kTokGatherMaxG = 1 << 21;

// Sums of the flagged partials (two float4 per slot) of a record's slots [sa, sa + tt); false if none is flagged.
__device__ __forceinline__ bool sum_record_slots(uint32_t tt, uint32_t sa, const uint32_t* __restrict__ slot_bits,
                                                 const float4* __restrict__ partials, float4& s0, float4& s1) {
    s0 = make_float4(0.f, 0.f, 0.f, 0.f);
    s1 = s0;
    if (tt == 0u) return false;
    const uint32_t w0 = sa >> 5, wlast = (sa + tt - 1u) >> 5;
    const int32_t lo = (int32_t)(sa & 31u), hi = lo + (int32_t)tt;
    // the first three words of the range together (a word past the range reads as zero)
    const uint32_t c1 = w0 + 1u <= wlast ? slot_bits[w0 + 1u] : 0u;
    const uint32_t c2 = w0 + 2u <= wlast ? slot_bits[w0 + 2u] : 0u;
    uint32_t bits = slot_bits[w0] & bit_range_mask(lo, hi);
    const uint32_t b1 = c1 & bit_range_mask(lo - 32, hi - 32), b2 = c2 & bit_range_mask(lo - 64, hi - 64);
    uint32_t w = w0;
    bool any = false;
    for (;;) {
        int64_t sl[kGatherInFlight];
#pragma unroll
        for (int u = 0; u < kGatherInFlight; ++u) {
            while (bits == 0u && w < wlast) {
                ++w;
                const int32_t k = (int32_t)(w - w0);
                bits = k == 1 ? b1 : k == 2 ? b2 : slot_bits[w] & bit_range_mask(lo - 32 * k, hi - 32 * k);
            }
            sl[u] = -1;
            if (bits) {
                sl[u] = (int64_t)w * 32 + __builtin_ctz(bits);
                bits &= bits - 1u;
            }
        }
        float4 p[kGatherInFlight][2];
#pragma unroll
        for (int u = 0; u < kGatherInFlight; ++u) {
            p[u][0] = sl[u] >= 0 ? partials[2 * sl[u]] : make_float4(0.f, 0.f, 0.f, 0.f);
            p[u][1] = sl[u] >= 0 ? partials[2 * sl[u] + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kGatherInFlight; ++u) {
            s0.x += p[u][0].x;
            s0.y += p[u][0].y;
            s0.z += p[u][0].z;
            s0.w += p[u][0].w;
            s1.x += p[u][1].x;
            s1.y += p[u][1].y;
            s1.z += p[u][1].z;
            s1.w += p[u][1].w;
        }
        any = any || sl[0] >= 0;
        if (sl[kGatherInFlight - 1] < 0) break;
    }
    return any;
}

template <int D, bool GATHER>
__global__ __launch_bounds__(kTokThreads) void k_tokens(const float* __restrict__ means, const float* __restrict__ opac,
                                                        int64_t G, int V, CamPack cams,
                                                        const uint64_t* __restrict__ rec_masks,
                                                        const float4* __restrict__ gv_sums,
                                                        const uint32_t* __restrict__ tiles_touched,
                                                        const uint32_t* __restrict__ slot_base,
                                                        const uint32_t* __restrict__ slot_bits,
                                                        const float4* __restrict__ partials, double eps, double lambda,
                                                        float* __restrict__ tokens) {
#pragma clang fp contract(fast)
    constexpr int DT = 9 + 3 * D;
    __shared__ __align__(16) float s_tok[kTokThreads / 64][32 * DT];
    const int64_t g0 = (int64_t)blockIdx.x * kTokThreads;
    const int64_t g = g0 + threadIdx.x;
    float z[DT];
    if (g < G) {
        const float mx = means[3 * g], my = means[3 * g + 1], mz = means[3 * g + 2];
        const float one_minus_o = 1.0f - opac[g];
        double Q = eps;
        double bnum[3] = {0.0, 0.0, 0.0};
        double anum = 0.0;
        double Anum[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
        float shnum[3 * D];
#pragma unroll
        for (int k = 0; k < 3 * D; ++k) shnum[k] = 0.0f;

        // every view's live / reached bit first (at most 32 views), the mask loads of 8 views in flight together
        uint32_t live_bits = 0u, reach_bits = 0u;
        float4 n0 = make_float4(0.f, 0.f, 0.f, 0.f), n1 = n0;
        if constexpr (GATHER) {  // one view: the record is the Gaussian
            const uint32_t tt = tiles_touched[g];
            live_bits = tt != 0u ? 1u : 0u;
            reach_bits = sum_record_slots(tt, slot_base[g], slot_bits, partials, n0, n1) ? 1u : 0u;
        } else
        for (int v0 = 0; v0 < V; v0 += 8) {
            uint64_t lw[8], rw[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t rid = (int64_t)(v0 + u) * G + g;
                lw[u] = v0 + u < V ? rec_masks[2 * (rid >> 6)] : 0ull;
                rw[u] = v0 + u < V ? rec_masks[2 * (rid >> 6) + 1] : 0ull;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint64_t bit = 1ull << ((((int64_t)(v0 + u) * G + g)) & 63);
                live_bits |= (uint32_t)((lw[u] & bit) != 0ull) << (v0 + u);
                reach_bits |= (uint32_t)((rw[u] & bit) != 0ull) << (v0 + u);
            }
        }
        // the reached views' sums are loaded one reached view ahead of the arithmetic (reached implies live)
        const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
        uint32_t pending = reach_bits;
        if (!GATHER && pending) {
            const int64_t rid = (int64_t)__builtin_ctz(pending) * G + g;
            n0 = gv_sums[2 * rid];
            n1 = gv_sums[2 * rid + 1];
        }
        for (int v = 0; v < V; ++v) {
            if (!((live_bits >> v) & 1u)) {  // culled in this view: q = eps, J = 0, no scores
                Q += eps;
                continue;
            }
            const bool reached = ((reach_bits >> v) & 1u) != 0u;
            float4 p0 = zero4, p1 = zero4;
            if (reached) {
                p0 = n0;
                p1 = n1;
                pending &= pending - 1u;  // v was the lowest pending view
                if (!GATHER && pending) {
                    const int64_t rid = (int64_t)__builtin_ctz(pending) * G + g;
                    n0 = gv_sums[2 * rid];
                    n1 = gv_sums[2 * rid + 1];
                }
            }
            // this view's terms in float32 (each within a few ulp), summed over the views in float64
            const float q = (float)eps + p0.x;
            Q += (double)q;
            const float smx = p0.z, smy = p0.w;  // conic * U_mu

            const float* cam = cams.c[v];
            const float R0 = cam[0], R1 = cam[1], R2 = cam[2], R3 = cam[3], R4 = cam[4], R5 = cam[5], R6 = cam[6],
                        R7 = cam[7], R8 = cam[8];
            const float t0 = cam[9], t1 = cam[10], t2 = cam[11];
            const float fx = cam[12], fy = cam[13];
            const float tcx = R0 * mx + R1 * my + R2 * mz + t0;
            const float tcy = R3 * mx + R4 * my + R5 * mz + t1;
            const float tcz = R6 * mx + R7 * my + R8 * mz + t2;
            const float iz = __builtin_amdgcn_rcpf(tcz);  // tcz >= the near plane for a live record
            const float jp00 = fx * iz, jp02 = -fx * tcx * iz * iz;
            const float jp11 = fy * iz, jp12 = -fy * tcy * iz * iz;
            const float J0[3] = {jp00 * R0 + jp02 * R6, jp00 * R1 + jp02 * R7, jp00 * R2 + jp02 * R8};
            const float J1[3] = {jp11 * R3 + jp12 * R6, jp11 * R4 + jp12 * R7, jp11 * R5 + jp12 * R8};
#pragma unroll
            for (int k = 0; k < 3; ++k) bnum[k] += (double)(J0[k] * smx + J1[k] * smy);
            anum += (double)(one_minus_o * p0.y);
            Anum[0] += (double)(q * (J0[0] * J0[0] + J1[0] * J1[0]));
            Anum[1] += (double)(q * (J0[0] * J0[1] + J1[0] * J1[1]));
            Anum[2] += (double)(q * (J0[0] * J0[2] + J1[0] * J1[2]));
            Anum[3] += (double)(q * (J0[1] * J0[1] + J1[1] * J1[1]));
            Anum[4] += (double)(q * (J0[1] * J0[2] + J1[1] * J1[2]));
            Anum[5] += (double)(q * (J0[2] * J0[2] + J1[2] * J1[2]));

            if (reached) {
                // SH basis along the view direction (from the camera centre -R^T t) times the masked colour sums
                const float dx = mx + (R0 * t0 + R3 * t1 + R6 * t2);
                const float dy = my + (R1 * t0 + R4 * t1 + R7 * t2);
                const float dz = mz + (R2 * t0 + R5 * t1 + R8 * t2);
                const float il = __builtin_amdgcn_rsqf(dx * dx + dy * dy + dz * dz);
                float B[D];
                sh_basis_f32(dx * il, dy * il, dz * il, D, B);
#pragma unroll
                for (int k = 0; k < D; ++k) {
                    shnum[3 * k] += B[k] * p1.x;
                    shnum[3 * k + 1] += B[k] * p1.y;
                    shnum[3 * k + 2] += B[k] * p1.z;
                }
            }
        }

        const double iQ = 1.0 / Q;
        double A[6];
#pragma unroll
        for (int k = 0; k < 6; ++k) A[k] = Anum[k] * iQ;
        A[0] += lambda;
        A[3] += lambda;
        A[5] += lambda;
        double ev[3];
        sym3_eigen_desc(A, ev);
        const double tr = A[0] + A[3] + A[5];
        z[0] = (float)(bnum[0] * iQ);
        z[1] = (float)(bnum[1] * iQ);
        z[2] = (float)(bnum[2] * iQ);
        z[3] = (float)(anum * iQ);
        const float fiQ = (float)iQ;
#pragma unroll
        for (int k = 0; k < 3 * D; ++k) z[4 + k] = shnum[k] * fiQ;
        // the logarithms in float32: the tokens are float32, and rounding the argument first moves the result
        // by at most 2^-24 (absolute)
        z[4 + 3 * D] = logf((float)Q);
        const double itr = 1.0 / (tr + eps);
        z[5 + 3 * D] = (float)(ev[0] * itr);
        z[6 + 3 * D] = (float)(ev[1] * itr);
        z[7 + 3 * D] = (float)(ev[2] * itr);
        z[8 + 3 * D] = logf((float)(tr + eps));
    }
    // copy-out: lanes 0-31, then lanes 32-63, stage their tokens and the wave stores them as one span; a
    // half's span starts a multiple of 32 * DT floats (a multiple of 4) into the output, so it leaves in float4
    // stores when the caller's array is 16-byte aligned
    static_assert((32 * DT) % 4 == 0, "whole float4 per half wave");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float* st = s_tok[wave];
    const bool aligned = (reinterpret_cast<uintptr_t>(tokens) & 15u) == 0u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t gh = g0 + 64 * wave + 32 * h;  // first Gaussian of this half
        if ((lane >> 5) == h && g < G) {
#pragma unroll
            for (int k = 0; k < DT; ++k) st[(lane & 31) * DT + k] = z[k];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int64_t left = G - gh;
        const int nvalid = left <= 0 ? 0 : (int)(left < 32 ? left : 32) * DT;
        float* out = tokens + gh * DT;
        const int n4 = aligned ? nvalid >> 2 : 0;
        const float4* s4 = reinterpret_cast<const float4*>(st);
        float4* o4 = reinterpret_cast<float4*>(out);
        for (int i = lane; i < n4; i += 64) o4[i] = s4[i];
        for (int i = 4 * n4 + lane; i < nvalid; i += 64) out[i] = st[i];
        // every lane has read the staged half before the next one overwrites it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

bool tokens_gather(const Sizes& s) { return s.V == 1 && s.G <= kTokGatherMaxG; }

hipError_t launch_tokens(const gs_gaussians& sc, const CamPack& cams, const Sizes& s, const Workspace& ws, float eps,
                         float lambda, float* tokens, hipStream_t st) {
    if (s.G == 0) return hipSuccess;
    const dim3 block(kTokThreads), grid((unsigned)((s.G + kTokThreads - 1) / kTokThreads));
    const bool gather = tokens_gather(s);  // the token kernel sums the records' slots itself
#define GSR_LAUNCH_TOKENS_G(DD, GG)                                                                              \
    hipLaunchKernelGGL((k_tokens<DD, GG>), grid, block, 0, st, sc.means, sc.opacities, s.G, s.V, cams, ws.rec_masks, \
                       ws.gv_sums, ws.tiles_touched, ws.slot_base, ws.slot_bits, ws.partials, (double)eps,          \
                       (double)lambda, tokens)
#define GSR_LAUNCH_TOKENS(DD)                   \
    if (gather) GSR_LAUNCH_TOKENS_G(DD, true);  \
    else GSR_LAUNCH_TOKENS_G(DD, false)
    switch (s.d) {
        case 1: GSR_LAUNCH_TOKENS(1); break;
        case 4: GSR_LAUNCH_TOKENS(4); break;
        case 9: GSR_LAUNCH_TOKENS(9); break;
        default: GSR_LAUNCH_TOKENS(16); break;
    }
#undef GSR_LAUNCH_TOKENS
#undef GSR_LAUNCH_TOKENS_G
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// diagnostic: the decision exponential over an array
// ---------------------------------------------------------------------------
__global__ void k_exp2(const float* __restrict__ in, float* __restrict__ out, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        out[i] = exp2_spec(in[i]);
}

hipError_t launch_exp2(const float* in, float* out, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_exp2, dim3((unsigned)blocks), dim3(256), 0, st, in, out, n);
    return hipGetLastError();
}

}  // namespace gsr
