// binning.hip -- tile binning and contributor sorting on gfx950.
//
// Order of work (Stage 1, step "tile binning and contributor sorting" of the
// Renderer Score Tokens proposal; the order within a tile is front to back):
//   0. exclusive scan of the per-record tile counts in record order (v * G + g):
//      the base of each record's partial-score slots for the replay;
//   1. stable LSD radix sort of the (view, Gaussian) records by float32 depth
//      bits (culled records carry 0xffffffff and sink to the end); the last
//      pass also gathers each record's tile rectangle and count into depth order;
//   2. exclusive scan of the tile counts in depth order -> pair offsets;
//   3. emission of one (tile, Gaussian) pair per covered tile, in depth order,
//      row-major over each record's tile rectangle;
//   4. stable LSD radix sort of the pairs by global tile id (view * tiles +
//      tile) carrying the Gaussian index: because emission was in (depth bits,
//      Gaussian) order and the sort is stable, each tile's list ends up ordered
//      by (depth bits, Gaussian index) -- a total order, so the lists are unique;
//   5. per-tile [start, end) ranges.
// Only the pairs (a 4-byte tile key and a 4-byte Gaussian index per pass) go
// through the tile sort; the depth sort runs once over the records instead of
// over every pair.
//
// Radix passes (8-bit digits; 4 passes for depths, 2 x 6 bits for 4096 tiles):
// per 8192-key block a digit histogram (per-wave counts aggregated by ballot
// matching, so skewed digits cost nothing), one device-wide exclusive scan of
// the digit-major histogram table, then a scatter that ranks keys stably inside
// the block -- each wave takes 64 keys at a time in index order, finds the lanes
// holding the same digit with one ballot per digit bit and counts in per-wave
// LDS counters; waves own consecutive 1024-key slices so wave order is index
// order -- and reorders the block's keys in LDS so that each digit's run leaves
// as one contiguous, coalesced span (32 keys per run on average at 8 bits).
#include "gsr_internal.hpp"

namespace gsr {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int kScanTile = kScanThreads * kScanItems;     // 4096
constexpr int kRadixThreads = 512;
constexpr int kRadixWaves = kRadixThreads / 64;
constexpr int kRadixItems = 16;
constexpr int kRadixTile = kRadixThreads * kRadixItems;  // 8192
static_assert(kRadixTile == kSortTile, "radix tile size");
// Sorts of at most kSmallSortKeys keys use tiles of half the size: a pass over few tiles takes about as long
// as one tile does (ranking, look-back and scatter in series), and a half tile halves its ranking.
constexpr int kSmallRadixItems = kRadixItems / 2;
static_assert(kRadixThreads * kSmallRadixItems == kSmallSortTile, "small radix tile size");
// and sorts of at most kTinySortKeys keys (a depth sort of a few hundred thousand records) quarter tiles
constexpr int kTinyRadixItems = kRadixItems / 4;
static_assert(kRadixThreads * kTinyRadixItems == kTinySortTile, "tiny radix tile size");
constexpr int kMaxDigitBits = 8;
constexpr int kMaxBins = 1 << kMaxDigitBits;
constexpr int kMaxPasses = kSortMaxPasses;
constexpr int kCtlTotals = kSortCtlTotals;

RadixDigits radix_digits(int bits) {
    if (bits < 1) bits = 1;
    const int passes = (bits + kMaxDigitBits - 1) / kMaxDigitBits;
    return RadixDigits{bits, passes, (bits + passes - 1) / passes};
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t value) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, p, n, value);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// wave / block scans
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        T y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// exclusive scan across the block (NT threads), returns the block total via *total
template <typename T, int NT>
__device__ __forceinline__ T block_exclusive_scan(T x, T* total, T* lds /* NT/64 entries */) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T inc = wave_inclusive_scan(x, lane);
    if (lane == 63) lds[wave] = inc;
    __syncthreads();
    T base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        T s = lds[w];
        if (w < wave) base += s;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return base + inc - x;
}

// tile count of a scan item: the item itself, or the count of a packed rectangle
__device__ __forceinline__ uint32_t scan_item(uint32_t x, bool packed_rect) {
    if (!packed_rect) return x;
    return x == 0xffffffffu ? 0u : (((x >> 16) & 0xffu) + 1u) * ((x >> 24) + 1u);
}

// Two-kernel exclusive scan for large inputs: per-block totals, then each block's offset from the totals
// before it and the block's own scan.
__global__ __launch_bounds__(kScanThreads) void k_scan_reduce(const uint32_t* __restrict__ in, int64_t n,
                                                              uint64_t* __restrict__ bsum, bool packed_rect) {
    __shared__ uint64_t lds[kScanThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    uint64_t s = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int64_t k = base + i * kScanThreads + threadIdx.x;
        if (k < n) s += scan_item(in[k], packed_rect);
    }
    uint64_t tot;
    block_exclusive_scan<uint64_t, kScanThreads>(s, &tot, lds);
    if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

// `in` and `out` may alias (each block reads its whole slice before writing it).
// Each block sums the totals of the blocks before it (at most a few thousand
// words, L2-resident) instead of waiting for a separate scan of them; the last
// block writes the grand total.
__global__ __launch_bounds__(kScanThreads) void k_scan_down(const uint32_t* in, int64_t n,
                                                            const uint64_t* __restrict__ bsum, int64_t nb,
                                                            uint32_t* out, uint64_t* __restrict__ total,
                                                            bool packed_rect, uint64_t* host_total) {
    // padded so that thread t's 16 consecutive items (t*17 + i) are bank-conflict free
    __shared__ uint32_t s[kScanTile + kScanTile / 16];
    __shared__ uint32_t lds[kScanThreads / 64];
    __shared__ uint64_t lds64[kScanThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int e = i * kScanThreads + threadIdx.x;
        const int64_t k = base + e;
        s[e + e / 16] = k < n ? scan_item(in[k], packed_rect) : 0u;
    }
    uint64_t before = 0;
    for (int64_t j = threadIdx.x; j < (int64_t)blockIdx.x; j += kScanThreads) before += bsum[j];
    uint64_t boff;
    (void)block_exclusive_scan<uint64_t, kScanThreads>(before, &boff, lds64);
    if (threadIdx.x == 0 && (int64_t)blockIdx.x == nb - 1) {
        const uint64_t t = boff + bsum[blockIdx.x];
        *total = t;
        if (host_total) __hip_atomic_store(host_total, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    __syncthreads();
    const int t = threadIdx.x;
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) local += s[t * 17 + i];
    uint32_t tot;
    uint32_t run = (uint32_t)boff + block_exclusive_scan<uint32_t, kScanThreads>(local, &tot, lds);
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const uint32_t v = s[t * 17 + i];
        s[t * 17 + i] = run;
        run += v;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int e = i * kScanThreads + threadIdx.x;
        const int64_t k = base + e;
        if (k < n) out[k] = s[e + e / 16];
    }
}

// Single-pass exclusive scan.  Blocks take 4096-item tiles in the order they
// start (a ticket counter that only grows: this launch's tickets start at
// ticket_base), load their tile into LDS and publish its total; then every
// thread of the block waits for and adds a strided share of the totals of all
// earlier tiles (at most a few thousand words, up to 8 per thread in flight at
// once), so a block's offset takes one round of loads whatever its position.
// A tile waits only on tiles that started before it, and every tile publishes
// its total before it waits, so the waits always end.  A word is
// tag << 48 | value (48 bits, saturating: the pair count of any workspace fits
// far below, and a saturated total only fails the capacity check, never a
// tag).  `in` and `out` may alias (each block reads its whole slice before
// writing it).  The last tile writes the grand total (and to pinned host
// memory when host_total is given).
constexpr uint64_t kScanValueMask = (1ull << 48) - 1ull;
constexpr int64_t kScanOnePassTiles = 512;  // the single pass for up to 2M items

__global__ __launch_bounds__(kScanThreads) void k_scan_onepass(const uint32_t* in, int64_t n, uint32_t* out,
                                                               uint64_t* __restrict__ flags, uint32_t* ticket,
                                                               uint32_t ticket_base, uint32_t tag, int64_t nb,
                                                               uint64_t* __restrict__ total, bool packed_rect,
                                                               uint64_t* host_total) {
    // padded so that thread t's 16 consecutive items (t*17 + i) are bank-conflict free
    __shared__ uint32_t s[kScanTile + kScanTile / 16];
    __shared__ uint32_t lds[kScanThreads / 64];
    __shared__ uint64_t lds64[kScanThreads / 64];
    __shared__ uint32_t s_tile;
    __shared__ uint64_t s_excl;
    if (threadIdx.x == 0) s_tile = atomicAdd(ticket, 1u) - ticket_base;
    __syncthreads();
    const int64_t tile = s_tile;
    const int64_t base = tile * kScanTile;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int e = i * kScanThreads + threadIdx.x;
        const int64_t k = base + e;
        s[e + e / 16] = k < n ? scan_item(in[k], packed_rect) : 0u;
    }
    __syncthreads();
    const int t = threadIdx.x;
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) local += s[t * 17 + i];
    uint64_t btot;
    (void)block_exclusive_scan<uint64_t, kScanThreads>((uint64_t)local, &btot, lds64);
    btot = btot < kScanValueMask ? btot : kScanValueMask;
    const uint64_t agg_tag = (uint64_t)tag << 48;
    if (threadIdx.x == 0)
        __hip_atomic_store(flags + tile, agg_tag | btot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the totals of every earlier tile
    constexpr int kLB = 8;
    uint64_t acc = 0;
    for (int64_t k0 = 0; k0 < tile; k0 += (int64_t)kScanThreads * kLB) {
        uint64_t w[kLB];
#pragma unroll
        for (int u = 0; u < kLB; ++u) {
            const int64_t k = k0 + u * kScanThreads + threadIdx.x;
            w[u] = k < tile ? __hip_atomic_load(flags + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : agg_tag;
        }
#pragma unroll
        for (int u = 0; u < kLB; ++u) {
            const int64_t k = k0 + u * kScanThreads + threadIdx.x;
            while ((w[u] & ~kScanValueMask) != agg_tag) {  // not published yet (a word past tile is agg_tag | 0)
                __builtin_amdgcn_s_sleep(1);
                w[u] = __hip_atomic_load(flags + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            acc += w[u] & kScanValueMask;
        }
    }
    uint64_t excl;
    (void)block_exclusive_scan<uint64_t, kScanThreads>(acc, &excl, lds64);
    excl = excl < kScanValueMask ? excl : kScanValueMask;
    if (threadIdx.x == 0) {
        s_excl = excl;
        if (tile == nb - 1) {
            const uint64_t inc = excl + btot < kScanValueMask ? excl + btot : kScanValueMask;
            *total = inc;
            if (host_total) __hip_atomic_store(host_total, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
    __syncthreads();
    const uint64_t boff = s_excl;
    uint32_t tot;
    uint32_t run = (uint32_t)boff + block_exclusive_scan<uint32_t, kScanThreads>(local, &tot, lds);
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const uint32_t v = s[t * 17 + i];
        s[t * 17 + i] = run;
        run += v;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int e = i * kScanThreads + threadIdx.x;
        const int64_t k = base + e;
        if (k < n) out[k] = s[e + e / 16];
    }
}

__global__ void k_zero_u64(uint64_t* __restrict__ p, uint64_t* host_p) {
    *p = 0ull;
    if (host_p) __hip_atomic_store(host_p, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

hipError_t launch_scan_u32(const uint32_t* in, int64_t n, uint32_t* out, ScanState& ss, uint64_t* total,
                           hipStream_t st, bool packed_rect_in, uint64_t* host_total) {
    const int64_t nb = (n + kScanTile - 1) / kScanTile;
    if (nb == 0) {
        hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(1), 0, st, total, host_total);
        return hipGetLastError();
    }
    if (nb > kScanOnePassTiles) {
        // many tiles: the single pass's ticket and waits cost more than a second launch (measured)
        hipLaunchKernelGGL(k_scan_reduce, dim3((unsigned)nb), dim3(kScanThreads), 0, st, in, n, ss.flags,
                           packed_rect_in);
        hipLaunchKernelGGL(k_scan_down, dim3((unsigned)nb), dim3(kScanThreads), 0, st, in, n, ss.flags, nb, out,
                           total, packed_rect_in, host_total);
        // the block totals overwrote the tagged words: clear them before the next single pass
        *ss.epoch = 0;
        return hipGetLastError();
    }
    // the tile words and the ticket are cleared on first use and before the tag or the ticket could wrap
    if (*ss.epoch == 0 || *ss.epoch >= kScanEpochLimit || *ss.ticket_base > 0xc0000000u) {
        hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(ss.flags), 2 * ss.flags_cap, 0u, st);
        if (e == hipSuccess) e = launch_fill_u32(ss.ticket, 1, 0u, st);
        if (e != hipSuccess) return e;
        *ss.epoch = 0;
        *ss.ticket_base = 0;
    }
    const uint32_t tag = ++*ss.epoch;
    const uint32_t tb = *ss.ticket_base;
    *ss.ticket_base += (uint32_t)nb;
    hipLaunchKernelGGL(k_scan_onepass, dim3((unsigned)nb), dim3(kScanThreads), 0, st, in, n, out, ss.flags, ss.ticket,
                       tb, tag, nb, total, packed_rect_in, host_total);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// radix sort
// ---------------------------------------------------------------------------
// Lanes of the wave holding the same digit (one ballot per digit bit); invalid lanes never match.  A lane
// differs from this one where some bit's ballot disagrees with this lane's bit: the ballot XOR this lane's bit
// sign-extended, ORed over the bits (a bit extract, a compare and two 32-bit XOR / OR halves per bit).
__device__ __forceinline__ uint64_t match_peers(uint32_t dgt, int bits, bool valid) {
    uint32_t dlo = ~(uint32_t)__ballot(valid), dhi = ~(uint32_t)(__ballot(valid) >> 32);
#pragma unroll
    for (int b = 0; b < kMaxDigitBits; ++b) {
        if (b >= bits) break;
        const uint32_t s = (uint32_t)__builtin_amdgcn_sbfe((int)dgt, b, 1);  // this lane's bit, sign-extended
        const uint64_t m = __ballot(s != 0u);
        dlo |= (uint32_t)m ^ s;
        dhi |= (uint32_t)(m >> 32) ^ s;
    }
    return ~(((uint64_t)dhi << 32) | dlo);
}

// Number of lanes below this one set in m.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Digit counts of every pass in one read of the keys: per-block LDS
// histograms, written per block to part[block][pass * 256 + digit].  Each
// thread reads two 4-key vectors per step and keeps, per pass, a run of equal
// digits in registers that it adds to LDS only when the digit changes, so
// skewed digits (the exponent byte of depths) do not pile atomics on one bin.
constexpr int kHistThreads = 1024;
constexpr int kHistMaxBlocks = kSortPartBlocks;

template <int PASSES>
__device__ __forceinline__ void hist_count(uint32_t key, int dbits, int bits, uint32_t (&cur)[PASSES],
                                           uint32_t (&run)[PASSES], uint32_t* h) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int shift = p * dbits;
        const int pb = shift + dbits <= bits ? dbits : bits - shift;
        const uint32_t d = (key >> shift) & ((1u << pb) - 1u);
        if (d != cur[p]) {
            if (run[p]) atomicAdd(&h[p * kMaxBins + cur[p]], run[p]);
            cur[p] = d;
            run[p] = 1u;
        } else {
            ++run[p];
        }
    }
}

template <int PASSES>
__global__ __launch_bounds__(kHistThreads) void k_digit_hist(const uint32_t* __restrict__ keys, int64_t n, int dbits,
                                                             int bits, uint32_t* __restrict__ part) {
    __shared__ uint32_t h[kMaxPasses * kMaxBins];
    for (int i = threadIdx.x; i < kMaxPasses * kMaxBins; i += kHistThreads) h[i] = 0u;
    __syncthreads();
    uint32_t cur[PASSES], run[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        cur[p] = 0u;
        run[p] = 0u;
    }
    const int64_t n4 = n >> 2;
    const uint4* k4 = reinterpret_cast<const uint4*>(keys);
    const int64_t stride = (int64_t)gridDim.x * kHistThreads;
    // eight 4-key vectors per thread and round, all loads in flight before the counting
    constexpr int kU = 8;
    for (int64_t q0 = (int64_t)blockIdx.x * kHistThreads + threadIdx.x; q0 < n4; q0 += kU * stride) {
        uint4 x[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t q = q0 + u * stride;
            x[u] = q < n4 ? k4[q] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (q0 + u * stride >= n4) break;
            hist_count<PASSES>(x[u].x, dbits, bits, cur, run, h);
            hist_count<PASSES>(x[u].y, dbits, bits, cur, run, h);
            hist_count<PASSES>(x[u].z, dbits, bits, cur, run, h);
            hist_count<PASSES>(x[u].w, dbits, bits, cur, run, h);
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) hist_count<PASSES>(keys[4 * n4 + threadIdx.x], dbits, bits, cur, run, h);
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        if (run[p]) atomicAdd(&h[p * kMaxBins + cur[p]], run[p]);
    __syncthreads();
    for (int i = threadIdx.x; i < PASSES * kMaxBins; i += kHistThreads)
        part[(int64_t)blockIdx.x * (kMaxPasses * kMaxBins) + i] = h[i];
}

// Totals of the per-block histograms: block b sums bins [64 b, 64 b + 64) of
// the pass-major table, its 16 waves over 16 histogram blocks each with every
// load in flight at once; block 0 also zeroes the passes' tile tickets.  With
// zero_rows it then clears its bins in all kHistMaxBlocks rows, which leaves
// the table zero for the next producer that adds into it (the pair emission).
__global__ __launch_bounds__(1024) void k_digit_totals(uint32_t* __restrict__ part, int nblocks,
                                                       uint32_t* __restrict__ ctl, bool zero_rows) {
    static_assert(kHistMaxBlocks <= 16 * 16, "one load per wave and row");
    __shared__ uint32_t s[16][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bin = blockIdx.x * 64 + lane;
    uint32_t x[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int r = wave * 16 + u;
        x[u] = r < nblocks ? part[(int64_t)r * (kMaxPasses * kMaxBins) + bin] : 0u;
    }
    uint32_t acc = 0u;
#pragma unroll
    for (int u = 0; u < 16; ++u) acc += x[u];
    if (zero_rows) {
#pragma unroll
        for (int u = 0; u < 16; ++u) part[(int64_t)(wave * 16 + u) * (kMaxPasses * kMaxBins) + bin] = 0u;
    }
    s[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        uint32_t t = 0u;
#pragma unroll
        for (int w = 0; w < 16; ++w) t += s[w][lane];
        ctl[kCtlTotals + bin] = t;
    }
    if (blockIdx.x == 0 && threadIdx.x < kMaxPasses) ctl[threadIdx.x] = 0u;
}


// One radix pass (see the file header).  Blocks take their tile of keys in
// the order they start (a ticket counter), publish their per-digit counts and
// resolve their global offsets by looking back over earlier tiles' published
// counts: a word per (tile, digit) holding the count and a tag -- the pass's
// epoch and whether the count is the inclusive prefix of all tiles up to this
// one or only this tile's own.  A tile publishes its own counts as soon as it
// has ranked its keys, orders them in LDS, and only then looks back, so the
// wait overlaps its own work.  A tile only waits on tiles that started before
// it, and every tile publishes before it waits, so the chain always resolves.
// Tile rectangles of the records can ride along (RectCarry): packed to 32 bits
// from the record-order array in the first pass, reordered through LDS in a
// second round after the keys, and unpacked with their tile counts in the last
// pass; or, when the tile grid is too large to pack, gathered by record in the
// last pass.  keys_out may be null.
// kPackedMid / kPackedLast: 32-bit words (sort key above bit rc.key_shift, the value below) sorted with no
// separate value array; the last pass writes the value bits and records every key's range.
enum RadixMode { kPlain = 0, kCarryRect = 1, kGatherRect = 2, kRanges = 3, kPackedMid = 4, kPackedLast = 5 };

template <int MODE, int ITEMS>
__global__ __launch_bounds__(kRadixThreads, 4) void k_onesweep(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in, int64_t n, int shift, int bits,
    uint32_t* __restrict__ ticket, const uint32_t* __restrict__ digit_tot, uint64_t* __restrict__ lookback,
    uint32_t epoch, uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out, RectCarry rc) {
    constexpr int kTileKeys = kRadixThreads * ITEMS;
    __shared__ uint32_t cnt[kRadixWaves][kMaxBins];  // per-wave counts, then per-wave block-local bases
    __shared__ uint32_t gdelta[kMaxBins];            // global position - block-local position, per digit
    __shared__ uint64_t scan_lds[kRadixThreads / 64];
    __shared__ uint32_t skey[kTileKeys];
    constexpr bool kPacked = MODE == kPackedMid || MODE == kPackedLast;
    __shared__ uint32_t sval[kPacked ? 1 : kTileKeys];
    __shared__ uint32_t s_tile;
    const int nbins = 1 << bits;
    const uint32_t mask = (uint32_t)nbins - 1u;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < kRadixWaves * kMaxBins; i += kRadixThreads) (&cnt[0][0])[i] = 0u;
    if (threadIdx.x == 0) s_tile = atomicAdd(ticket, 1u);
    __syncthreads();
    const int64_t tile = s_tile;

    const int64_t bbase = tile * kTileKeys;
    // element indices within the tile, 32-bit (cheap to recompute where needed)
    const int nblk = (int)(n - bbase < kTileKeys ? n - bbase : kTileKeys);
    const int wbase = wave * (kTileKeys / kRadixWaves) + lane;
    uint32_t key[ITEMS], val[ITEMS], rank[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int e = wbase + i * 64;
        const bool valid = e < nblk;
        key[i] = valid ? keys_in[bbase + e] : 0u;
        val[i] = (valid && !kPacked) ? (vals_in ? vals_in[bbase + e] : (uint32_t)(bbase + e)) : 0u;
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const bool valid = wbase + i * 64 < nblk;
        const uint32_t dgt = (key[i] >> shift) & mask;
        const uint64_t peers = match_peers(dgt, bits, valid);
        const uint32_t below = lanes_below(peers);
        const uint32_t c = valid ? cnt[wave][dgt] : 0u;
        rank[i] = c + below;
        if (valid && below == 0u) cnt[wave][dgt] = c + (uint32_t)__popcll(peers);
    }
    __syncthreads();
    // publish this tile's digit counts first, so later tiles can look past it
    // while this one is still ordering its keys
    const int dgt = threadIdx.x;
    uint32_t tot = 0, gtot = 0;
    uint64_t* mine = lookback + tile * kMaxBins + dgt;
    const uint32_t tag = epoch << 1;
    if (dgt < nbins) {
#pragma unroll
        for (int w = 0; w < kRadixWaves; ++w) tot += cnt[w][dgt];
        gtot = digit_tot[dgt];
        __hip_atomic_store(mine, ((uint64_t)(tile == 0 ? tag | 1u : tag) << 32) | tot, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    // block-local digit offsets and the pass's global digit offsets in one
    // 64-bit scan: (digit total << 32) + block count, one digit per thread
    uint64_t both_total;
    const uint64_t both = block_exclusive_scan<uint64_t, kRadixThreads>(((uint64_t)gtot << 32) | tot, &both_total,
                                                                        scan_lds);
    const uint32_t loff = (uint32_t)both;
    const uint32_t digit_off = (uint32_t)(both >> 32);
    if (dgt < nbins) {
        uint32_t s = loff;
#pragma unroll
        for (int w = 0; w < kRadixWaves; ++w) {
            const uint32_t c = cnt[w][dgt];
            cnt[w][dgt] = s;
            s += c;
        }
    }
    __syncthreads();
    // block-local reorder: each digit's keys become one contiguous run; the LDS
    // positions (< 8192) are kept two to a register for a carried second reorder
    uint32_t lpk[ITEMS / 2];
#pragma unroll
    for (int i = 0; i < ITEMS / 2; ++i) lpk[i] = 0u;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        if (wbase + i * 64 >= nblk) continue;
        const uint32_t lp = cnt[wave][(key[i] >> shift) & mask] + rank[i];
        skey[lp] = key[i];
        if (!kPacked) sval[lp] = val[i];
        lpk[i >> 1] |= lp << (16 * (i & 1));
    }
    // decoupled look-back over the earlier tiles' published counts
    if (dgt < nbins) {
        uint32_t excl = 0;
        if (tile > 0) {
            // look back in windows of 8 predecessors, all loads in flight together
            constexpr int kWin = 8;
            int64_t j = tile - 1;
            for (;;) {
                uint64_t w[kWin];
#pragma unroll
                for (int q = 0; q < kWin; ++q)
                    w[q] = (j - q >= 0) ? __hip_atomic_load(lookback + (j - q) * kMaxBins + dgt, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)
                                        : 0ull;
                int used = 0;
                bool fin = false;
#pragma unroll
                for (int q = 0; q < kWin; ++q) {
                    const uint32_t h = (uint32_t)(w[q] >> 32);
                    if (fin || used != q || (h & ~1u) != tag) continue;
                    excl += (uint32_t)w[q];
                    used = q + 1;
                    fin = (h & 1u) != 0u;
                }
                if (fin) break;
                j -= used;
                if (used == 0) __builtin_amdgcn_s_sleep(1);
            }
            __hip_atomic_store(mine, ((uint64_t)(tag | 1u) << 32) | (excl + tot), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        gdelta[dgt] = digit_off + excl - loff;
    }
    __syncthreads();
    if (MODE == kCarryRect) {
        // keys and values out; each element's output position is parked in the value buffer
#pragma unroll 4
        for (int i = 0; i < ITEMS; ++i) {
            const int lp = i * kRadixThreads + threadIdx.x;
            if (lp >= nblk) break;
            const uint32_t k = skey[lp];
            const uint32_t pos = gdelta[(k >> shift) & mask] + (uint32_t)lp;
            if (keys_out) keys_out[pos] = k;
            vals_out[pos] = sval[lp];
            sval[lp] = pos;
        }
        // second reorder, through the key buffer: the carried rectangles, loaded only now
        __syncthreads();
        uint32_t q[ITEMS];
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {  // all loads in flight, then the LDS stores
            const int e = wbase + i * 64;
            q[i] = 0u;
            if (e < nblk) q[i] = rc.pack_src ? pack_rect(rc.pack_src[bbase + e]) : rc.pay_in[bbase + e];
        }
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            if (wbase + i * 64 >= nblk) continue;
            skey[(lpk[i >> 1] >> (16 * (i & 1))) & 0xffffu] = q[i];
        }
        __syncthreads();
#pragma unroll 4
        for (int i = 0; i < ITEMS; ++i) {
            const int lp = i * kRadixThreads + threadIdx.x;
            if (lp >= nblk) break;
            const uint32_t q = skey[lp];
            const uint32_t pos = sval[lp];
            if (rc.pay_out) {
                rc.pay_out[pos] = q;
            } else {
                const uint2 r = unpack_rect(q);
                rc.rect_out[pos] = r;
                rc.tt_out[pos] = ((r.y & 0xffffu) - (r.x & 0xffffu)) * ((r.y >> 16) - (r.x >> 16));
            }
        }
        return;
    }
    uint32_t pos[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int lp = i * kRadixThreads + threadIdx.x;
        const bool ok = lp < nblk;
        const uint32_t k = ok ? skey[lp] : 0u;
        pos[i] = gdelta[(k >> shift) & mask] + (uint32_t)lp;
        if (ok && kPacked) {
            if (MODE == kPackedMid) {
                keys_out[pos[i]] = k;
            } else {
                vals_out[pos[i]] = k & rc.low_mask;
                const uint32_t key_k = k >> rc.key_shift;
                if (lp == 0 || (skey[lp - 1] >> rc.key_shift) != key_k) atomicMin(&rc.ranges[key_k].x, pos[i]);
                if (lp == nblk - 1 || (skey[lp + 1] >> rc.key_shift) != key_k)
                    atomicMax(&rc.ranges[key_k].y, pos[i] + 1u);
            }
        } else if (ok) {
            if (keys_out) keys_out[pos[i]] = k;
            vals_out[pos[i]] = sval[lp];
            if (MODE == kRanges) {
                // equal keys are adjacent in the tile and contiguous in the output across tiles:
                // a key's range is the min / max over the tiles of its first / last position
                if (lp == 0 || skey[lp - 1] != k) atomicMin(&rc.ranges[k].x, pos[i]);
                if (lp == nblk - 1 || skey[lp + 1] != k) atomicMax(&rc.ranges[k].y, pos[i] + 1u);
            }
        }
    }
    if (MODE == kGatherRect) {
        // final depth pass without a carried rectangle: gather it by record, all gathers in flight together
        uint2 r[ITEMS];
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int lp = i * kRadixThreads + threadIdx.x;
            r[i] = lp < nblk ? rc.gather_src[sval[lp]] : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int lp = i * kRadixThreads + threadIdx.x;
            if (lp >= nblk) continue;
            rc.rect_out[pos[i]] = r[i];
            rc.tt_out[pos[i]] = ((r[i].y & 0xffffu) - (r[i].x & 0xffffu)) * ((r[i].y >> 16) - (r[i].x >> 16));
        }
    }
}

hipError_t launch_radix_sort(const uint32_t* keys_in, const uint32_t* vals_in, int64_t n, int bits,
                             uint32_t* kbuf0, uint32_t* kbuf1, uint32_t* vbuf0, uint32_t* vbuf1,
                             const RectSort* rs, uint2* ranges, bool hist_ready, int key_shift,
                             const SortScratch& sc, uint32_t* epoch, hipStream_t st, uint32_t** keys_out,
                             uint32_t** vals_out) {
    const RadixDigits rd = radix_digits(bits);
    bits = rd.bits;
    const int passes = rd.passes, dbits = rd.dbits;
    const bool tiny = n <= kTinySortKeys;
    const bool small = n <= kSmallSortKeys;
    const int64_t tile_keys = tiny ? kTinySortTile : small ? kSmallSortTile : kRadixTile;
    const int64_t nb = (n + tile_keys - 1) / tile_keys;
    // packed words: key bits [key_shift, key_shift + bits), counted beforehand, no value array, no rectangles
    const bool packed = key_shift > 0;
    // a single pass cannot read the packed rectangles from the array it writes them to
    if (rs && rs->out_packed && (!rs->pay_a || (passes == 1 && rs->pay_init == rs->tt_out))) return hipErrorInvalidValue;
    if (packed && (!hist_ready || vals_in || rs || !ranges || key_shift + bits > 32)) return hipErrorInvalidValue;
    uint32_t* kb[2] = {kbuf0, kbuf1};
    uint32_t* vb[2] = {vbuf0, vbuf1};
    if (keys_out) *keys_out = kb[(passes - 1) & 1];
    if (vals_out) *vals_out = vb[(passes - 1) & 1];
    if (n <= 0) return hipSuccess;
    int64_t hb = (n + 8 * kHistThreads - 1) / (8 * kHistThreads);
    if (hb > kHistMaxBlocks) hb = kHistMaxBlocks;
    if (hist_ready) hb = kHistMaxBlocks;  // the producer of the keys left their digit counts in every row
    else
    switch (passes) {
        case 1: hipLaunchKernelGGL(k_digit_hist<1>, dim3((unsigned)hb), dim3(kHistThreads), 0, st, keys_in, n, dbits, bits, sc.part); break;
        case 2: hipLaunchKernelGGL(k_digit_hist<2>, dim3((unsigned)hb), dim3(kHistThreads), 0, st, keys_in, n, dbits, bits, sc.part); break;
        case 3: hipLaunchKernelGGL(k_digit_hist<3>, dim3((unsigned)hb), dim3(kHistThreads), 0, st, keys_in, n, dbits, bits, sc.part); break;
        default: hipLaunchKernelGGL(k_digit_hist<4>, dim3((unsigned)hb), dim3(kHistThreads), 0, st, keys_in, n, dbits, bits, sc.part); break;
    }
    // a sort that counted its own digits leaves the histogram table zero for the pair emission
    hipLaunchKernelGGL(k_digit_totals, dim3((unsigned)(passes * kMaxBins / 64)), dim3(1024), 0, st, sc.part, (int)hb,
                       sc.ctl, !hist_ready);
    const uint32_t* ksrc = keys_in;
    const uint32_t* vsrc = vals_in;
    for (int p = 0; p < passes; ++p) {
        const int shift = p * dbits + key_shift;
        const int pb = (p * dbits + dbits <= bits) ? dbits : bits - p * dbits;
        const bool last = p == passes - 1;
        uint32_t* kdst = (last && !keys_out) ? nullptr : kb[p & 1];
        uint32_t* vdst = vb[p & 1];
        const uint32_t ep = next_epoch(epoch);
        RectCarry rc{};
        if (rs && rs->pay_a) {  // carried: pack in pass 0, ping-pong, unpack in the last pass
            if (p == 0) {  // packed by the producer of the records, or packed here on load
                if (rs->pay_init) rc.pay_in = rs->pay_init;
                else rc.pack_src = rs->rect;
            } else {
                rc.pay_in = p & 1 ? rs->pay_a : rs->pay_b;
            }
            if (last && rs->out_packed) {
                rc.pay_out = rs->tt_out;
            } else if (last) {
                rc.rect_out = rs->rect_out;
                rc.tt_out = rs->tt_out;
            } else {
                rc.pay_out = p & 1 ? rs->pay_b : rs->pay_a;
            }
            if (passes == 1) {  // a single pass packs (or reads the packed form) and unpacks
                rc.pack_src = rs->pay_init ? nullptr : rs->rect;
                rc.pay_in = rs->pay_init;
            }
        } else if (rs && last) {
            rc.gather_src = rs->rect;
            rc.rect_out = rs->rect_out;
            rc.tt_out = rs->tt_out;
        } else if (!rs && last) {
            rc.ranges = ranges;
        }
        rc.key_shift = key_shift;
        rc.low_mask = packed ? (1u << key_shift) - 1u : ~0u;
        const int mode = packed                     ? (last ? kPackedLast : kPackedMid)
                         : (rc.pack_src || rc.pay_in) ? kCarryRect
                         : rc.gather_src            ? kGatherRect
                         : rc.ranges                ? kRanges
                                                    : kPlain;
#define GSR_ONESWEEP(M)                                                                                        \
    do {                                                                                                       \
        if (tiny)                                                                                              \
            hipLaunchKernelGGL((k_onesweep<M, kTinyRadixItems>), dim3((unsigned)nb), dim3(kRadixThreads), 0, st,  \
                               ksrc, vsrc, n, shift, pb, sc.ctl + p, sc.ctl + kCtlTotals + p * kMaxBins,         \
                               sc.lookback, ep, kdst, vdst, rc);                                               \
        else if (small)                                                                                        \
            hipLaunchKernelGGL((k_onesweep<M, kSmallRadixItems>), dim3((unsigned)nb), dim3(kRadixThreads), 0, st, \
                               ksrc, vsrc, n, shift, pb, sc.ctl + p, sc.ctl + kCtlTotals + p * kMaxBins,         \
                               sc.lookback, ep, kdst, vdst, rc);                                               \
        else                                                                                                   \
            hipLaunchKernelGGL((k_onesweep<M, kRadixItems>), dim3((unsigned)nb), dim3(kRadixThreads), 0, st,     \
                               ksrc, vsrc, n, shift, pb, sc.ctl + p, sc.ctl + kCtlTotals + p * kMaxBins,         \
                               sc.lookback, ep, kdst, vdst, rc);                                               \
    } while (0)
        if (mode == kCarryRect) GSR_ONESWEEP(kCarryRect);
        else if (mode == kGatherRect) GSR_ONESWEEP(kGatherRect);
        else if (mode == kRanges) GSR_ONESWEEP(kRanges);
        else if (mode == kPackedMid) GSR_ONESWEEP(kPackedMid);
        else if (mode == kPackedLast) GSR_ONESWEEP(kPackedLast);
        else GSR_ONESWEEP(kPlain);
#undef GSR_ONESWEEP
        ksrc = kdst;
        vsrc = vdst;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// pair emission and ranges
// ---------------------------------------------------------------------------
// One block per RECS consecutive records (depth order).  The block's pairs
// form one contiguous span of the output; each thread takes every 256th pair of
// the span, finds its record by binary search over the records' offsets in LDS,
// and writes the pair's global tile id and Gaussian: coalesced stores whatever
// the records' tile counts are.  Per record the staging splits the record index
// into view and Gaussian and keeps the global id of the rectangle's first tile,
// its width and the width's reciprocal, so a pair's row and column in the
// rectangle take a float estimate and an exact integer correction instead of
// two integer divisions.  With PASSES > 0 it also counts the digits of the tile
// ids for the tile sort (LDS histogram, then atomics into the shared rows,
// which k_ranges_init zeroed).  RECS trades the length of each thread's chain of binary searches (a block's
// pairs over 256 threads) against the number of blocks and of their histogram atomics: 128 records per block
// for up to 2M records (measured: the 512x960 compact scene's emission 27 -> 13 us), 256 above (neutral to
// 6 % faster than 512 on 5.9M and 7.3M records).
constexpr int kEmitSmallRecs = 128;
constexpr int kEmitRecs = 256;
constexpr int64_t kEmitSmallMaxRecords = 1 << 21;

template <int PASSES, int RECS>
__global__ __launch_bounds__(256) void k_emit(const uint32_t* __restrict__ rid_sorted,
                                              const uint2* __restrict__ rect_sorted,
                                              const uint32_t* __restrict__ tt_sorted,
                                              const uint32_t* __restrict__ offsets, int64_t VG, uint32_t G, int T,
                                              int TX, uint32_t* __restrict__ pkey, uint32_t* __restrict__ pair_g,
                                              RadixDigits rd, int packed_gbits, uint32_t* __restrict__ part,
                                              uint2* __restrict__ ranges, int64_t n_tiles) {
    // the tile ranges start as {~0u, 0} (a grid-stride share per block): the tile sort's last pass records them
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_tiles; i += (int64_t)gridDim.x * 256)
        ranges[i] = make_uint2(0xffffffffu, 0u);
    __shared__ uint32_t s_off[RECS];
    __shared__ uint32_t s_g[RECS];     // Gaussian index
    __shared__ uint32_t s_key0[RECS];  // global tile id of the rectangle's first tile
    __shared__ uint32_t s_wx[RECS];    // rectangle width in tiles
    __shared__ float s_inv[RECS];      // its reciprocal (an estimate, corrected per pair)
    __shared__ uint32_t h[PASSES > 0 ? PASSES * kMaxBins : 1];
    __shared__ uint32_t s_end;
    const int64_t k0 = (int64_t)blockIdx.x * RECS;
    const int last = (int)((VG - 1 - k0) < RECS - 1 ? (VG - 1 - k0) : RECS - 1);
    for (int i = threadIdx.x; i < RECS; i += 256) {
        const int64_t k = k0 + i;
        if (k < VG) {
            const uint32_t off = offsets[k];
            uint2 r;
            if (rect_sorted) {
                r = rect_sorted[k];
                if (i == last) s_end = off + tt_sorted[k];
            } else {  // packed rectangles in tt_sorted
                const uint32_t q = tt_sorted[k];
                r = unpack_rect(q);
                if (i == last) s_end = off + scan_item(q, true);
            }
            const uint32_t rid = rid_sorted[k];
            const uint32_t v = rid / G;
            const uint32_t x0 = r.x & 0xffffu, y0 = r.x >> 16, wx = (r.y & 0xffffu) - x0;
            s_off[i] = off;
            s_g[i] = rid - v * G;
            s_key0[i] = v * (uint32_t)T + y0 * (uint32_t)TX + x0;
            s_wx[i] = wx;
            s_inv[i] = wx ? __builtin_amdgcn_rcpf((float)wx) : 0.0f;  // a record with pairs has wx >= 1
        }
    }
    if (PASSES > 0)
        for (int i = threadIdx.x; i < PASSES * kMaxBins; i += 256) h[i] = 0u;
    __syncthreads();
    const uint32_t pstart = s_off[0], pend = s_end;
    for (uint32_t p = pstart + threadIdx.x; p < pend; p += 256) {
        int lo = 0, hi = last;
        while (lo < hi) {  // largest t with s_off[t] <= p (it has a non-empty rectangle holding p)
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= p) lo = mid;
            else hi = mid - 1;
        }
        const uint32_t j = p - s_off[lo];  // the pair's index in its rectangle, row-major
        const uint32_t wx = s_wx[lo];
        // row = floor(j / wx) from the float estimate (off by a few at most), made exact by the remainder
        uint32_t row = (uint32_t)((float)j * s_inv[lo]);
        int32_t col = (int32_t)(j - row * wx);
        while (col < 0) {
            --row;
            col += (int32_t)wx;
        }
        while (col >= (int32_t)wx) {
            ++row;
            col -= (int32_t)wx;
        }
        const uint32_t key = s_key0[lo] + row * (uint32_t)TX + (uint32_t)col;
        const uint32_t g = s_g[lo];
        if (packed_gbits > 0) {
            pkey[p] = (key << packed_gbits) | g;
        } else {
            pkey[p] = key;
            pair_g[p] = g;
        }
#pragma unroll
        for (int q = 0; q < PASSES; ++q) {
            const int shift = q * rd.dbits;
            const int pb = shift + rd.dbits <= rd.bits ? rd.dbits : rd.bits - shift;
            atomicAdd(&h[q * kMaxBins + ((key >> shift) & ((1u << pb) - 1u))], 1u);
        }
    }
    if (PASSES > 0) {
        __syncthreads();
        uint32_t* row = part + (int64_t)(blockIdx.x % kHistMaxBlocks) * (kMaxPasses * kMaxBins);
        for (int i = threadIdx.x; i < PASSES * kMaxBins; i += 256)
            if (h[i]) atomicAdd(&row[i], h[i]);
    }
}

hipError_t launch_emit(const Sizes& s, Workspace& ws, const uint32_t* rid_sorted, const RadixDigits* rd,
                       int packed_gbits, bool rects_packed, hipStream_t st) {
    if (s.VG == 0) return hipSuccess;
    const bool small = s.VG <= kEmitSmallMaxRecords;
    const int recs = small ? kEmitSmallRecs : kEmitRecs;
    const dim3 grid((unsigned)((s.VG + recs - 1) / recs)), block(256);
    const RadixDigits d = rd ? *rd : RadixDigits{};
#define GSR_EMIT_R(PP, RR)                                                                                        \
    hipLaunchKernelGGL((k_emit<PP, RR>), grid, block, 0, st, rid_sorted, rects_packed ? nullptr : ws.rect_sorted, \
                       ws.tt_sorted, ws.offsets, s.VG,                                                           \
                       (uint32_t)s.G, s.T, s.TX, ws.pkey_emit, ws.pair_g, d, packed_gbits, ws.sort_part, ws.ranges, \
                       (int64_t)s.V * s.T)
#define GSR_EMIT(PP)                          \
    if (small) GSR_EMIT_R(PP, kEmitSmallRecs); \
    else GSR_EMIT_R(PP, kEmitRecs)
    switch (rd ? rd->passes : 0) {
        case 0: GSR_EMIT(0); break;
        case 1: GSR_EMIT(1); break;
        case 2: GSR_EMIT(2); break;
        case 3: GSR_EMIT(3); break;
        default: GSR_EMIT(4); break;
    }
#undef GSR_EMIT
#undef GSR_EMIT_R
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_ranges_init(uint2* __restrict__ ranges, int64_t n, uint32_t* __restrict__ part,
                                                     int64_t n_part) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        ranges[i] = make_uint2(0xffffffffu, 0u);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_part; i += stride) part[i] = 0u;
}

// a copy of the ranges with the ones no key reached ({~0u, 0}) as {0, 0}
__global__ __launch_bounds__(256) void k_ranges_export(const uint2* __restrict__ ranges, uint2* __restrict__ out,
                                                       int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const uint2 r = ranges[i];
        out[i] = r.x > r.y ? make_uint2(0u, 0u) : r;
    }
}

hipError_t launch_ranges_init(uint2* ranges, int64_t n_tiles, uint32_t* part, hipStream_t st) {
    const int64_t n_part = part ? (int64_t)kHistMaxBlocks * kMaxPasses * kMaxBins : 0;
    const int64_t n = n_tiles > n_part ? n_tiles : n_part;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    if (n > 0)
        hipLaunchKernelGGL(k_ranges_init, dim3((unsigned)blocks), dim3(256), 0, st, ranges, n_tiles, part, n_part);
    return hipGetLastError();
}

// The traversals that follow the render (replay, backward, feature composite, attribution) take the tiles
// in decreasing order of the work the render measured for them, so that the longest do not start last and
// the final wave of blocks is short.  Work is bucketed (2 buckets per octave) and tiles keep their order
// within a bucket, so tiles of similar work stay next to their neighbours.  One block; stable per-wave
// ranking within each 1024-tile chunk.
__device__ __forceinline__ uint32_t work_bucket(uint32_t w) {
    // half octaves of w + 1: twice the position k of its top bit, plus the bit below it (split at 1.5 * 2^k)
    const uint32_t x = w + 1u;
    const uint32_t k = 31u - (uint32_t)__builtin_clz(x);
    const uint32_t b = 2u * k + (k > 0u ? (x >> (k - 1u)) & 1u : 0u);
    return 63u - (b > 63u ? 63u : b);
}

__global__ __launch_bounds__(1024) void k_tile_order(const uint32_t* __restrict__ work, int64_t n,
                                                     uint32_t* __restrict__ order) {
    __shared__ uint32_t base[64];
    __shared__ uint32_t wcnt[16][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    if (threadIdx.x < 64) base[threadIdx.x] = 0u;
    for (int i = threadIdx.x; i < 16 * 64; i += 1024) (&wcnt[0][0])[i] = 0u;
    __syncthreads();
    for (int64_t t = threadIdx.x; t < n; t += 1024) atomicAdd(&base[work_bucket(work[t])], 1u);
    __syncthreads();
    if (wave == 0) {  // bucket starts: one wave's exclusive scan of the 64 counts
        const uint32_t c = base[lane];
        base[lane] = wave_inclusive_scan(c, lane) - c;
    }
    __syncthreads();
    for (int64_t c0 = 0; c0 < n; c0 += 1024) {
        const int64_t t = c0 + threadIdx.x;
        const bool valid = t < n;
        const uint32_t b = valid ? work_bucket(work[t]) : 0u;
        const uint64_t peers = match_peers(b, 6, valid);
        const uint64_t lower = peers & lt_mask;
        if (valid && lower == 0ull) wcnt[wave][b] = (uint32_t)__popcll(peers);
        __syncthreads();
        if (valid) {
            uint32_t pos = base[b] + (uint32_t)__popcll(lower);
            for (int w = 0; w < wave; ++w) pos += wcnt[w][b];
            order[pos] = (uint32_t)t;
        }
        __syncthreads();
        if (threadIdx.x < 64) {
            uint32_t s = 0u;
            for (int w = 0; w < 16; ++w) {
                s += wcnt[w][threadIdx.x];
                wcnt[w][threadIdx.x] = 0u;
            }
            base[threadIdx.x] += s;
        }
        __syncthreads();
    }
}

hipError_t launch_tile_order(const uint32_t* work, int64_t n_tiles, uint32_t* order, hipStream_t st) {
    if (n_tiles > 0) hipLaunchKernelGGL(k_tile_order, dim3(1), dim3(1024), 0, st, work, n_tiles, order);
    return hipGetLastError();
}

hipError_t launch_ranges_export(const uint2* ranges, uint2* out, int64_t n_tiles, hipStream_t st) {
    if (n_tiles > 0)
        hipLaunchKernelGGL(k_ranges_export, dim3((unsigned)((n_tiles + 255) / 256)), dim3(256), 0, st, ranges, out,
                           n_tiles);
    return hipGetLastError();
}

}  // namespace gsr
