// binning.hip -- tile binning and contributor sorting on gfx950.
//
// Order of work (Stage 1, step "tile binning and contributor sorting" of the
// Renderer Score Tokens proposal; the order within a tile is front to back):
//   1. stable LSD radix sort of the (view, Gaussian) records by float32 depth
//      bits (culled records carry 0xffffffff and sink to the end);
//   2. exclusive scan of the per-record tile counts in that depth order;
//   3. emission of one (tile, Gaussian) pair per covered tile, in depth order,
//      row-major over each record's tile rectangle;
//   4. stable LSD radix sort of the pairs by global tile id (view * tiles +
//      tile): because emission was in (depth bits, Gaussian) order and the
//      sort is stable, each tile's list ends up ordered by (depth bits,
//      Gaussian index) -- a total order, so the lists are unique;
//   5. per-tile [start, end) ranges.
// Only the pairs (2 x 4 bytes per pass) go through the tile sort; the depth
// sort runs once over the records instead of over every pair.
//
// Radix passes: per 4096-key block a digit histogram (per-wave LDS counters),
// one device-wide exclusive scan of the digit-major histogram table, then a
// scatter that ranks keys stably inside the block: each wave takes 64 keys at a
// time in index order, finds the lanes holding the same digit with one ballot
// per digit bit, and counts in per-wave LDS counters; waves own consecutive
// 1024-key slices so wave order is index order.
#include "gsr_internal.hpp"

namespace gsr {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int kScanTile = kScanThreads * kScanItems;  // 4096
constexpr int kRadixThreads = 256;
constexpr int kRadixItems = 16;
constexpr int kRadixTile = kRadixThreads * kRadixItems;  // 4096

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

// exclusive scan across the block (blockDim.x = 256 or 1024), returns the block total via *total
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

__device__ __forceinline__ uint32_t scan_load(const uint32_t* __restrict__ in, const uint32_t* __restrict__ idx,
                                              int64_t k) {
    return idx ? in[idx[k]] : in[k];
}

__global__ __launch_bounds__(kScanThreads) void k_scan_reduce(const uint32_t* __restrict__ in,
                                                              const uint32_t* __restrict__ idx, int64_t n,
                                                              uint64_t* __restrict__ bsum) {
    __shared__ uint64_t lds[kScanThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    uint64_t s = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int64_t k = base + i * kScanThreads + threadIdx.x;
        if (k < n) s += scan_load(in, idx, k);
    }
    uint64_t tot;
    block_exclusive_scan<uint64_t, kScanThreads>(s, &tot, lds);
    if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

__global__ __launch_bounds__(1024) void k_scan_top(uint64_t* __restrict__ bsum, int64_t nb,
                                                   uint64_t* __restrict__ total) {
    __shared__ uint64_t lds[16];
    uint64_t carry = 0;
    for (int64_t c = 0; c < nb; c += 1024) {
        const int64_t k = c + threadIdx.x;
        const uint64_t x = k < nb ? bsum[k] : 0;
        uint64_t tot;
        const uint64_t ex = block_exclusive_scan<uint64_t, 1024>(x, &tot, lds);
        if (k < nb) bsum[k] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) *total = carry;
}

// `in` and `out` may alias (each block reads its whole slice before writing it)
__global__ __launch_bounds__(kScanThreads) void k_scan_down(const uint32_t* in, const uint32_t* __restrict__ idx,
                                                            int64_t n, const uint64_t* __restrict__ boff,
                                                            uint32_t* out) {
    // padded so that thread t's 16 consecutive items (t*17 + i) are bank-conflict free
    __shared__ uint32_t s[kScanTile + kScanTile / 16];
    __shared__ uint32_t lds[kScanThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int e = i * kScanThreads + threadIdx.x;
        const int64_t k = base + e;
        s[e + e / 16] = k < n ? scan_load(in, idx, k) : 0u;
    }
    __syncthreads();
    const int t = threadIdx.x;
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) local += s[t * 17 + i];
    uint32_t tot;
    uint32_t run = (uint32_t)boff[blockIdx.x] + block_exclusive_scan<uint32_t, kScanThreads>(local, &tot, lds);
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

hipError_t launch_scan_u32(const uint32_t* in, const uint32_t* idx, int64_t n, uint32_t* out,
                           uint64_t* block_scratch, uint64_t* total, hipStream_t st) {
    const int64_t nb = (n + kScanTile - 1) / kScanTile;
    if (nb > 0) hipLaunchKernelGGL(k_scan_reduce, dim3((unsigned)nb), dim3(kScanThreads), 0, st, in, idx, n, block_scratch);
    hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(1024), 0, st, block_scratch, nb, total);
    if (nb > 0) hipLaunchKernelGGL(k_scan_down, dim3((unsigned)nb), dim3(kScanThreads), 0, st, in, idx, n, block_scratch, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// radix sort
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRadixThreads) void k_radix_hist(const uint32_t* __restrict__ keys, int64_t n, int shift,
                                                              int bits, uint32_t* __restrict__ hist, int64_t nb) {
    __shared__ uint32_t h[4][256];
    const int nbins = 1 << bits;
    const uint32_t mask = (uint32_t)nbins - 1u;
    const int wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 4 * 256; i += kRadixThreads) (&h[0][0])[i] = 0u;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kRadixTile;
#pragma unroll 4
    for (int i = 0; i < kRadixItems; ++i) {
        const int64_t k = base + i * kRadixThreads + threadIdx.x;
        if (k < n) atomicAdd(&h[wave][(keys[k] >> shift) & mask], 1u);
    }
    __syncthreads();
    for (int dgt = threadIdx.x; dgt < nbins; dgt += kRadixThreads)
        hist[(int64_t)dgt * nb + blockIdx.x] = h[0][dgt] + h[1][dgt] + h[2][dgt] + h[3][dgt];
}

__global__ __launch_bounds__(kRadixThreads) void k_radix_scatter(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in, int64_t n, int shift, int bits,
    const uint32_t* __restrict__ hist_scan, int64_t nb, uint32_t* __restrict__ keys_out,
    uint32_t* __restrict__ vals_out, const uint32_t* __restrict__ gather, uint32_t* __restrict__ inv) {
    __shared__ uint32_t cnt[4][256];
    __shared__ uint32_t gbase[4][256];
    const int nbins = 1 << bits;
    const uint32_t mask = (uint32_t)nbins - 1u;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 4 * 256; i += kRadixThreads) (&cnt[0][0])[i] = 0u;
    __syncthreads();

    const int64_t base = (int64_t)blockIdx.x * kRadixTile + (int64_t)wave * (kRadixTile / 4);
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t key[kRadixItems], val[kRadixItems], rank[kRadixItems];
#pragma unroll
    for (int i = 0; i < kRadixItems; ++i) {
        const int64_t k = base + i * 64 + lane;
        const bool valid = k < n;
        key[i] = valid ? keys_in[k] : 0u;
        val[i] = valid ? (vals_in ? vals_in[k] : (uint32_t)k) : 0u;
        const uint32_t dgt = (key[i] >> shift) & mask;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < bits; ++b) {
            const bool bit = (dgt >> b) & 1u;
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const uint64_t lower = peers & lt_mask;
        const uint32_t c = valid ? cnt[wave][dgt] : 0u;
        rank[i] = c + (uint32_t)__popcll(lower);
        if (valid && lower == 0ull) cnt[wave][dgt] = c + (uint32_t)__popcll(peers);
    }
    __syncthreads();
    for (int dgt = threadIdx.x; dgt < nbins; dgt += kRadixThreads) {
        uint32_t s = hist_scan[(int64_t)dgt * nb + blockIdx.x];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            gbase[w][dgt] = s;
            s += cnt[w][dgt];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRadixItems; ++i) {
        const int64_t k = base + i * 64 + lane;
        if (k >= n) continue;
        const uint32_t dgt = (key[i] >> shift) & mask;
        const uint32_t pos = gbase[wave][dgt] + rank[i];
        keys_out[pos] = key[i];
        if (gather) {
            vals_out[pos] = gather[val[i]];
            inv[val[i]] = pos;
        } else {
            vals_out[pos] = val[i];
        }
    }
}

hipError_t launch_radix_sort(const uint32_t* keys_in, const uint32_t* vals_in, int64_t n, int bits,
                             uint32_t* kbuf0, uint32_t* kbuf1, uint32_t* vbuf0, uint32_t* vbuf1,
                             const uint32_t* gather, uint32_t* gather_out, uint32_t* inv, uint32_t* hist,
                             uint64_t* block_scratch, uint64_t* total, hipStream_t st, uint32_t** keys_out,
                             uint32_t** vals_out) {
    if (bits < 1) bits = 1;
    const int passes = (bits + 7) / 8;
    const int dbits = (bits + passes - 1) / passes;
    const int64_t nb = (n + kRadixTile - 1) / kRadixTile;
    uint32_t* kb[2] = {kbuf0, kbuf1};
    uint32_t* vb[2] = {vbuf0, vbuf1};
    if (keys_out) *keys_out = kb[(passes - 1) & 1];
    if (vals_out) *vals_out = gather ? gather_out : vb[(passes - 1) & 1];
    if (n <= 0) return hipSuccess;
    const uint32_t* ksrc = keys_in;
    const uint32_t* vsrc = vals_in;
    for (int p = 0; p < passes; ++p) {
        const int shift = p * dbits;
        const int pb = (shift + dbits <= bits) ? dbits : bits - shift;
        const bool last = p == passes - 1;
        uint32_t* kdst = kb[p & 1];
        uint32_t* vdst = (last && gather) ? gather_out : vb[p & 1];
        hipLaunchKernelGGL(k_radix_hist, dim3((unsigned)nb), dim3(kRadixThreads), 0, st, ksrc, n, shift, pb, hist, nb);
        hipError_t e = launch_scan_u32(hist, nullptr, (int64_t)(1 << pb) * nb, hist, block_scratch, total, st);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_radix_scatter, dim3((unsigned)nb), dim3(kRadixThreads), 0, st, ksrc, vsrc, n, shift, pb,
                           hist, nb, kdst, vdst, last ? gather : nullptr, last ? inv : nullptr);
        ksrc = kdst;
        vsrc = vdst;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// pair emission and ranges
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_emit(const uint32_t* __restrict__ rid_sorted, const uint32_t* __restrict__ offsets,
                                              const uint32_t* __restrict__ tiles_touched, float4* __restrict__ rec2,
                                              int64_t VG, int64_t G, int T, int TX, uint32_t* __restrict__ pkey,
                                              uint32_t* __restrict__ pair_g) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= VG) return;
    const uint32_t rid = rid_sorted[k];
    const uint32_t cnt = tiles_touched[rid];
    if (cnt == 0) return;
    const uint32_t off = offsets[k];
    const float4 r2 = rec2[rid];
    const uint32_t lo = __float_as_uint(r2.z), hi = __float_as_uint(r2.w);
    const int x0 = (int)(lo & 0xffffu), y0 = (int)(lo >> 16), x1 = (int)(hi & 0xffffu);
    const uint32_t v = (uint32_t)(rid / G);
    const uint32_t g = (uint32_t)(rid - (int64_t)v * G);
    reinterpret_cast<float*>(rec2 + rid)[1] = __uint_as_float(off);
    const int wx = x1 - x0;
    const uint32_t vbase = v * (uint32_t)T;
    for (uint32_t j = 0; j < cnt; ++j) {
        const int ty = y0 + (int)(j / (uint32_t)wx), tx = x0 + (int)(j % (uint32_t)wx);
        pkey[off + j] = vbase + (uint32_t)(ty * TX + tx);
        pair_g[off + j] = g;
    }
}

hipError_t launch_emit(const Sizes& s, Workspace& ws, const uint32_t* rid_sorted, hipStream_t st) {
    if (s.VG == 0) return hipSuccess;
    hipLaunchKernelGGL(k_emit, dim3((unsigned)((s.VG + 255) / 256)), dim3(256), 0, st, rid_sorted, ws.offsets,
                       ws.tiles_touched, ws.rec2, s.VG, s.G, s.T, s.TX, ws.pkey_a, ws.pair_g);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_ranges(const uint32_t* __restrict__ keys, int64_t n, uint2* __restrict__ ranges) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t k = keys[i];
    if (i == 0 || keys[i - 1] != k) ranges[k].x = (uint32_t)i;
    if (i == n - 1 || keys[i + 1] != k) ranges[k].y = (uint32_t)(i + 1);
}

hipError_t launch_ranges(const uint32_t* sorted_keys, int64_t n, uint2* ranges, int64_t n_tiles, hipStream_t st) {
    hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(ranges), 2 * n_tiles, 0u, st);
    if (e != hipSuccess) return e;
    if (n > 0) hipLaunchKernelGGL(k_ranges, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, sorted_keys, n, ranges);
    return hipGetLastError();
}

}  // namespace gsr
