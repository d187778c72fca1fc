// gsr_internal.hpp -- host-side context and kernel launchers (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gsr.h"
#include "gsr_device.hpp"

namespace gsr {

// Workspace carve-up.  Every array lives in caller-owned device memory.
struct Workspace {
    // per (view, Gaussian) record, rid = v * G + g
    float4* rec0;          // {mx, my, s1, s2}: centre (float32 part) and exponent factors
    float4* rec1;          // {s3, opacity, colour r, colour g} (colour before clamping)
    float4* rec2;          // {colour b, entry box: two binary16 half-widths, mx_lo, my_lo}
    uint2* rect;           // tile rectangle: {x0 | y0 << 16, x1 | y1 << 16}, zero when culled
    uint32_t* depth_key;   // depth bits, 0xffffffff when culled
    uint32_t* tiles_touched;
    uint32_t* slot_base;   // exclusive scan of tiles_touched in record order: the record's first partial slot
    // depth sort (ping-pong) and the pair offsets in depth order
    uint32_t* dkey_b;
    uint32_t* drid_a;
    uint32_t* drid_b;
    uint2* rect_sorted;    // tile rectangles in depth order
    uint32_t* tt_sorted;   // tile counts in depth order
    uint32_t* offsets;     // exclusive scan of tt_sorted (also the depth sort's key scratch)
    uint32_t* pay_a;       // packed rectangles carried through the depth sort (ping-pong)
    uint32_t* pay_b;
    // scan / histogram scratch
    uint64_t* scan_blocks; // single-pass scan: one tagged word per 4096-item tile
    uint64_t* scan_total;  // [0] pair count, [1] slot total, [3] the scans' ticket counter (low word)
    uint64_t* lookback;    // radix look-back words, [radix tile][256 digits]
    uint32_t* sort_ctl;    // radix control: per-pass tile tickets, then per-pass digit offsets
    uint32_t* sort_part;   // per-block digit histograms of the radix sorts
    // (tile, Gaussian) pairs
    uint32_t* pkey_emit;   // global tile id of each pair, depth order
    uint32_t* pkey_b;
    uint32_t* pkey_c;
    uint32_t* pval_a;
    uint32_t* pval_b;
    uint32_t* pair_g;      // Gaussian of each emitted pair, depth order
    uint2* ranges;         // per tile [start, end)
    uint32_t* tile_work;   // per tile: list entries the render processed before its pixels were done
    uint32_t* tile_order;  // tiles by decreasing tile_work: the order the traversals after the render take them
    float4* partials;      // per slot, score replay (2 float4): {W, U_a, conic * U_mu (2)}, {masked U_rgb (3), 0};
                           // backward (3 float4): {U, U_x, U_y, U_xx}, {U_xy, U_yy, masked V_rg}, {masked V_b, 0, 0, 0}
    float4* gv_sums;       // per reached record: the sums of the same layout (2 or 3 float4)
    uint64_t* rec_masks;   // per 64 records: {live mask, reached mask}
    float4* pixel;         // per pixel: rendered colour (rgb), final transmittance
    uint2* pixel_stats;    // per pixel: entries evaluated, entries past the distance cut
    uint8_t* events;       // per sorted pair the render processed: bit w set when some pixel of wave w
                           // contributed or saturated at that entry
    uint32_t* slot_bits;   // per slot: set when the replay wrote the slot's partial (cleared by the render)
};

struct Sizes {
    int64_t G;
    int32_t d;
    int32_t V;
    int32_t W, H, TX, TY, T;
    int64_t VG;
    uint64_t max_pairs;
    int64_t scan_blocks_cap;
    int64_t sort_tiles_cap;   // radix tiles of the larger of the two sorts
};

// Radix sort layout shared by the launcher and the workspace carve-up.
constexpr int kSortTile = 8192;       // keys per radix tile (512 threads x 16)
constexpr int kSmallSortTile = 4096;  // keys per radix tile of a sort of at most kSmallSortKeys keys
constexpr int64_t kSmallSortKeys = 1 << 21;
constexpr int kTinySortTile = 2048;   // keys per radix tile of a sort of at most kTinySortKeys keys
constexpr int64_t kTinySortKeys = 1 << 19;
constexpr int kSortMaxPasses = 4;     // 8-bit digits of 32-bit keys
constexpr int kSortCtlTotals = 8;     // sort_ctl: [0, 8) tickets, then kSortMaxPasses x 256 digit totals
constexpr int kSortCtlWords = kSortCtlTotals + kSortMaxPasses * 256;
constexpr int kSortPartBlocks = 256;  // blocks of the digit histogram
struct SortScratch {
    uint64_t* lookback;
    uint32_t* ctl;
    uint32_t* part;
};
// Look-back words are tagged with a per-pass epoch (31 bits, never 0), so they
// need no clearing between passes; the owner clears them once before the
// first pass and again before the epoch would wrap.
inline uint32_t next_epoch(uint32_t* e) { return ++*e; }
constexpr uint32_t kEpochLimit = 0x7fff0000u;

size_t carve_workspace(const Sizes& s, char* base, Workspace* ws);  // base == nullptr: size only
Sizes make_sizes(const gs_dims& d);

// ---- launchers (return hipGetLastError of the launch) ----------------------
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t st);
// pay_init (optional): also the packed rectangles (pack_rect) per record, for the depth sort's first pass
hipError_t launch_project(const gs_gaussians& sc, const CamPack& cams, const Sizes& s, float near_plane,
                          float far_plane, int antialiased, uint32_t* pay_init, Workspace& ws, hipStream_t st);
// State of the single-pass scans of a context: one tagged word per 4096-item tile (flags_cap words), a ticket
// counter that only grows, the last tag and the tickets handed out since the last clear (host side).
struct ScanState {
    uint64_t* flags;
    int64_t flags_cap;
    uint32_t* ticket;
    uint32_t* epoch;
    uint32_t* ticket_base;
};
constexpr uint32_t kScanEpochLimit = 0x7ff0u;  // tags fit 15 bits
// exclusive scan of in (u32) into out (may alias); total -> *total (device u64).  With packed_rect_in the
// items are packed rectangles (pack_rect) and their tile counts are scanned.
// host_total (optional): a device address of pinned host memory that receives the total as well.
hipError_t launch_scan_u32(const uint32_t* in, int64_t n, uint32_t* out, ScanState& ss, uint64_t* total,
                           hipStream_t st, bool packed_rect_in = false, uint64_t* host_total = nullptr);
// Tile rectangles that a record sort moves into sorted order with the values:
// rect[val] becomes rect_out[pos] with its tile count tt_out[pos].  With
// pay_a/pay_b (u32, n each) the rectangles are carried through the passes
// packed to 32 bits (tile grids of at most 256 x 256 only); without, the last
// pass gathers rect[val].
struct RectSort {
    const uint2* rect;
    uint2* rect_out;
    uint32_t* tt_out;
    uint32_t* pay_a;
    uint32_t* pay_b;
    const uint32_t* pay_init;  // optional: the rectangles already packed, in input order (read by pass 0)
    bool out_packed;           // with pay_a/pay_b: the last pass writes the packed words into tt_out instead of
                               // the rectangles and tile counts (rect_out unused)
};
// Per-launch form of the same (device side).
struct RectCarry {
    const uint2* pack_src;   // pass 0: rectangles in input order, packed on load
    const uint32_t* pay_in;  // later passes: packed rectangles in input order
    uint32_t* pay_out;       // packed rectangles in output order (all but the last pass)
    const uint2* gather_src; // last pass without carrying: gather rect[val]
    uint2* rect_out;         // last pass: unpacked rectangles
    uint32_t* tt_out;        // last pass: tile counts
    uint2* ranges;           // last pass of a key sort: per-key [start, end) (atomic min / max)
    int key_shift;           // packed words: the key's lowest bit (the value lies below it)
    uint32_t low_mask;       // packed words: (1 << key_shift) - 1
};
// Digit layout of the LSD radix sorts: `passes` passes of at most 8 bits, all `dbits` wide but the last.
struct RadixDigits {
    int bits, passes, dbits;
};
RadixDigits radix_digits(int bits);
// Stable LSD radix sort of (keys, vals) on bits [0, bits), digits of up to 8
// bits; vals_in == null means identity values (the input index).  Pass p writes
// kbuf[p & 1] / vbuf[p & 1], so these must differ from each other and from
// keys_in/vals_in except that kbuf1/vbuf1 may alias keys_in/vals_in (consumed
// by pass 0).  rs (optional) moves tile rectangles along.  *keys_out /
// *vals_out receive the arrays holding the result; with keys_out == null the
// final pass does not write keys.  Each pass takes a new epoch from *epoch.
// With ranges (and no rs), the last pass also records every key's output range
// [start, end) in ranges[key], which the caller initialises to {~0u, 0}.
// With hist_ready, the keys' digit counts (layout radix_digits(bits)) are
// already summed in the kSortPartBlocks rows of sc.part and are not recounted.
// With key_shift > 0 the keys are packed words, key in bits [key_shift,
// key_shift + bits) and a value below: no vals_in, no rs, hist_ready and ranges
// required; the final pass writes each word's value bits to *vals_out (and no
// keys) and records the ranges of the keys.
hipError_t launch_radix_sort(const uint32_t* keys_in, const uint32_t* vals_in, int64_t n, int bits,
                             uint32_t* kbuf0, uint32_t* kbuf1, uint32_t* vbuf0, uint32_t* vbuf1,
                             const RectSort* rs, uint2* ranges, bool hist_ready, int key_shift,
                             const SortScratch& sc, uint32_t* epoch, hipStream_t st, uint32_t** keys_out,
                             uint32_t** vals_out);
// The depth-ordered rectangles are rect_sorted with their tile counts tt_sorted, or, with rects_packed, the
// packed words in tt_sorted.
// (tile, Gaussian) pairs of the depth-ordered records into pkey_emit / pair_g, or, with packed_gbits > 0,
// into pkey_emit alone as (tile << packed_gbits) | Gaussian; with rd, their tile ids' digit counts
// (layout *rd) are added into the rows of sort_part, which must be zero beforehand.
hipError_t launch_emit(const Sizes& s, Workspace& ws, const uint32_t* rid_sorted, const RadixDigits* rd,
                       int packed_gbits, bool rects_packed, hipStream_t st);
// ranges before a sort that records them: {~0u, 0} everywhere (those no key reaches stay so: start > end is
// an empty range); the init also zeroes the kSortPartBlocks histogram rows of part when given
hipError_t launch_ranges_init(uint2* ranges, int64_t n_tiles, uint32_t* part, hipStream_t st);
// a copy of the ranges with the empty ones as {0, 0}
hipError_t launch_ranges_export(const uint2* ranges, uint2* out, int64_t n_tiles, hipStream_t st);
// tiles bucketed by work (2 buckets per octave), largest first, in tile order within a bucket
hipError_t launch_tile_order(const uint32_t* work, int64_t n_tiles, uint32_t* order, hipStream_t st);
hipError_t launch_render(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, uint64_t n_pairs,
                         const float bg[3], float* color, float* T_final, int32_t* n_contrib, hipStream_t st,
                         bool prev_order_valid);  // tile_order holds an order a previous render measured
// per-pixel work counts of the render's traversal (same decisions) into ws.pixel_stats
hipError_t launch_render_stats(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, hipStream_t st);
hipError_t launch_replay(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, const float* observed,
                         float eps, float den_min, hipStream_t st);
// per record, the sums of the NQ-float4 partials of the slots flagged in slot_bits, plus the
// live / reached masks (nq = 2: score replay, 3: backward)
hipError_t launch_gather_slots(const Sizes& s, const Workspace& ws, int nq, hipStream_t st);
hipError_t launch_backward(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, const float* grad_color,
                           hipStream_t st);
// per (Gaussian, view): the record's backward sums and the chain rule to the parameters, summed over views
hipError_t launch_backward_finalize(const gs_gaussians& sc, const CamPack& cams, const Sizes& s,
                                    const Workspace& ws, int antialiased, const gs_gaussian_grads& out,
                                    hipStream_t st);
// Tokens from the per-record sums of k_gather_slots, or, where tokens_gather(s) holds (one view, up to 2M
// Gaussians), from the slots directly (the gather kernel is then not needed).
bool tokens_gather(const Sizes& s);
hipError_t launch_tokens(const gs_gaussians& sc, const CamPack& cams, const Sizes& s, const Workspace& ws,
                         float eps, float lambda, float* tokens, hipStream_t st);
hipError_t launch_exp2(const float* in, float* out, int64_t n, hipStream_t st);
// per-channel background of one feature-composite launch (at most 16 channels)
struct FeatBg {
    float v[16];
};
hipError_t launch_render_features(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, const float* feat,
                                  int C, const float* bg_host, float* out, hipStream_t st);
hipError_t launch_attribute(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, const float* map, int C,
                            float* out, hipStream_t st);
hipError_t launch_topk(const Sizes& s, const Workspace& ws, const uint32_t* sorted_g, int k, int32_t* ids, float* w,
                       hipStream_t st);

}  // namespace gsr
