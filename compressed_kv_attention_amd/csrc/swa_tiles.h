// swa_tiles.h -- visibility predicate, tile classification and tile
// enumeration shared by every prefill kernel and by the debug-visibility
// kernel, so that the mask the kernels apply is the mask that is checked.
//
// Sources (web pages; cited by title and section):
//   [NW] "How the 256-Token Sliding Window Works with Tools as KV Sinks in
//        Needle", section "KV Sinks for Tools: Pinning Critical Context":
//        packing (same segment, segment > 0) & causal & (recent | sink), the
//        window term applied only when a window is set.
//   [CA] "Compressed attention and the copy probe", section "Two kinds of
//        columns, pooled blocks and exact recent keys": columns are [pooled
//        blocks, exact keys]; block j shows once (j + 1) * b <= t - W + 1.
#pragma once

#include "swa_common.h"

namespace swa {

enum : int { TILE_SKIP = 0, TILE_FULL = 1, TILE_PARTIAL = 2 };
enum : int { COL_EXACT = 0, COL_POOLED = 1 };

// Element predicate of plain mode.
// (Evaluated without short-circuit branches.)
__device__ __forceinline__ bool visible_plain(int seg_q, int seg_k, bool sink_k, int q, int k, int window) {
    const bool keep = (seg_q > 0) & (seg_k == seg_q) & (k <= q);
    const bool in_window = (window == 0) | ((q - k) < window) | sink_k;
    return keep & in_window;
}

// Exact-key predicate of compressed mode: causal window, no segments, no sinks.
__device__ __forceinline__ bool visible_exact_window(int q, int t, int window) {
    return (t <= q) & ((q - t) < window);
}

// Number of pooled blocks visible to row q: blocks j with (j+1)*b <= q-W+1,
// i.e. j < floor((q - W + 1) / b), capped at nblk.
__device__ __forceinline__ int pooled_visible_count(int q, int window, int block, int nblk) {
    const int lim = q - window + 1;
    if (lim < block) return 0;
    const int n = lim / block;
    return n < nblk ? n : nblk;
}

// Summary of a group of query rows r0..r1 (all < T) and of their segment ids.
struct RowSum {
    int r0, r1, smin, smax;
};
// Summary of the valid keys k0..k1 (< nkeys) of one key sub-tile.
struct KeySum {
    int smin, smax, any_sink, all_sink;
};

// Classify a (row group, key sub-tile [k0, k0 + sub)) pair of plain mode, or
// of the exact columns of compressed mode (plain == false: no segments, no
// sinks).  FULL means every (row, key) pair is visible; SKIP means none is.
// A sub-tile that runs past the last key is never FULL.
__device__ __forceinline__ int classify_exact(const RowSum& r, const KeySum& ks, int k0, int sub,
                                              int nkeys, int window, bool plain) {
    if (k0 >= nkeys || r.r1 < r.r0) return TILE_SKIP;
    const int k_last = min(k0 + sub - 1, nkeys - 1);
    const bool complete = (k0 + sub) <= nkeys;
    // causal
    if (k0 > r.r1) return TILE_SKIP;
    const bool causal_full = k_last <= r.r0;
    // window (and sinks in plain mode)
    bool win_full = true;
    if (window != 0) {
        const bool any_sink = plain && ks.any_sink;
        const bool all_sink = plain && ks.all_sink;
        if (r.r0 - k_last >= window && !any_sink) return TILE_SKIP;
        win_full = (r.r1 - k0 < window) || all_sink;
    }
    // packing
    bool seg_full = true;
    if (plain) {
        const int rlo = max(1, r.smin);
        if (r.smax <= 0 || ks.smax < rlo || ks.smin > r.smax) return TILE_SKIP;
        seg_full = (r.smin == r.smax) && (ks.smin == ks.smax) && (ks.smin == r.smin) && (r.smin > 0);
    }
    return (causal_full && win_full && seg_full && complete) ? TILE_FULL : TILE_PARTIAL;
}

// Classify pooled columns [j0, j0 + sub) for rows r0..r1.
__device__ __forceinline__ int classify_pooled(const RowSum& r, int j0, int sub, int window, int block,
                                               int nblk) {
    if (j0 >= nblk || r.r1 < r.r0) return TILE_SKIP;
    const int nv_lo = pooled_visible_count(r.r0, window, block, nblk);
    const int nv_hi = pooled_visible_count(r.r1, window, block, nblk);
    if (j0 >= nv_hi) return TILE_SKIP;
    if (j0 + sub - 1 < nv_lo) return TILE_FULL;  // implies j0 + sub <= nblk
    return TILE_PARTIAL;
}

// Key tiles a workgroup with rows [q0, q1] must visit, in this order:
// pooled tiles (compressed mode), sink tiles lying before the window band
// (plain mode with a window and sink flags), then the band itself.
struct TilePlan {
    int n_pooled;   // pooled tiles 0 .. n_pooled-1
    int band_lo;    // exact tiles band_lo .. band_hi
    int band_hi;
    int sink_keys;  // sink flags are scanned over keys [0, sink_keys)
};

__device__ __forceinline__ TilePlan plan_tiles(int q0, int q1, int window, int block, int nblk,
                                               bool has_prefix, int BN) {
    TilePlan p;
    p.n_pooled = 0;
    if (block > 0) {
        const int nv = pooled_visible_count(q1, window, block, nblk);
        p.n_pooled = (nv + BN - 1) / BN;
    }
    const int lo_key = (window > 0) ? max(0, q0 - window + 1) : 0;
    p.band_lo = lo_key / BN;
    p.band_hi = q1 / BN;
    p.sink_keys = (block == 0 && window > 0 && has_prefix) ? p.band_lo * BN : 0;
    return p;
}

// Block-wide scan of the sink flags over keys [0, n_keys): bit t of `bits`
// is set when key tile t (of BN keys) holds at least one sink.  `bits` is in
// LDS with ceil(n_keys / BN / 32) words.  Ends with a barrier.
__device__ __forceinline__ void scan_sink_tiles(const uint8_t* prefix_row, int n_keys, int BN,
                                                uint32_t* bits, int tid, int nthreads) {
    const int ntiles = (n_keys + BN - 1) / BN;
    const int nwords = (ntiles + 31) / 32;
    for (int w = tid; w < nwords; w += nthreads) bits[w] = 0u;
    __syncthreads();
    for (int i = tid; i < n_keys; i += nthreads) {
        if (prefix_row[i]) {
            const int t = i / BN;
            atomicOr(&bits[t >> 5], 1u << (t & 31));
        }
    }
    __syncthreads();
}

// Walks a TilePlan.  Every thread of a workgroup walks the same sequence.
struct TileIter {
    int phase;  // 0 pooled, 1 sinks, 2 band, 3 done
    int idx;
    int word;
    uint32_t bits;
    int sink_words;
    TilePlan plan;
    const uint32_t* sink_bits;

    __device__ __forceinline__ void init(const TilePlan& p, const uint32_t* sb, int BN) {
        plan = p;
        sink_bits = sb;
        const int ntiles = (p.sink_keys + BN - 1) / BN;
        sink_words = (ntiles + 31) / 32;
        phase = 0;
        idx = 0;
        word = -1;
        bits = 0u;
    }

    __device__ __forceinline__ bool next(int& kind, int& tile) {
        if (phase == 0) {
            if (idx < plan.n_pooled) {
                kind = COL_POOLED;
                tile = idx++;
                return true;
            }
            phase = 1;
        }
        if (phase == 1) {
            while (bits == 0u) {
                if (++word >= sink_words) break;
                bits = sink_bits[word];
            }
            if (bits != 0u) {
                const int b = __builtin_ctz(bits);
                bits &= bits - 1u;
                kind = COL_EXACT;
                tile = word * 32 + b;
                return true;
            }
            phase = 2;
            idx = plan.band_lo;
        }
        if (phase == 2) {
            if (idx <= plan.band_hi) {
                kind = COL_EXACT;
                tile = idx++;
                return true;
            }
            phase = 3;
        }
        return false;
    }
};

}  // namespace swa
