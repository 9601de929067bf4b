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

// Sub-tile classes.  In FULL and PARTIAL_POS sub-tiles of plain mode every
// valid key lies in one segment (KeySum::smin); a row sees keys of the
// sub-tile only if it belongs to that segment, which the kernels test once
// per row ("lane gate") instead of once per element.  FULL: a row that passes
// the gate sees every key.  PARTIAL_POS: it sees key k iff the positional test
// (unsigned)(q - k) < wlim holds, with the bound classify_exact returns.
// PARTIAL: the full packing & causal & (recent | sink) predicate per element.
enum : int { TILE_SKIP = 0, TILE_FULL = 1, TILE_PARTIAL_POS = 2, TILE_PARTIAL = 3 };
enum : int { COL_EXACT = 0, COL_POOLED = 1 };

// Window limit as an unsigned bound on d = q - k: visible positions are
// 0 <= d < window, or 0 <= d when no window is set.
__device__ __forceinline__ unsigned window_limit(int window) { return window != 0 ? (unsigned)window : 0x7fffffffu; }

// Packed key info: segment id (negative ids count as padding, 0) | sink << 31.
__device__ __forceinline__ int pack_key_info(int seg, bool sink) { return (seg < 0 ? 0 : seg) | ((int)sink << 31); }

// Positional predicate: causal and inside the window.
__device__ __forceinline__ bool visible_pos(int d, unsigned wlim) { return (unsigned)d < wlim; }

// Full plain-mode predicate for a row of segment seg_q > 0 (rows of segment
// <= 0 see nothing and are excluded by the caller): same segment, and
// (causal and recent) or (causal and sink).  [NW §"KV Sinks for Tools"]
__device__ __forceinline__ bool visible_full(int d, unsigned wlim, int info, int seg_q) {
    const bool same_seg = ((info ^ seg_q) & 0x7fffffff) == 0;
    return same_seg & (((unsigned)d < wlim) | ((info < 0) & (d >= 0)));
}

// Element predicate of plain mode in terms of ids (used by the debug path):
// packing & causal & (recent | sink).
__device__ __forceinline__ bool visible_plain(int seg_q, int seg_k, bool sink_k, int q, int k, int window) {
    if (seg_q <= 0) return false;
    return visible_full(q - k, window_limit(window), pack_key_info(seg_k, sink_k), seg_q);
}

// Exact-key predicate of compressed mode: causal window, no segments, no sinks.
__device__ __forceinline__ bool visible_exact_window(int q, int t, int window) {
    return visible_pos(q - t, window_limit(window));
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
// Summary of the valid keys of one key sub-tile.  When the valid keys do not
// all share one segment the range is widened to [0, INT_MAX] (never SKIP or
// FULL by segment; the element predicate decides).
struct KeySum {
    int smin, smax, any_sink, all_sink;
};
__device__ __forceinline__ KeySum make_key_sum(bool uniform, int seg, bool any_sink, bool all_sink) {
    KeySum k;
    k.smin = uniform ? seg : 0;
    k.smax = uniform ? seg : 0x7fffffff;
    k.any_sink = any_sink;
    k.all_sink = all_sink;
    return k;
}

// The key metadata of one 64-key tile j of batch row b, written by one wave
// (lane l: key 64 j + l, valid below T, with segment sg and sink flag sk):
//   info[b][t]     packed segment | sink << 31 of every valid key
//   ksub[b][2j+h]  KeySum of keys [64j + 32h, 64j + 32h + 32) ∩ [0, T)
//   tsink[b][j]    (min, max) segment of the tile's sink keys,
//                  (INT_MAX, INT_MIN) when it holds none
__device__ __forceinline__ void write_key_tile_meta(int b, int j, int lane, int T, int ntile, bool valid, int sg,
                                                    bool sk, int32_t* info, int32_t* ksub, int32_t* tsink) {
    const int inf = valid ? pack_key_info(sg, sk) : 0;
    if (valid) info[(size_t)b * T + 64 * j + lane] = inf;
    const int seg = inf & 0x7fffffff;
    const bool sink = inf < 0;
    const int half = lane >> 5;
    const int s_first = half ? __builtin_amdgcn_readlane(seg, 32) : __builtin_amdgcn_readlane(seg, 0);
    const uint64_t eq_b = __ballot(!valid || seg == s_first);
    const uint64_t any_b = __ballot(valid && sink);
    const uint64_t all_b = __ballot(!valid || sink);
    const int smn = wave_min_i32(valid && sink ? seg : 0x7fffffff);
    const int smx = wave_max_i32(valid && sink ? seg : (int)0x80000000);
    if ((lane & 31) == 0) {
        const uint32_t eq_h = (uint32_t)(eq_b >> (32 * half));
        const uint32_t any_h = (uint32_t)(any_b >> (32 * half));
        const uint32_t all_h = (uint32_t)(all_b >> (32 * half));
        const KeySum ks = make_key_sum(eq_h == 0xffffffffu, s_first, any_h != 0u, all_h == 0xffffffffu);
        *(int4*)(ksub + ((size_t)b * 2 * ntile + 2 * j + half) * 4) = make_int4(ks.smin, ks.smax, ks.any_sink,
                                                                              ks.all_sink);
    }
    if (lane == 0) *(int2*)(tsink + ((size_t)b * ntile + j) * 2) = make_int2(smn, smx);
}

// Classify a (row group, key sub-tile [k0, k0 + sub)) pair of plain mode, or
// of the exact columns of compressed mode (plain == false: no segments, no
// sinks).  SKIP: no pair is visible.  For FULL and PARTIAL_POS, wlim_eff is
// the bound of the positional test: the window limit, or no window when every
// key of the sub-tile is a sink (a sink stays visible to its segment however
// far back it lies) or when the window cannot cut any causal pair.  A sub-tile
// that runs past the last key is never FULL.
__device__ __forceinline__ int classify_exact(const RowSum& r, const KeySum& ks, int k0, int sub, int nkeys,
                                              int window, bool plain, unsigned& wlim_eff) {
    wlim_eff = window_limit(window);
    if (k0 >= nkeys || r.r1 < r.r0) return TILE_SKIP;
    if (k0 > r.r1) return TILE_SKIP;  // every key lies after every row
    const int k_last = min(k0 + sub - 1, nkeys - 1);
    const bool complete = (k0 + sub) <= nkeys;
    const bool causal_full = k_last <= r.r0;
    const bool sinks = plain && ks.any_sink;
    // every pair lies at distance >= window and no key is a sink
    if (window != 0 && r.r0 - k_last >= window && !sinks) return TILE_SKIP;
    if (plain) {
        const int rlo = max(1, r.smin);
        if (r.smax <= 0 || ks.smax < rlo || ks.smin > r.smax) return TILE_SKIP;
        if (ks.smin != ks.smax) return TILE_PARTIAL;  // keys of several segments
    }
    // every causal pair lies inside the window
    const bool in_window = window == 0 || r.r1 - k0 < window;
    if (!in_window && sinks) {
        if (!ks.all_sink) return TILE_PARTIAL;  // sinks and non-sinks at the window edge
        wlim_eff = 0x7fffffffu;                 // all sinks: the causal test alone
    }
    const bool pos_full = causal_full && complete && (in_window || wlim_eff == 0x7fffffffu);
    return pos_full ? TILE_FULL : TILE_PARTIAL_POS;
}

// Lane gate of FULL and PARTIAL_POS sub-tiles for a row of segment seg_q that
// is visible at all (row_vis): plain mode needs the keys' segment.
__device__ __forceinline__ bool lane_gate(bool row_vis, bool plain, int seg_q, const KeySum& ks) {
    return row_vis && (!plain || seg_q == ks.smin);
}

// Classify pooled columns [j0, j0 + sub) for rows r0..r1.  Partial pooled
// sub-tiles use the per-row count of visible blocks.
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

// Block-wide segment range [lo, hi] of rows q0..q1 (lo >= 1; hi < lo when
// every row is padding).  red is 2 ints of LDS scratch.  Ends with a barrier.
__device__ __forceinline__ void row_segment_range(const int32_t* seg_row, int q0, int q1, int* red, int tid,
                                                  int nthreads, int& lo, int& hi) {
    if (!seg_row) {
        lo = hi = 1;
        return;
    }
    int smn = 0x7fffffff, smx = 0;
    for (int r = q0 + tid; r <= q1; r += nthreads) {
        const int s = seg_row[r];
        smn = min(smn, s);
        smx = max(smx, s);
    }
    for (int o = 1; o < 64; o <<= 1) {
        smn = min(smn, __shfl_xor(smn, o, 64));
        smx = max(smx, __shfl_xor(smx, o, 64));
    }
    if (tid == 0) {
        red[0] = 0x7fffffff;
        red[1] = 0;
    }
    __syncthreads();
    if ((tid & 63) == 0) {
        atomicMin(&red[0], smn);
        atomicMax(&red[1], smx);
    }
    __syncthreads();
    lo = max(1, red[0]);
    hi = red[1];
    __syncthreads();
}

// One thread's 16-key chunk of the sink scan: raw flags and segment ids,
// loaded first and evaluated once the rows' segment range is known.
struct SinkChunk {
    uint4 pre;    // 16 sink flags (bytes)
    int4 seg[4];  // 16 segment ids (only when seg_row != NULL)
};

__device__ __forceinline__ void sink_chunk_load(const uint8_t* prefix_row, const int32_t* seg_row, int i0,
                                                bool aligned16, SinkChunk& c) {
    if (aligned16) {
        c.pre = *(const uint4*)(prefix_row + i0);
        if (seg_row) {
            for (int g = 0; g < 4; ++g) c.seg[g] = *(const int4*)(seg_row + i0 + 4 * g);
        }
    } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        for (int j = 0; j < 16; ++j) w[j >> 2] |= (uint32_t)prefix_row[i0 + j] << (8 * (j & 3));
        c.pre = make_uint4(w[0], w[1], w[2], w[3]);
        if (seg_row) {
            for (int g = 0; g < 4; ++g)
                c.seg[g] = make_int4(seg_row[i0 + 4 * g], seg_row[i0 + 4 * g + 1], seg_row[i0 + 4 * g + 2],
                                     seg_row[i0 + 4 * g + 3]);
        }
    }
}

// True when some key of the chunk is a sink whose segment lies in [lo, hi].
__device__ __forceinline__ bool sink_chunk_hit(const SinkChunk& c, bool has_seg, int lo, int hi) {
    const uint32_t pws[4] = {c.pre.x, c.pre.y, c.pre.z, c.pre.w};
    bool f = false;
    for (int g = 0; g < 4; ++g) {
        const int ss[4] = {c.seg[g].x, c.seg[g].y, c.seg[g].z, c.seg[g].w};
        for (int j = 0; j < 4; ++j) {
            const int s = has_seg ? ss[j] : 1;
            f |= (((pws[g] >> (8 * j)) & 0xffu) != 0u) & (s >= lo) & (s <= hi);
        }
    }
    return f;
}

// Block-wide scan over keys [0, n_keys) (n_keys a multiple of 16): bit t of
// `bits` (LDS, ceil(n_keys / BN / 32) words) is set when key tile t of BN
// keys holds a sink whose segment lies in [lo, hi] -- the only sinks rows of
// those segments can see.  `first` (optional) is this thread's chunk at keys
// [16 * tid, 16 * tid + 16), loaded in advance.  Ends with a barrier.
__device__ __forceinline__ void scan_sink_tiles(const uint8_t* prefix_row, const int32_t* seg_row, int n_keys,
                                                int BN, int lo, int hi, bool aligned16, uint32_t* bits, int tid,
                                                int nthreads, const SinkChunk* first = nullptr) {
    const int ntiles = (n_keys + BN - 1) / BN;
    const int nwords = (ntiles + 31) / 32;
    for (int w = tid; w < nwords; w += nthreads) bits[w] = 0u;
    __syncthreads();
    if (hi >= lo) {
        for (int i0 = 16 * tid; i0 < n_keys; i0 += 16 * nthreads) {
            SinkChunk c;
            if (first != nullptr && i0 == 16 * tid) c = *first;
            else sink_chunk_load(prefix_row, seg_row, i0, aligned16, c);
            if (sink_chunk_hit(c, seg_row != nullptr, lo, hi)) {
                const int t = i0 / BN;
                atomicOr(&bits[t >> 5], 1u << (t & 31));
            }
        }
    }
    __syncthreads();
}

// Block-wide segment range [lo, hi] from per-lane row segments (rows past
// the end pass has_row = false).  red is 2 ints of LDS scratch.  Ends with a
// barrier.
__device__ __forceinline__ void row_segment_range_from_lanes(int seg, bool has_row, int* red, int tid, int& lo,
                                                             int& hi) {
    int smn = has_row ? seg : 0x7fffffff, smx = has_row ? seg : 0;
    for (int o = 1; o < 64; o <<= 1) {
        smn = min(smn, __shfl_xor(smn, o, 64));
        smx = max(smx, __shfl_xor(smx, o, 64));
    }
    if (tid == 0) {
        red[0] = 0x7fffffff;
        red[1] = 0;
    }
    __syncthreads();
    if ((tid & 63) == 0) {
        atomicMin(&red[0], smn);
        atomicMax(&red[1], smx);
    }
    __syncthreads();
    lo = max(1, red[0]);
    hi = red[1];
    __syncthreads();
}

// Sink tiles of a workgroup with rows [q0, q1]: row segment range, then scan.
__device__ __forceinline__ void plan_sink_tiles(const TilePlan& plan, const int32_t* seg_row,
                                                const uint8_t* prefix_row, int T, int q0, int q1, int BN, int* red,
                                                uint32_t* bits, int tid, int nthreads) {
    if (plan.sink_keys <= 0) return;
    int lo, hi;
    row_segment_range(seg_row, q0, q1, red, tid, nthreads, lo, hi);
    scan_sink_tiles(prefix_row, seg_row, plan.sink_keys, BN, lo, hi, (T & 15) == 0, bits, tid, nthreads);
}

// Walks a TilePlan: the window band first (its first tile is known before any
// sink scan, so its loads can start at once), then the pooled tiles or the
// sink tiles.  Every thread of a workgroup walks the same sequence; the order
// does not change the result (one softmax over all visited keys).
struct TileIter {
    int phase;  // 0 band, 1 pooled, 2 sinks, 3 done
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
        idx = p.band_lo;
        word = -1;
        bits = 0u;
    }

    __device__ __forceinline__ bool next(int& kind, int& tile) {
        if (phase == 0) {
            if (idx <= plan.band_hi) {
                kind = COL_EXACT;
                tile = idx++;
                return true;
            }
            phase = plan.n_pooled > 0 ? 1 : 2;
            idx = 0;
        }
        if (phase == 1) {
            if (idx < plan.n_pooled) {
                kind = COL_POOLED;
                tile = idx++;
                return true;
            }
            return false;
        }
        if (phase == 2) {
            while (bits == 0u) {
                if (++word >= sink_words) return false;
                bits = sink_bits[word];
            }
            const int b = __builtin_ctz(bits);
            bits &= bits - 1u;
            kind = COL_EXACT;
            tile = word * 32 + b;
            return true;
        }
        return false;
    }
};

}  // namespace swa
