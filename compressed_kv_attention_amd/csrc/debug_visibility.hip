// debug_visibility.hip -- writes out the mask exactly as the prefill kernels
// apply it: the workgroup walks the same TileIter over the same TilePlan, and
// each (row group, key sub-tile) pair is classified with the same functions
// (swa_tiles.h).  An element is visible iff its tile was enumerated and its
// pair is FULL and the row passes the lane gate, PARTIAL_POS and the row passes
// the gate and the positional test, or PARTIAL and the element predicate holds.  A tile that the
// iterator yields twice (which would count its keys twice) marks the rows of
// the workgroup with count -1.
#include "swa_common.h"
#include "swa_internal.h"
#include "swa_tiles.h"

namespace swa {
namespace {

constexpr int kDbgMaxT = kDebugMaxT;
constexpr int kDbgMaxRows = 256;
constexpr int kDbgSub = 32;
constexpr int kDbgSubTiles = kDbgMaxT / kDbgSub;  // per column kind

struct DbgGeom {
    int wg_rows, cls_rows, BN;
};

__global__ __launch_bounds__(256) void debug_vis_kernel(PrefillArgs a, DbgGeom g, uint8_t* mask, int32_t* count) {
    __shared__ uint32_t enum_bits[2][kDbgMaxT / 32 / 32 + 1];
    __shared__ uint32_t sink_bits[kDbgMaxT / 32 / 32 + 1];
    __shared__ int row_sum[kDbgMaxRows / 32][4];  // row groups of 32 (MFMA) or 64 (f32)
    __shared__ int key_sum[kDbgSubTiles][4];
    __shared__ int cnt[kDbgMaxRows];
    __shared__ int dup;
    __shared__ int red[2];

    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int T = a.T, b = blockIdx.z;
    const bool plain = a.block == 0;
    const int npool = plain ? 0 : a.nblk;
    const int Tk = npool + T;
    const int q0 = blockIdx.x * g.wg_rows;
    const int q1 = min(q0 + g.wg_rows - 1, T - 1);
    const int nrows = q1 - q0 + 1;
    const int32_t* seg = a.seg ? a.seg + (size_t)b * T : nullptr;
    const uint8_t* pre = a.prefix ? a.prefix + (size_t)b * T : nullptr;

    for (int i = tid; i < 2 * (kDbgMaxT / 32 / 32 + 1); i += nthreads) (&enum_bits[0][0])[i] = 0u;
    for (int i = tid; i < kDbgMaxRows; i += nthreads) cnt[i] = 0;
    if (tid == 0) dup = 0;

    const TilePlan plan = plan_tiles(q0, q1, a.window, a.block, a.nblk, a.prefix != nullptr, g.BN);
    plan_sink_tiles(plan, seg, pre, T, q0, q1, g.BN, red, sink_bits, tid, nthreads);
    __syncthreads();
    if (tid == 0) {
        TileIter it;
        it.init(plan, sink_bits, g.BN);
        int kind, tile;
        while (it.next(kind, tile)) {
            uint32_t& w = enum_bits[kind][tile >> 5];
            const uint32_t bit = 1u << (tile & 31);
            if (w & bit) dup = 1;
            w |= bit;
        }
    }
    // row-group summaries (groups of cls_rows rows starting at q0)
    const int ngroups = (nrows + g.cls_rows - 1) / g.cls_rows;
    for (int gi = tid; gi < ngroups; gi += nthreads) {
        const int r0 = q0 + gi * g.cls_rows;
        const int r1 = min(r0 + g.cls_rows - 1, T - 1);
        int smin = 0x7fffffff, smax = (int)0x80000000;
        for (int r = r0; r <= r1; ++r) {
            const int s = seg ? seg[r] : 1;
            smin = min(smin, s);
            smax = max(smax, s);
        }
        row_sum[gi][0] = r0;
        row_sum[gi][1] = r1;
        row_sum[gi][2] = smin;
        row_sum[gi][3] = smax;
    }
    // exact-column sub-tile summaries (same meaning as the kernels' ballots)
    const int nsub = (T + kDbgSub - 1) / kDbgSub;
    for (int si = tid; si < nsub; si += nthreads) {
        const int k_lo = si * kDbgSub, k_hi = min(si * kDbgSub + kDbgSub, T);
        const int s_first = plain ? (seg ? max(seg[k_lo], 0) : 1) : 0;
        bool uniform = true, any = false, all = true;
        for (int k = k_lo; k < k_hi; ++k) {
            const int s = plain ? (seg ? max(seg[k], 0) : 1) : 0;
            const bool sk = plain && pre && pre[k] != 0;
            uniform &= s == s_first;
            any |= sk;
            all &= sk;
        }
        const KeySum ks = make_key_sum(uniform, s_first, any, all);
        key_sum[si][0] = ks.smin;
        key_sum[si][1] = ks.smax;
        key_sum[si][2] = ks.any_sink;
        key_sum[si][3] = ks.all_sink;
    }
    __syncthreads();

    for (size_t idx = tid; idx < (size_t)nrows * Tk; idx += nthreads) {
        const int r = (int)(idx / Tk);
        const int col = (int)(idx % Tk);
        const int q = q0 + r;
        const int gi = r / g.cls_rows;
        RowSum rs;
        rs.r0 = row_sum[gi][0];
        rs.r1 = row_sum[gi][1];
        rs.smin = row_sum[gi][2];
        rs.smax = row_sum[gi][3];
        const bool pooled = col < npool;
        const int key = pooled ? col : col - npool;
        const int tile = key / g.BN;
        const int kind = pooled ? COL_POOLED : COL_EXACT;
        bool vis = false;
        if (enum_bits[kind][tile >> 5] & (1u << (tile & 31))) {
            const int k0 = (key / kDbgSub) * kDbgSub;
            const int seg_q = plain ? (seg ? seg[q] : 1) : 1;
            const bool row_vis = seg_q > 0;
            int cls;
            unsigned wlim = window_limit(a.window);
            KeySum ks{0, 0, 0, 0};
            if (pooled) {
                cls = classify_pooled(rs, k0, kDbgSub, a.window, a.block, a.nblk);
            } else {
                const int si = key / kDbgSub;
                ks.smin = key_sum[si][0];
                ks.smax = key_sum[si][1];
                ks.any_sink = key_sum[si][2];
                ks.all_sink = key_sum[si][3];
                cls = classify_exact(rs, ks, k0, kDbgSub, T, a.window, plain, wlim);
            }
            if (pooled) {
                if (cls == TILE_FULL) vis = true;
                else if (cls != TILE_SKIP) vis = key < pooled_visible_count(q, a.window, a.block, a.nblk);
            } else if (cls == TILE_FULL) {
                vis = lane_gate(row_vis, plain, seg_q, ks);
            } else if (cls == TILE_PARTIAL_POS) {
                vis = lane_gate(row_vis, plain, seg_q, ks) && visible_pos(q - key, wlim);
            } else if (cls == TILE_PARTIAL) {
                vis = row_vis && visible_full(q - key, wlim, pack_key_info(seg ? seg[key] : 1, pre && pre[key] != 0),
                                              seg_q);
            }
        }
        if (mask) mask[((size_t)b * T + q) * Tk + col] = vis ? 1 : 0;
        if (vis) atomicAdd(&cnt[r], 1);
    }
    __syncthreads();
    for (int r = tid; r < nrows; r += nthreads) count[(size_t)b * T + q0 + r] = dup ? -1 : cnt[r];
}

}  // namespace

hipError_t launch_debug_visibility(const PrefillArgs& a, bool mfma_geom, uint8_t* mask, int32_t* count,
                                   hipStream_t s) {
    DbgGeom g;
    if (mfma_geom) {
        g.wg_rows = 32 * a.rbs;
        g.cls_rows = 32;
        g.BN = 64;
    } else {
        g.wg_rows = 64;
        g.cls_rows = 64;
        g.BN = 32;
    }
    dim3 grid((a.T + g.wg_rows - 1) / g.wg_rows, 1, a.B);
    hipLaunchKernelGGL(debug_vis_kernel, grid, dim3(256), 0, s, a, g, mask, count);
    return hipGetLastError();
}

}  // namespace swa
