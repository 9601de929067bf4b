// prefill_f32.hip -- fp32 prefill attention on the vector ALUs of gfx950.
//
// Same mask, same tile enumeration and same column layout as the bf16 MFMA
// kernel (see swa_tiles.h for the sources), with true fp32 inputs, products
// and accumulation.  One wave per workgroup, one query row per lane; K/V
// tiles of 32 keys are staged in LDS in fp32 and shared by the 64 rows.  With
// RoPE, q is rotated here as it is loaded; the keys arrive already rotated.  Used for fp32 inputs, where the
// tolerance is far tighter than bf16 MFMA inputs allow.
#include "swa_common.h"
#include "swa_internal.h"
#include "swa_tiles.h"

namespace swa {
namespace {

constexpr int BNF = 32;  // keys per tile
constexpr int ROWS = 64; // rows per workgroup
constexpr int kSinkWordsF = (kMaxT / BNF + 31) / 32;

template <int D>
struct SmemF32 {
    float ks[BNF][D + 1];
    float vs[BNF][D + 1];
    int kinfo[BNF];
    int ksum[4];
    uint32_t sink_bits[kSinkWordsF];
};

template <int D, bool ROPE>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
    __shared__ SmemF32<D> sm;
    const int lane = threadIdx.x;
    const int T = a.T;
    const int b = blockIdx.z;
    const int hq = blockIdx.y;
    const int G = a.Hq / a.Hkv;
    const int hkv = hq / G;
    const int q0 = blockIdx.x * ROWS;
    const int q1 = min(q0 + ROWS - 1, T - 1);
    const int my_q = q0 + lane;
    const bool row_ok = my_q < T;
    const bool plain = a.block == 0;

    float qr[D];
    {
        const float* qrow = (const float*)a.q + (((size_t)b * a.Hq + hq) * T + (row_ok ? my_q : 0)) * D;
#pragma unroll
        for (int d = 0; d < D; ++d) qr[d] = row_ok ? qrow[d] : 0.f;
        if (ROPE && row_ok) {
            const float* cs = a.rope_cos + (size_t)my_q * (D / 2);
            const float* sn = a.rope_sin + (size_t)my_q * (D / 2);
#pragma unroll
            for (int i = 0; i < D / 2; ++i) {
                const float x1 = qr[i], x2 = qr[i + D / 2];
                qr[i] = x1 * cs[i] - x2 * sn[i];
                qr[i + D / 2] = x2 * cs[i] + x1 * sn[i];
            }
        }
    }
    int seg_q = 0;
    if (row_ok) seg_q = a.seg ? a.seg[(size_t)b * T + my_q] : 1;
    const bool row_vis = row_ok && (!plain || seg_q > 0);  // padding rows see nothing
    const unsigned wlim = window_limit(a.window);
    RowSum rs;
    rs.r0 = q0;
    rs.r1 = q1;
    rs.smin = wave_imin_xor(row_ok ? seg_q : 0x7fffffff, 1, 32);
    rs.smax = wave_imax_xor(row_ok ? seg_q : (int)0x80000000, 1, 32);

    const TilePlan plan = plan_tiles(q0, q1, a.window, a.block, a.nblk, a.prefix != nullptr, BNF);
    plan_sink_tiles(plan, a.seg ? a.seg + (size_t)b * T : nullptr, a.prefix ? a.prefix + (size_t)b * T : nullptr, T,
                    q0, q1, BNF, sm.ksum, sm.sink_bits, lane, 64);
    TileIter it;
    it.init(plan, sm.sink_bits, BNF);

    float m_run = kNegInf, l_run = 0.f;
    float o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = 0.f;

    int kind = 0, tile = 0;
    while (it.next(kind, tile)) {
        const bool pooled = kind == COL_POOLED;
        const int nkeys = pooled ? a.nblk : T;
        const size_t head_off = ((size_t)b * a.Hkv + hkv) * (size_t)nkeys * D;
        const float* kg = (const float*)(pooled ? a.pk : a.k) + head_off;
        const float* vg = (const float*)(pooled ? a.pv : a.v) + head_off;
        const int k0 = tile * BNF;
        __syncthreads();
        // stage: lane -> (key = e / D, channel = e % D) over the tile
        for (int e = lane; e < BNF * D; e += 64) {
            const int key = e / D, d = e % D, gk = k0 + key;
            float kv = 0.f, vv = 0.f;
            if (gk < nkeys) {
                kv = kg[(size_t)gk * D + d];
                vv = vg[(size_t)gk * D + d];
            }
            sm.ks[key][d] = kv;
            sm.vs[key][d] = vv;
        }
        if (lane < BNF) {
            const int gk = k0 + lane;
            int info = 0;
            if (!pooled && gk < nkeys) {
                const int s = a.seg ? a.seg[(size_t)b * T + gk] : 1;
                const bool sk = a.prefix ? (a.prefix[(size_t)b * T + gk] != 0) : false;
                info = pack_key_info(s, sk);
            }
            sm.kinfo[lane] = info;
        }
        {
            // summary over the 32 keys (lanes 32..63 mirror lanes 0..31)
            const int kl = lane & 31;
            const int gk = k0 + kl;
            const bool valid = gk < nkeys;
            int info = 0;
            if (!pooled && valid) {
                const int s = a.seg ? a.seg[(size_t)b * T + gk] : 1;
                const bool sk = a.prefix ? (a.prefix[(size_t)b * T + gk] != 0) : false;
                info = pack_key_info(s, sk);
            }
            const int sgv = info & 0x7fffffff;
            const int s_first = __builtin_amdgcn_readlane(sgv, 0);
            const uint64_t eq_b = __ballot(!valid || sgv == s_first);
            const uint64_t any_b = __ballot(valid && info < 0);
            const uint64_t all_b = __ballot(!valid || info < 0);
            if (lane == 0) {
                const KeySum ks = make_key_sum((uint32_t)eq_b == 0xffffffffu, s_first, (uint32_t)any_b != 0u,
                                               (uint32_t)all_b == 0xffffffffu);
                sm.ksum[0] = ks.smin;
                sm.ksum[1] = ks.smax;
                sm.ksum[2] = ks.any_sink;
                sm.ksum[3] = ks.all_sink;
            }
        }
        __syncthreads();
        int cls;
        unsigned wl = wlim;
        bool gate = row_vis;
        if (pooled) {
            cls = classify_pooled(rs, k0, BNF, a.window, a.block, a.nblk);
        } else {
            KeySum ks;
            ks.smin = sm.ksum[0];
            ks.smax = sm.ksum[1];
            ks.any_sink = sm.ksum[2];
            ks.all_sink = sm.ksum[3];
            cls = classify_exact(rs, ks, k0, BNF, nkeys, a.window, plain, wl);
            gate = lane_gate(row_vis, plain, seg_q, ks);
        }
        if (cls == TILE_SKIP) continue;
        const int pooled_n = (pooled && row_ok) ? pooled_visible_count(my_q, a.window, a.block, a.nblk) : 0;
        // one key at a time: exact online softmax update (rescale only when the max grows)
#pragma unroll 1
        for (int j = 0; j < BNF; ++j) {
            const int gk = k0 + j;
            bool vis;
            if (pooled) vis = row_vis && (cls == TILE_FULL || gk < pooled_n);
            else if (cls == TILE_FULL) vis = gate;
            else if (cls == TILE_PARTIAL_POS) vis = gate && visible_pos(my_q - gk, wl);
            else vis = row_vis && visible_full(my_q - gk, wlim, sm.kinfo[j], seg_q);
            if (!vis) continue;
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) dot = fmaf(qr[d], sm.ks[j][d], dot);
            const float sj = dot * a.scale;
            if (sj > m_run) {
                const float corr = expf(m_run - sj);
                m_run = sj;
                l_run *= corr;
#pragma unroll
                for (int d = 0; d < D; ++d) o[d] *= corr;
            }
            const float p = expf(sj - m_run);
            l_run += p;
#pragma unroll
            for (int d = 0; d < D; ++d) o[d] = fmaf(p, sm.vs[j][d], o[d]);
        }
    }

    if (!row_ok) return;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* orow = (float*)a.out + (((size_t)b * a.Hq + hq) * T + my_q) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
    if (a.lse) a.lse[((size_t)b * a.Hq + hq) * T + my_q] = l_run > 0.f ? m_run + logf(l_run) : kNegInf;
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
    dim3 grid((a.T + ROWS - 1) / ROWS, a.Hq, a.B);
    dim3 block(64);
    const bool rope = a.rope_len > 0;
    if (a.D == 64) {
        if (rope) hipLaunchKernelGGL((prefill_f32_kernel<64, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((prefill_f32_kernel<64, false>), grid, block, 0, s, a);
    } else {
        if (rope) hipLaunchKernelGGL((prefill_f32_kernel<32, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((prefill_f32_kernel<32, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace swa
