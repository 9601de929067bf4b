// prefill_bf16.hip -- bf16 prefill attention on gfx950 MFMA.
//
// Computes softmax attention under the packing & causal & (recent | sink)
// mask of [NW] "How the 256-Token Sliding Window Works with Tools as KV Sinks
// in Needle" (section "KV Sinks for Tools: Pinning Critical Context"), and the
// compressed-column variant of [CA] "Compressed attention and the copy probe"
// (sections "Two kinds of columns, pooled blocks and exact recent keys" and
// "Pool before rotating, not after").
//
// Work decomposition.  A workgroup owns one (batch, kv head) pair and
// 32 * rbs query rows for hpw query heads of that kv head's GQA group; each
// of its hpw * rbs waves owns 32 rows of one head.  The heads of a group share
// every K/V tile the workgroup stages in LDS.
//
// Per key tile of 64 keys (K row-major, V transposed in LDS), each wave works
// on two 32-key sub-tiles:
//   S^T = K Q^T      4 x v_mfma_f32_32x32x16_bf16 (keys are the M rows)
//   online softmax   per query = per lane column, so the running max, sum
//                    and rescale are lane-local (one xor-32 exchange for max)
//   O^T += V^T P^T   2 x 2 MFMAs; P^T comes straight from the S^T registers
// Sub-tiles the mask hides completely are skipped, sub-tiles it shows
// completely skip the element predicate (swa_tiles.h).
#include "swa_common.h"
#include "swa_internal.h"
#include "swa_tiles.h"

namespace swa {
namespace {

constexpr int BN = 64;   // keys per LDS tile
constexpr int SUB = 32;  // keys per MFMA sub-tile
constexpr int kSinkWords = (kMaxT / BN + 31) / 32;

template <int D>
struct SmemBf16 {
    uint16_t ks[BN][D + 8];  // K tile, row-major, padded rows
    uint16_t vt[D][BN + 8];  // V tile, transposed (key-contiguous per channel)
    int kseg[BN];
    uint8_t ksink[BN];
    int ksum[BN / SUB][4];  // per sub-tile: seg min, seg max, any sink, all sink
    uint32_t sink_bits[kSinkWords];
};

__device__ __forceinline__ void unpack8(const uint4& x, float* f) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ uint4 pack8(const float* f) {
    uint4 r;
    r.x = pack_bf16x2(f[0], f[1]);
    r.y = pack_bf16x2(f[2], f[3]);
    r.z = pack_bf16x2(f[4], f[5]);
    r.w = pack_bf16x2(f[6], f[7]);
    return r;
}

// Rotate-half RoPE of 8 channel pairs: x1 holds channels d..d+7 (< D/2), x2
// holds d+D/2..d+D/2+7; cs/sn point at the table entries of channels d..d+7.
__device__ __forceinline__ void rotate8(uint4& x1, uint4& x2, const float* cs, const float* sn) {
    float a[8], bb[8], c[8], s[8];
    unpack8(x1, a);
    unpack8(x2, bb);
    *(float4*)&c[0] = *(const float4*)cs;
    *(float4*)&c[4] = *(const float4*)(cs + 4);
    *(float4*)&s[0] = *(const float4*)sn;
    *(float4*)&s[4] = *(const float4*)(sn + 4);
    float y1[8], y2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        y1[i] = a[i] * c[i] - bb[i] * s[i];
        y2[i] = bb[i] * c[i] + a[i] * s[i];
    }
    x1 = pack8(y1);
    x2 = pack8(y2);
}

template <int D, bool ROPE>
__device__ __forceinline__ void stage_tile(const PrefillArgs& a, SmemBf16<D>& sm, int kind, int tile, int b,
                                           int hkv, int tid, int nthreads) {
    const bool pooled = kind == COL_POOLED;
    const int nkeys = pooled ? a.nblk : a.T;
    const size_t head_off = ((size_t)b * a.Hkv + hkv) * (size_t)nkeys * D;
    const uint16_t* kg = (const uint16_t*)(pooled ? a.pk : a.k) + head_off;
    const uint16_t* vg = (const uint16_t*)(pooled ? a.pv : a.v) + head_off;
    const int k0 = tile * BN;

    // K: element e -> key e / P, chunk pair (p, p + P) of 8 channels each.
    constexpr int P = D / 16;
    for (int e = tid; e < BN * P; e += nthreads) {
        const int key = e / P, p = e % P, gk = k0 + key;
        uint4 x1 = make_uint4(0, 0, 0, 0), x2 = make_uint4(0, 0, 0, 0);
        if (gk < nkeys) {
            x1 = *(const uint4*)(kg + (size_t)gk * D + 8 * p);
            x2 = *(const uint4*)(kg + (size_t)gk * D + 8 * p + D / 2);
            if (ROPE && !pooled)
                rotate8(x1, x2, a.rope_cos + (size_t)gk * (D / 2) + 8 * p,
                        a.rope_sin + (size_t)gk * (D / 2) + 8 * p);
        }
        *(uint4*)&sm.ks[key][8 * p] = x1;
        *(uint4*)&sm.ks[key][8 * p + D / 2] = x2;
    }

    // V, transposed: element e -> key pair kp, channel chunk dc.
    constexpr int DC = D / 8;
    for (int e = tid; e < (BN / 2) * DC; e += nthreads) {
        const int kp = e % (BN / 2), dc = e / (BN / 2);
        const int g0 = k0 + 2 * kp;
        uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
        if (g0 < nkeys) v0 = *(const uint4*)(vg + (size_t)g0 * D + 8 * dc);
        if (g0 + 1 < nkeys) v1 = *(const uint4*)(vg + (size_t)(g0 + 1) * D + 8 * dc);
        const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w};
        const uint32_t w1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(uint32_t*)&sm.vt[8 * dc + 2 * i][2 * kp] = (w0[i] & 0xffffu) | (w1[i] << 16);
            *(uint32_t*)&sm.vt[8 * dc + 2 * i + 1][2 * kp] = (w0[i] >> 16) | (w1[i] & 0xffff0000u);
        }
    }

    // Key segment / sink flags and per-sub-tile summaries (wave 0; BN == 64).
    if (tid < BN) {
        const int gk = k0 + tid;
        const bool valid = gk < nkeys;
        int s = 0, sk = 0;
        if (!pooled && valid) {
            s = a.seg ? a.seg[(size_t)b * a.T + gk] : 1;
            sk = a.prefix ? (a.prefix[(size_t)b * a.T + gk] != 0) : 0;
        }
        sm.kseg[tid] = s;
        sm.ksink[tid] = (uint8_t)sk;
        int smin = valid ? s : 0x7fffffff;
        int smax = valid ? s : (int)0x80000000;
        int any = (valid && sk) ? 1 : 0;
        int all = (!valid || sk) ? 1 : 0;
        smin = wave_imin_xor(smin, 1, 16);
        smax = wave_imax_xor(smax, 1, 16);
        any = wave_imax_xor(any, 1, 16);
        all = wave_imin_xor(all, 1, 16);
        if ((tid & 31) == 0) {
            sm.ksum[tid >> 5][0] = smin;
            sm.ksum[tid >> 5][1] = smax;
            sm.ksum[tid >> 5][2] = any;
            sm.ksum[tid >> 5][3] = all;
        }
    }
}

template <int D, bool ROPE>
__global__ __launch_bounds__(256) void prefill_bf16_kernel(PrefillArgs a) {
    static_assert(D == 32 || D == 64, "head dim");
    __shared__ __align__(16) SmemBf16<D> sm;
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int lq = lane & 31;

    const int T = a.T;
    const int G = a.Hq / a.Hkv;
    const int groups = G / a.hpw;
    const int b = blockIdx.z;
    const int hkv = blockIdx.y / groups;
    const int hsub = blockIdx.y % groups;
    const int wg_rows = 32 * a.rbs;
    const int q0 = blockIdx.x * wg_rows;
    const int q1 = min(q0 + wg_rows - 1, T - 1);
    const int my_h = hkv * G + hsub * a.hpw + (wave % a.hpw);
    const int r0 = q0 + 32 * (wave / a.hpw);
    const bool wave_active = r0 < T;
    const int my_q = r0 + lq;
    const bool row_ok = my_q < T;
    const bool plain = a.block == 0;

    // Q^T operand: lane holds row my_q, channels 16c + 8h .. +7 for each c.
    bf16x8 qf[D / 16];
    {
        uint4 raw[D / 16];
        const uint16_t* qrow = (const uint16_t*)a.q + (((size_t)b * a.Hq + my_h) * T + (row_ok ? my_q : 0)) * D;
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
            raw[c] = row_ok ? *(const uint4*)(qrow + 16 * c + 8 * h) : make_uint4(0, 0, 0, 0);
        if (ROPE && row_ok) {
#pragma unroll
            for (int c = 0; c < D / 32; ++c) {
                const int d0 = 16 * c + 8 * h;
                rotate8(raw[c], raw[c + D / 32], a.rope_cos + (size_t)my_q * (D / 2) + d0,
                        a.rope_sin + (size_t)my_q * (D / 2) + d0);
            }
        }
#pragma unroll
        for (int c = 0; c < D / 16; ++c) qf[c] = __builtin_bit_cast(bf16x8, raw[c]);
    }

    // Rows of this wave: segment ids and their range.
    int seg_q = 0;
    if (row_ok) seg_q = a.seg ? a.seg[(size_t)b * T + my_q] : 1;
    RowSum rs;
    rs.r0 = r0;
    rs.r1 = min(r0 + 31, T - 1);
    rs.smin = wave_imin_xor(row_ok ? seg_q : 0x7fffffff, 1, 16);
    rs.smax = wave_imax_xor(row_ok ? seg_q : (int)0x80000000, 1, 16);

    const TilePlan plan = plan_tiles(q0, q1, a.window, a.block, a.nblk, a.prefix != nullptr, BN);
    if (plan.sink_keys > 0)
        scan_sink_tiles(a.prefix + (size_t)b * T, plan.sink_keys, BN, sm.sink_bits, tid, nthreads);
    TileIter it;
    it.init(plan, sm.sink_bits, BN);

    const float c_log2 = a.scale * kLog2e;
    float m_run = kNegInf;
    float l_run = 0.f;
    f32x16 o[D / 32];
#pragma unroll
    for (int n = 0; n < D / 32; ++n) o[n] = f32x16{};

    int kind = 0, tile = 0;
    while (it.next(kind, tile)) {
        __syncthreads();
        stage_tile<D, ROPE>(a, sm, kind, tile, b, hkv, tid, nthreads);
        __syncthreads();
        if (!wave_active) continue;
        const int nkeys = kind == COL_POOLED ? a.nblk : T;
#pragma unroll
        for (int st = 0; st < BN / SUB; ++st) {
            const int k0 = tile * BN + st * SUB;
            int cls;
            if (kind == COL_POOLED) {
                cls = classify_pooled(rs, k0, SUB, a.window, a.block, a.nblk);
            } else {
                KeySum ks;
                ks.smin = sm.ksum[st][0];
                ks.smax = sm.ksum[st][1];
                ks.any_sink = sm.ksum[st][2];
                ks.all_sink = sm.ksum[st][3];
                cls = classify_exact(rs, ks, k0, SUB, nkeys, a.window, plain);
            }
            if (cls == TILE_SKIP) continue;

            f32x16 s = f32x16{};
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const bf16x8 ka = *(const bf16x8*)&sm.ks[st * SUB + lq][16 * c + 8 * h];
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[c], s, 0, 0, 0);
            }
            // Scores leave the accumulator into plain registers; the mask is applied
            // with selects (no divergent writes into the MFMA result vector).
            float sv[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) sv[j] = s[j];
            if (cls == TILE_PARTIAL) {
                const int pooled_n = (kind == COL_POOLED && row_ok)
                                         ? pooled_visible_count(my_q, a.window, a.block, a.nblk)
                                         : 0;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int kidx = st * SUB + 8 * (j >> 2) + 4 * h + (j & 3);
                    const int gk = tile * BN + kidx;
                    bool vis;
                    if (kind == COL_POOLED) {
                        vis = gk < pooled_n;
                    } else if (plain) {
                        const int seg_k = sm.kseg[kidx];
                        const bool sink_k = sm.ksink[kidx] != 0;
                        vis = visible_plain(seg_q, seg_k, sink_k, my_q, gk, a.window);
                    } else {
                        vis = visible_exact_window(my_q, gk, a.window);
                    }
                    sv[j] = (vis & row_ok) ? sv[j] : kNegInf;
                }
            }
            float mx = sv[0];
#pragma unroll
            for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sv[j]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run, mx);
            const float base = (m_new == kNegInf) ? 0.f : m_new * c_log2;
            const float corr = __builtin_amdgcn_exp2f(m_run * c_log2 - base);
            m_run = m_new;
            float p[16];
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                p[j] = __builtin_amdgcn_exp2f(sv[j] * c_log2 - base);
                psum += p[j];
            }
            l_run = l_run * corr + psum;
#pragma unroll
            for (int n = 0; n < D / 32; ++n) o[n] *= corr;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                uint4 pw;
                pw.x = pack_bf16x2(p[8 * m + 0], p[8 * m + 1]);
                pw.y = pack_bf16x2(p[8 * m + 2], p[8 * m + 3]);
                pw.z = pack_bf16x2(p[8 * m + 4], p[8 * m + 5]);
                pw.w = pack_bf16x2(p[8 * m + 6], p[8 * m + 7]);
                const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
                for (int n = 0; n < D / 32; ++n) {
                    const uint16_t* vrow = &sm.vt[32 * n + lq][st * SUB + 16 * m + 4 * h];
                    uint4 vw;
                    const uint2 lo = *(const uint2*)vrow;
                    const uint2 hi = *(const uint2*)(vrow + 8);
                    vw.x = lo.x;
                    vw.y = lo.y;
                    vw.z = hi.x;
                    vw.w = hi.y;
                    o[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw), pb, o[n], 0, 0, 0);
                }
            }
        }
    }

    if (!wave_active) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (row_ok) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* orow = (uint16_t*)a.out + (((size_t)b * a.Hq + my_h) * T + my_q) * D;
#pragma unroll
        for (int n = 0; n < D / 32; ++n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = 32 * n + 8 * i + 4 * h;
                uint2 w;
                w.x = pack_bf16x2(o[n][4 * i] * inv, o[n][4 * i + 1] * inv);
                w.y = pack_bf16x2(o[n][4 * i + 2] * inv, o[n][4 * i + 3] * inv);
                *(uint2*)(orow + d) = w;
            }
        }
        if (a.lse && h == 0)
            a.lse[((size_t)b * a.Hq + my_h) * T + my_q] = l_tot > 0.f ? m_run * a.scale + __logf(l_tot) : kNegInf;
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
    const int G = a.Hq / a.Hkv;
    const int wg_rows = 32 * a.rbs;
    dim3 grid((a.T + wg_rows - 1) / wg_rows, a.Hkv * (G / a.hpw), a.B);
    dim3 block(64 * a.hpw * a.rbs);
    const bool rope = a.rope_len > 0;
    if (a.D == 64) {
        if (rope) hipLaunchKernelGGL((prefill_bf16_kernel<64, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((prefill_bf16_kernel<64, false>), grid, block, 0, s, a);
    } else {
        if (rope) hipLaunchKernelGGL((prefill_bf16_kernel<32, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((prefill_bf16_kernel<32, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace swa
