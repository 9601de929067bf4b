// backward.hip -- gradients of the windowed+sink prefill (plain mode).
//
// The packing & causal & (recent | sink) mask of [NW] "How the 256-Token
// Sliding Window Works with Tools as KV Sinks in Needle" (section "KV Sinks
// for Tools: Pinning Critical Context") is the training-side mask ([NS]
// "256-token滑动窗口+KV sink：Needle 2工具钉住机制源码分析", section "KV sink
// 如何「钉住」工具"); the pages give no backward.  These kernels compute the
// plain derivative of the forward, from the forward's output and row lse:
//   P = exp(scale q k^T - lse),  dP = dO v^T,  Delta = rowsum(dO o),
//   dS = P (dP - Delta),  dq = scale dS k,  dk = scale dS^T q,  dv = P^T dO.
// Everything is fp32.  A preparation pass converts q, k, v and dO to fp32
// (rotating q and k when a RoPE table is given) and forms Delta; a
// query-major pass walks each query row's visible keys (the forward's tile
// enumeration) for dq; a key-major pass walks each key's visible queries for
// dk and dv, one query head per wave, and the heads of a GQA group are summed.  With RoPE, dq and
// dk are rotated back (by the negative angle) before they are stored.
//
// Both passes use lane pairs: lanes l and l + 32 of a wave hold the two channel
// halves of one row (rotate-half RoPE pairs channel i with i + D/2, so the
// pair also holds every rotation pair), and each dot product is two partial
// sums added across the pair.
#include "swa_common.h"
#include "swa_internal.h"
#include "swa_tiles.h"

namespace swa {
namespace {

constexpr int BT = 32;  // rows (keys or queries) per staged tile and per wave

template <class X>
__device__ __forceinline__ float load_f(const X* p, size_t i);
template <>
__device__ __forceinline__ float load_f<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

// One row of q (and dO, o) per 64-lane block: lane d < D holds channel d.
// Writes q (rotated at the row's position when a table is given) and dO in
// fp32, and Delta = sum_d dO o.
template <class X>
__global__ __launch_bounds__(64) void bwd_prep_q_kernel(BwdArgs a, float* q32, float* do32, float* delta) {
    const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int D = a.D;
    const size_t row = ((size_t)b * a.Hq + h) * a.T + t;
    const int d = lane % D;
    float x = load_f((const X*)a.q, row * D + d);
    const float go = load_f((const X*)a.dout, row * D + d);
    const float o = load_f((const X*)a.out, row * D + d);
    if (a.rope_cos) {
        const float other = __shfl_xor(x, D / 2, 64);
        const int i = d % (D / 2);
        const float c = a.rope_cos[(size_t)t * (D / 2) + i], s = a.rope_sin[(size_t)t * (D / 2) + i];
        x = d < D / 2 ? x * c - other * s : x * c + other * s;
    }
    float prod = lane < D ? go * o : 0.f;
    for (int off = 1; off < 64; off <<= 1) prod += __shfl_xor(prod, off, 64);
    if (lane < D) {
        q32[row * D + d] = x;
        do32[row * D + d] = go;
    }
    if (lane == 0) delta[row] = prod;
}

// One row of k and v per 64-lane block: k rotated when a table is given.
template <class X>
__global__ __launch_bounds__(64) void bwd_prep_kv_kernel(BwdArgs a, float* k32, float* v32) {
    const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int D = a.D;
    const size_t row = ((size_t)b * a.Hkv + h) * a.T + t;
    const int d = lane % D;
    float x = load_f((const X*)a.k, row * D + d);
    const float vv = load_f((const X*)a.v, row * D + d);
    if (a.rope_cos) {
        const float other = __shfl_xor(x, D / 2, 64);
        const int i = d % (D / 2);
        const float c = a.rope_cos[(size_t)t * (D / 2) + i], s = a.rope_sin[(size_t)t * (D / 2) + i];
        x = d < D / 2 ? x * c - other * s : x * c + other * s;
    }
    if (lane < D) {
        k32[row * D + d] = x;
        v32[row * D + d] = vv;
    }
}

// Rotate a lane pair's halves back by the negative angle at position `pos`:
// (x1, x2) -> (x1 c + x2 s, x2 c - x1 s) for the pair (i, i + D/2).
template <int H>
__device__ __forceinline__ void unrotate_half(float (&g)[H], int half, const BwdArgs& a, int pos) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
        const float other = __shfl_xor(g[i], 32, 64);
        const float c = a.rope_cos[(size_t)pos * H + i], s = a.rope_sin[(size_t)pos * H + i];
        g[i] = half == 0 ? g[i] * c + other * s : g[i] * c - other * s;
    }
}

template <int D>
struct SmemDq {
    float ks[BT][D];  // (rows 16-byte aligned: every lane of a half reads the same row)
    float vs[BT][D];
    int kinfo[BT];
    int ksum[4];
    uint32_t sink_bits[(kMaxT / BT + 31) / 32];
};

// dq: one wave per 32 query rows of one head; lane pair (r, half).
template <int D>
__global__ __launch_bounds__(64) void bwd_dq_kernel(BwdArgs a, const float* q32, const float* k32, const float* v32,
                                                    const float* do32, const float* delta) {
    constexpr int H = D / 2;
    __shared__ SmemDq<D> sm;
    const int lane = threadIdx.x;
    const int r = lane & 31, half = lane >> 5;
    const int T = a.T;
    const int b = blockIdx.z, hq = blockIdx.y;
    const int hkv = hq / (a.Hq / a.Hkv);
    const int q0 = blockIdx.x * BT;
    const int q1 = min(q0 + BT - 1, T - 1);
    const int my_q = q0 + r;
    const bool row_ok = my_q < T;
    const size_t qrow = ((size_t)b * a.Hq + hq) * T + (row_ok ? my_q : 0);
    float qh[H], gh[H], dq[H];
#pragma unroll
    for (int i = 0; i < H; ++i) {
        qh[i] = row_ok ? q32[qrow * D + half * H + i] : 0.f;
        gh[i] = row_ok ? do32[qrow * D + half * H + i] : 0.f;
        dq[i] = 0.f;
    }
    const float lse = row_ok ? a.lse[qrow] : kNegInf;
    const float dlt = row_ok ? delta[qrow] : 0.f;
    int seg_q = 0;
    if (row_ok) seg_q = a.seg ? a.seg[(size_t)b * T + my_q] : 1;
    const bool row_vis = row_ok && seg_q > 0 && lse != kNegInf;
    const unsigned wlim = window_limit(a.window);
    RowSum rs;
    rs.r0 = q0;
    rs.r1 = q1;
    rs.smin = wave_imin_xor(row_ok ? seg_q : 0x7fffffff, 1, 32);
    rs.smax = wave_imax_xor(row_ok ? seg_q : (int)0x80000000, 1, 32);

    const TilePlan plan = plan_tiles(q0, q1, a.window, 0, 0, a.prefix != nullptr, BT);
    plan_sink_tiles(plan, a.seg ? a.seg + (size_t)b * T : nullptr, a.prefix ? a.prefix + (size_t)b * T : nullptr, T,
                    q0, q1, BT, sm.ksum, sm.sink_bits, lane, 64);
    TileIter it;
    it.init(plan, sm.sink_bits, BT);
    const size_t head = ((size_t)b * a.Hkv + hkv) * (size_t)T * D;
    int kind = 0, tile = 0;
    while (it.next(kind, tile)) {
        const int k0 = tile * BT;
        __syncthreads();
        for (int e = lane; e < BT * D; e += 64) {
            const int key = e / D, d = e % D, gk = k0 + key;
            sm.ks[key][d] = gk < T ? k32[head + (size_t)gk * D + d] : 0.f;
            sm.vs[key][d] = gk < T ? v32[head + (size_t)gk * D + d] : 0.f;
        }
        if (lane < BT) {
            const int gk = k0 + lane;
            int info = 0;
            if (gk < T) {
                const int s = a.seg ? a.seg[(size_t)b * T + gk] : 1;
                const bool sk = a.prefix ? (a.prefix[(size_t)b * T + gk] != 0) : false;
                info = pack_key_info(s, sk);
            }
            sm.kinfo[lane] = info;
        }
        __syncthreads();
#pragma unroll 1
        for (int j = 0; j < BT; ++j) {
            const int gk = k0 + j;
            const bool vis = row_vis && gk < T && visible_full(my_q - gk, wlim, sm.kinfo[j], seg_q);
            float sp = 0.f, dp = 0.f;
#pragma unroll
            for (int i = 0; i < H; ++i) {
                sp = fmaf(qh[i], sm.ks[j][half * H + i], sp);
                dp = fmaf(gh[i], sm.vs[j][half * H + i], dp);
            }
            sp += __shfl_xor(sp, 32, 64);
            dp += __shfl_xor(dp, 32, 64);
            if (!vis) continue;
            const float p = expf(sp * a.scale - lse);
            const float ds = p * (dp - dlt) * a.scale;
#pragma unroll
            for (int i = 0; i < H; ++i) dq[i] = fmaf(ds, sm.ks[j][half * H + i], dq[i]);
        }
    }
    if (a.rope_cos) unrotate_half<H>(dq, half, a, row_ok ? my_q : 0);
    if (!row_ok) return;
#pragma unroll
    for (int i = 0; i < H; ++i) a.dq[qrow * D + half * H + i] = dq[i];
}

template <int D>
struct SmemDkv {
    float qs[BT][D];
    float gs[BT][D];
    float lse[BT];
    float dlt[BT];
    int seg[BT];
};

// dk, dv: one wave per 32 keys and one query head; lane pair (r, half).  The
// queries that can see a key of the block: the rows from the block's first
// key to its last key + W - 1 (every row after it without a window), and,
// when the block holds sink keys, every later row of their segments.  With
// GQA groups of G > 1 heads each head's share goes to the per-head buffers
// pk/pv ([B][Hq][T][D]) and bwd_sum_heads_kernel adds them in head order.
template <int D>
__global__ __launch_bounds__(64) void bwd_dkv_kernel(BwdArgs a, const float* q32, const float* k32, const float* v32,
                                                     const float* do32, const float* delta, float* pk, float* pv) {
    constexpr int H = D / 2;
    __shared__ SmemDkv<D> sm;
    const int lane = threadIdx.x;
    const int r = lane & 31, half = lane >> 5;
    const int T = a.T;
    const int b = blockIdx.z, hq = blockIdx.y;
    const int G = a.Hq / a.Hkv;
    const int hkv = hq / G;
    const int s0 = blockIdx.x * BT;
    const int my_k = s0 + r;
    const bool key_ok = my_k < T;
    const size_t krow = ((size_t)b * a.Hkv + hkv) * T + (key_ok ? my_k : 0);
    float kh[H], vh[H], dk[H], dv[H];
#pragma unroll
    for (int i = 0; i < H; ++i) {
        kh[i] = key_ok ? k32[krow * D + half * H + i] : 0.f;
        vh[i] = key_ok ? v32[krow * D + half * H + i] : 0.f;
        dk[i] = 0.f;
        dv[i] = 0.f;
    }
    int seg_k = 0;
    bool sink_k = false;
    if (key_ok) {
        seg_k = a.seg ? a.seg[(size_t)b * T + my_k] : 1;
        sink_k = a.prefix ? a.prefix[(size_t)b * T + my_k] != 0 : false;
    }
    const int info_k = pack_key_info(seg_k, sink_k);
    const unsigned wlim = window_limit(a.window);
    // rows to walk: the band, and with sinks in the block every later row of their segments
    const int s1 = min(s0 + BT - 1, T - 1);
    const int band_end = a.window != 0 ? min(T - 1, s1 + a.window - 1) : T - 1;
    const bool has_sink = a.window != 0 && __ballot(key_ok && sink_k && seg_k > 0) != 0;
    const int sk_lo = wave_imin_xor(key_ok && sink_k && seg_k > 0 ? seg_k : 0x7fffffff, 1, 32);
    const int sk_hi = wave_imax_xor(key_ok && sink_k && seg_k > 0 ? seg_k : (int)0x80000000, 1, 32);
    const int last = has_sink ? T - 1 : band_end;
    for (int t0 = (s0 / BT) * BT; t0 <= last; t0 += BT) {
        // a tile past the band matters only if one of its rows is in a sink segment of the block
        if (t0 > band_end) {
            const int tq = t0 + (lane & 31);
            const int sq = tq < T ? (a.seg ? a.seg[(size_t)b * T + tq] : 1) : 0;
            if (__ballot(sq >= sk_lo && sq <= sk_hi) == 0) continue;
        }
        {
            const size_t qhead = ((size_t)b * a.Hq + hq) * (size_t)T;
            __syncthreads();
            for (int e = lane; e < BT * D; e += 64) {
                const int qi = e / D, d = e % D, tq = t0 + qi;
                sm.qs[qi][d] = tq < T ? q32[(qhead + tq) * D + d] : 0.f;
                sm.gs[qi][d] = tq < T ? do32[(qhead + tq) * D + d] : 0.f;
            }
            if (lane < BT) {
                const int tq = t0 + lane;
                sm.lse[lane] = tq < T ? a.lse[qhead + tq] : kNegInf;
                sm.dlt[lane] = tq < T ? delta[qhead + tq] : 0.f;
                sm.seg[lane] = tq < T ? (a.seg ? a.seg[(size_t)b * T + tq] : 1) : 0;
            }
            __syncthreads();
#pragma unroll 1
            for (int j = 0; j < BT; ++j) {
                const int tq = t0 + j;
                const int sq = sm.seg[j];
                const bool vis = key_ok && tq < T && sq > 0 && sm.lse[j] != kNegInf &&
                                 visible_full(tq - my_k, wlim, info_k, sq);
                float sp = 0.f, dp = 0.f;
#pragma unroll
                for (int i = 0; i < H; ++i) {
                    sp = fmaf(sm.qs[j][half * H + i], kh[i], sp);
                    dp = fmaf(sm.gs[j][half * H + i], vh[i], dp);
                }
                sp += __shfl_xor(sp, 32, 64);
                dp += __shfl_xor(dp, 32, 64);
                if (!vis) continue;
                const float p = expf(sp * a.scale - sm.lse[j]);
                const float ds = p * (dp - sm.dlt[j]) * a.scale;
#pragma unroll
                for (int i = 0; i < H; ++i) {
                    dv[i] = fmaf(p, sm.gs[j][half * H + i], dv[i]);
                    dk[i] = fmaf(ds, sm.qs[j][half * H + i], dk[i]);
                }
            }
        }
    }
    if (a.rope_cos) unrotate_half<H>(dk, half, a, key_ok ? my_k : 0);
    if (!key_ok) return;
    float* ok = G == 1 ? a.dk + krow * D : pk + (((size_t)b * a.Hq + hq) * T + my_k) * D;
    float* ov = G == 1 ? a.dv + krow * D : pv + (((size_t)b * a.Hq + hq) * T + my_k) * D;
#pragma unroll
    for (int i = 0; i < H; ++i) {
        ok[half * H + i] = dk[i];
        ov[half * H + i] = dv[i];
    }
}

// dk, dv of a kv head = the sum of its G query heads' shares, in head order.
__global__ void bwd_sum_heads_kernel(BwdArgs a, const float* pk, const float* pv) {
    const int G = a.Hq / a.Hkv;
    const long long n = (long long)a.B * a.Hkv * a.T * a.D;
    const long long per_head = (long long)a.T * a.D;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
        const long long bh = i / per_head, e = i % per_head;  // bh = b * Hkv + hkv
        const long long src = (bh * G) * per_head + e;         // first query head of the group
        float sk = 0.f, sv = 0.f;
        for (int g = 0; g < G; ++g) {
            sk += pk[src + g * per_head];
            sv += pv[src + g * per_head];
        }
        a.dk[i] = sk;
        a.dv[i] = sv;
    }
}

// ---- bf16 inputs: the same gradients on bf16 matrix instructions ---------
//
// The operands are those of the forward's MFMA kernel: q rotated and scaled
// by scale * log2 e (rounded to bf16 once), k rotated (rounded once), v and
// dO as given; P = exp2(s' - lse log2 e) comes out in fp32 and enters the
// gradient products rounded to bf16, as P does in the forward.  Sub-tiles are
// 32 x 32 with the forward's operand layouts (transposed LDS reads for the
// operands whose rows are the reduction dimension):
//   query-major, per 32 keys:  S^T = K Q'^T,  dP^T = V dO^T,
//                              dS^T = P^T (dP^T - Delta),  dQ^T += K^T dS^T
//   key-major, per 32 queries: S = Q' K^T,  dP = dO V^T,  dS = P (dP - Delta),
//                              dV^T += dO^T P,  dK^T += Q'^T dS
// dq = scale dQ, dk = dK / log2 e (Q' carries scale log2 e), dv = dV.

__device__ __forceinline__ uint32_t bwd_pk_bf16(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

// q' = bf16((rotate(q) at t) * scale * log2 e) and Delta = sum dO o, one
// thread per (row, 8 channel pairs: channels i0 .. i0+7 and their partners
// i0 + D/2 ..); a row's D/16 threads are adjacent.  16-byte accesses.
__device__ __forceinline__ void unpack8_bf16(const uint4& x, float* f) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__global__ __launch_bounds__(256) void bwd_prep_bf16_q_kernel(BwdArgs a, uint16_t* qs, float* delta) {
    const int D = a.D, H = D / 2, per_row = H / 8;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long rows = (long long)a.B * a.Hq * a.T;
    const bool ok = idx < rows * per_row;
    const long long row = ok ? idx / per_row : 0;
    const int i0 = (int)(idx - row * per_row) * 8;
    const int t = (int)(row % a.T);
    const size_t base = (size_t)row * D + i0;
    const float mul = a.scale * kLog2e;
    float part = 0.f;
    if (ok) {
        float x1[8], x2[8], g1[8], g2[8], o1[8], o2[8];
        unpack8_bf16(*(const uint4*)((const uint16_t*)a.q + base), x1);
        unpack8_bf16(*(const uint4*)((const uint16_t*)a.q + base + H), x2);
        unpack8_bf16(*(const uint4*)((const uint16_t*)a.dout + base), g1);
        unpack8_bf16(*(const uint4*)((const uint16_t*)a.dout + base + H), g2);
        unpack8_bf16(*(const uint4*)((const uint16_t*)a.out + base), o1);
        unpack8_bf16(*(const uint4*)((const uint16_t*)a.out + base + H), o2);
        if (a.rope_cos) {
            const float4 c0 = *(const float4*)(a.rope_cos + (size_t)t * H + i0);
            const float4 c1 = *(const float4*)(a.rope_cos + (size_t)t * H + i0 + 4);
            const float4 s0 = *(const float4*)(a.rope_sin + (size_t)t * H + i0);
            const float4 s1 = *(const float4*)(a.rope_sin + (size_t)t * H + i0 + 4);
            const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float y1 = x1[e] * c[e] - x2[e] * sn[e], y2 = x2[e] * c[e] + x1[e] * sn[e];
                x1[e] = y1;
                x2[e] = y2;
            }
        }
        uint32_t w1[4], w2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w1[i] = bwd_pk_bf16(x1[2 * i] * mul, x1[2 * i + 1] * mul);
            w2[i] = bwd_pk_bf16(x2[2 * i] * mul, x2[2 * i + 1] * mul);
        }
        *(uint4*)(qs + base) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
        *(uint4*)(qs + base + H) = make_uint4(w2[0], w2[1], w2[2], w2[3]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            part = fmaf(g1[e], o1[e], part);
            part = fmaf(g2[e], o2[e], part);
        }
    }
    // the row's per_row (2 or 4) adjacent threads add their parts
    for (int off = 1; off < per_row; off <<= 1) part += __shfl_xor(part, off, 64);
    if (ok && i0 == 0) delta[row] = part;
}

// k rotated at its position, rounded to bf16 once (the forward's key pre-pass).
__global__ __launch_bounds__(256) void bwd_prep_bf16_k_kernel(BwdArgs a, uint16_t* ks) {
    const int D = a.D, H = D / 2, per_row = H / 8;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long rows = (long long)a.B * a.Hkv * a.T;
    if (idx >= rows * per_row) return;
    const long long row = idx / per_row;
    const int i0 = (int)(idx - row * per_row) * 8;
    const int t = (int)(row % a.T);
    const uint16_t* k = (const uint16_t*)a.k + row * D;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x1 = bf16_bits_to_f32(k[i0 + e]), x2 = bf16_bits_to_f32(k[H + i0 + e]);
        const float c = a.rope_cos[(size_t)t * H + i0 + e], sn = a.rope_sin[(size_t)t * H + i0 + e];
        ks[row * D + i0 + e] = (uint16_t)f32_to_bf16_bits(x1 * c - x2 * sn);
        ks[row * D + H + i0 + e] = (uint16_t)f32_to_bf16_bits(x2 * c + x1 * sn);
    }
}

// LDS tiles of 32 rows, row-major with a 16-byte pad per row.
template <int D>
struct Bf16Tile {
    static constexpr int RS = D + 8;  // row stride in bf16
    uint16_t x[32 * RS];
};
// The 32 rows (src + r * D, rows >= nrows read as zero) of a tile, 16 bytes
// per lane per piece, as one wave loads them: every load is issued before any
// of the stores below, so staging a tile costs one memory round trip.
template <int D>
struct TileRows {
    static constexpr int CPR = D / 8;           // 16-byte pieces per row
    static constexpr int PER = 32 * CPR / 64;   // pieces per lane
    u32x4 x[PER];  // a plain vector type: copies of an aggregate would go through memory
    // Every lane loads, rows past the end (nrows >= 1) from the last row, so that
    // no load sits under a branch.  Those copies are finite data whose products
    // the mask sends to zero: their rows are invisible to every key.
    __device__ __forceinline__ void load(const uint16_t* src, int nrows, int lane) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int piece = lane + 64 * i, r = piece / CPR, c = piece % CPR;
            x[i] = *(const u32x4*)(src + (size_t)(r < nrows ? r : nrows - 1) * D + 8 * c);
        }
    }
    __device__ __forceinline__ void store(Bf16Tile<D>& t, int lane) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int piece = lane + 64 * i, r = piece / CPR, c = piece % CPR;
            *(u32x4*)&t.x[r * Bf16Tile<D>::RS + 8 * c] = x[i];
        }
    }
};
// Operand of the sub-tile's rows (A operand: row l % 32, channels 16c + 8 (l / 32) ..).
template <int D>
__device__ __forceinline__ bf16x8 tile_row(const Bf16Tile<D>& t, int c, int lane) {
    return __builtin_bit_cast(bf16x8, *(const uint4*)&t.x[(lane & 31) * Bf16Tile<D>::RS + 16 * c + 8 * (lane >> 5)]);
}
// Transposed operand (A operand of a product whose reduction runs over the
// tile's rows): rows 16m .. 16m + 15 and channels 32n .. 32n + 31, from two
// transposing reads per 8 rows (the forward's V^T reads on a plain layout).
template <int D>
__device__ __forceinline__ bf16x8 tile_tr(const Bf16Tile<D>& t, int m, int n, int lane) {
    const int g = lane >> 4, hh = g >> 1, j = lane & 15, r = j >> 2, a4 = j & 3;
    const int ch = 32 * n + 16 * (g & 1) + 4 * a4;
    const uint32_t base = lds_off(&t.x[0]);
    const u32x2 lo = lds_load_tr16(base + (uint32_t)(((16 * m + 4 * hh + r) * Bf16Tile<D>::RS + ch) * 2));
    const u32x2 hi = lds_load_tr16(base + (uint32_t)(((16 * m + 8 + 4 * hh + r) * Bf16Tile<D>::RS + ch) * 2));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}
// B operand of a row of global memory (row r's channels 16c + 8 (l / 32) ..).
__device__ __forceinline__ bf16x8 row_operand(const uint16_t* row, int c, int lane) {
    return __builtin_bit_cast(bf16x8, *(const uint4*)(row + 16 * c + 8 * (lane >> 5)));
}
// The 16 accumulator values of a lane as the bf16 B operands of the two
// 16-row steps (elements 8m .. 8m + 7).
__device__ __forceinline__ void pack_steps(const float (&x)[16], bf16x8 (&b)[2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
        b[m] = __builtin_bit_cast(bf16x8, make_uint4(bwd_pk_bf16(x[8 * m], x[8 * m + 1]), bwd_pk_bf16(x[8 * m + 2], x[8 * m + 3]),
                                                     bwd_pk_bf16(x[8 * m + 4], x[8 * m + 5]),
                                                     bwd_pk_bf16(x[8 * m + 6], x[8 * m + 7])));
}

template <int D>
struct SmemDqMfma {
    Bf16Tile<D> k, v;
    __attribute__((aligned(16))) int kinfo[32];
    int red[4];
    uint32_t sink_bits[(kMaxT / BT + 31) / 32];
};

// dq: a workgroup of four waves per 32 query rows and four query heads of one
// GQA group (one head per wave; they share every staged K/V tile); the
// forward's walk over key tiles of 32 (band first, then the tiles holding
// visible sinks).
template <int D>
// (four waves per SIMD: a launch of the needle's size then fits in one round,
// at the cost of a few registers kept in scratch)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void bwd_dq_mfma_kernel(BwdArgs a, const uint16_t* qs, const uint16_t* kr,
                                                          const float* delta) {
    constexpr int NC = D / 16;
    __shared__ __align__(16) SmemDqMfma<D> sm;
    const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, h = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = a.T;
    const int G = a.Hq / a.Hkv, ngs = (G + 3) / 4;
    const int b = blockIdx.z, hkv = blockIdx.y / ngs;
    const int gh = (blockIdx.y - hkv * ngs) * 4 + wave;  // head within the group
    const bool wave_on = gh < G;  // (waves past the group's last head only stage tiles)
    const int hq = hkv * G + min(gh, G - 1);
    const int q0 = blockIdx.x * BT;
    const int q1 = min(q0 + BT - 1, T - 1);
    const int my_q = q0 + lq;
    const bool row_ok = my_q < T;
    const size_t qrow = ((size_t)b * a.Hq + hq) * T + (row_ok ? my_q : q0);
    bf16x8 qf[NC], gf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        qf[c] = row_operand(qs + qrow * D, c, lane);
        gf[c] = row_operand((const uint16_t*)a.dout + qrow * D, c, lane);
    }
    const float lse = row_ok ? a.lse[qrow] : kNegInf;
    const float dlt = row_ok ? delta[qrow] : 0.f;
    int seg_q = 0;
    if (row_ok) seg_q = a.seg ? a.seg[(size_t)b * T + my_q] : 1;
    const bool row_vis = row_ok && seg_q > 0 && lse != kNegInf;
    const float nl = row_vis ? -lse * kLog2e : kNegInf;
    const unsigned wlim = window_limit(a.window);

    const TilePlan plan = plan_tiles(q0, q1, a.window, 0, 0, a.prefix != nullptr, BT);
    plan_sink_tiles(plan, a.seg ? a.seg + (size_t)b * T : nullptr, a.prefix ? a.prefix + (size_t)b * T : nullptr, T,
                    q0, q1, BT, sm.red, sm.sink_bits, tid, 256);
    TileIter it;
    it.init(plan, sm.sink_bits, BT);
    const uint16_t* khead = kr + ((size_t)b * a.Hkv + hkv) * (size_t)T * D;
    const uint16_t* vhead = (const uint16_t*)a.v + ((size_t)b * a.Hkv + hkv) * (size_t)T * D;
    f32x16 dqa[D / 32];
#pragma unroll
    for (int n = 0; n < D / 32; ++n) dqa[n] = f32x16{};
    // Staging: thread tid moves piece tid (16 bytes) of the tile's K and V rows
    // and, below 32, key tid's info; the next tile's pieces are loaded into
    // registers while the current tile is computed.
    constexpr int CPR = D / 8;
    const int pr = tid / CPR, pc = tid % CPR;
    const bool mover = tid < 32 * CPR;
    // Unconditional loads from clamped rows, so that no load sits under a
    // branch.  Rows past the end hold copies of the last key, invisible to every
    // query (the mask tests the key index), and their infos are cleared when
    // stored, where the loaded values are needed anyway.
    struct Staged {
        uint4 k, v;
        int sg, sk;
    };
    auto fetch = [&](int k0, Staged& x) {
        const int last = T - k0 - 1;
        const int rr = min(min(pr, BT - 1), last);
        x.k = *(const uint4*)(khead + (size_t)(k0 + rr) * D + 8 * pc);
        x.v = *(const uint4*)(vhead + (size_t)(k0 + rr) * D + 8 * pc);
        const int gk = k0 + min(tid & (BT - 1), last);
        x.sg = a.seg ? a.seg[(size_t)b * T + gk] : 1;
        x.sk = a.prefix ? a.prefix[(size_t)b * T + gk] : 0;
    };
    int kind = 0, tile = 0;
    bool have = it.next(kind, tile);
    Staged cur{make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), 0, 0};
    if (have) fetch(tile * BT, cur);
    while (have) {
        const int k0 = tile * BT;
        int kn = 0, tn = 0;
        const bool have_next = it.next(kn, tn);
        __syncthreads();  // every wave is done with the previous tile
        if (mover) {
            *(uint4*)&sm.k.x[pr * Bf16Tile<D>::RS + 8 * pc] = cur.k;
            *(uint4*)&sm.v.x[pr * Bf16Tile<D>::RS + 8 * pc] = cur.v;
        }
        if (tid < BT) sm.kinfo[tid] = k0 + tid < T ? pack_key_info(cur.sg, cur.sk != 0) : 0;
        __syncthreads();
        if (have_next) fetch(tn * BT, cur);
        tile = tn;
        have = have_next;
        if (!wave_on) continue;
        // S^T = K Q'^T, started from the mask: -lse log2 e where visible, -inf elsewhere
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // keys 8i + 4h + r of the tile (r = 0..3: elements 4i + r), their infos in one read
            const u32x4 inf = lds_load128(lds_off(&sm.kinfo[8 * i + 4 * h]));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kk = 8 * i + 4 * h + r;
                const bool vis = row_vis & (k0 + kk < T) & visible_full(my_q - (k0 + kk), wlim, (int)inf[r], seg_q);
                sacc[4 * i + r] = vis ? nl : kNegInf;
            }
        }
        f32x16 dpa = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_row<D>(sm.k, c, lane), qf[c], sacc, 0, 0, 0);
            dpa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_row<D>(sm.v, c, lane), gf[c], dpa, 0, 0, 0);
        }
        float ds[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) ds[j] = __builtin_amdgcn_exp2f(sacc[j]) * (dpa[j] - dlt);
        bf16x8 db[2];
        pack_steps(ds, db);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int n = 0; n < D / 32; ++n)
                dqa[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_tr<D>(sm.k, m, n, lane), db[m], dqa[n], 0, 0, 0);
    }
    // lane holds query my_q, channels 32n + 8i + 4h + r (element 4i + r of block n)
    // (each lane holds D/2 of the row's channels: blocks n of 16 values)
    float g[D / 2];
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int e = 0; e < 16; ++e) g[16 * n + e] = dqa[n][e] * a.scale;
    if (!row_ok || !wave_on) return;
    // channel of value e: 32 (e / 16) + 8 ((e % 16) / 4) + 4 h + e % 4
    auto chan = [&](int e) { return 32 * (e >> 4) + 8 * ((e & 15) >> 2) + 4 * h + (e & 3); };
    if (a.rope_cos) {
        // back by the negative angle: channel d < D/2 pairs with d + D/2, held by
        // this lane too (D = 64: the other 32-channel block; D = 32: i + 2)
        constexpr int HALF = D / 2;
#pragma unroll
        for (int e = 0; e < D / 2; ++e) {
            const int d = chan(e);
            if (d >= HALF) continue;
            const int e2 = D == 64 ? e + 16 : e + 8;
            const float c = a.rope_cos[(size_t)my_q * HALF + d], sn = a.rope_sin[(size_t)my_q * HALF + d];
            const float x1 = g[e], x2 = g[e2];
            g[e] = x1 * c + x2 * sn;
            g[e2] = x2 * c - x1 * sn;
        }
    }
    float* out = a.dq + qrow * D;
#pragma unroll
    for (int e = 0; e < D / 2; e += 4)
        __builtin_nontemporal_store(f32x4{g[e], g[e + 1], g[e + 2], g[e + 3]}, (f32x4*)(out + chan(e)));
}

template <int D>
struct SmemDkvMfma {
    struct Wave {
        Bf16Tile<D> q, go;
        __attribute__((aligned(16))) float lse2[32];  // lse * log2 e of the tile's queries (-inf: none)
        __attribute__((aligned(16))) float dlt[32];
        __attribute__((aligned(16))) int seg[32];
    } w[4];
    // query tiles past the band holding rows of the block's sink segments
    uint32_t qbits[(kMaxT / BT + 31) / 32];
};

// dk, dv: a workgroup of four waves per 32 keys of one kv head; wave w walks
// the query tiles that can see the keys for the query heads w, w + 4, ... of
// the group (each wave stages its own tiles), and the four waves' sums are
// added in head order at the end.
template <int D>
// (two waves per SIMD: the compiler keeps every value, the next tile's rows
// included, in registers)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkv_mfma_kernel(BwdArgs a, const uint16_t* qs, const uint16_t* kr,
                                                           const float* delta) {
    constexpr int NC = D / 16;
    __shared__ __align__(16) SmemDkvMfma<D> sm;
    const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, h = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    typename SmemDkvMfma<D>::Wave& ws = sm.w[wave];
    const int T = a.T;
    const int b = blockIdx.z, hkv = blockIdx.y;
    const int G = a.Hq / a.Hkv;
    const int s0 = blockIdx.x * BT;
    const int my_k = s0 + lq;
    const bool key_ok = my_k < T;
    const size_t krow = ((size_t)b * a.Hkv + hkv) * T + (key_ok ? my_k : s0);
    bf16x8 kf[NC], vf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        kf[c] = row_operand(kr + krow * D, c, lane);
        vf[c] = row_operand((const uint16_t*)a.v + krow * D, c, lane);
    }
    int seg_k = 0;
    bool sink_k = false;
    if (key_ok) {
        seg_k = a.seg ? a.seg[(size_t)b * T + my_k] : 1;
        sink_k = a.prefix ? a.prefix[(size_t)b * T + my_k] != 0 : false;
    }
    const int info_k = pack_key_info(seg_k, sink_k);
    const unsigned wlim = window_limit(a.window);
    // rows to walk: the band, and with sinks in the block every later row of their segments
    const int s1 = min(s0 + BT - 1, T - 1);
    const int band_end = a.window != 0 ? min(T - 1, s1 + a.window - 1) : T - 1;
    const bool has_sink = a.window != 0 && __ballot(key_ok && sink_k && seg_k > 0) != 0;
    const int sk_lo = wave_imin_xor(key_ok && sink_k && seg_k > 0 ? seg_k : 0x7fffffff, 1, 32);
    const int sk_hi = wave_imax_xor(key_ok && sink_k && seg_k > 0 ? seg_k : (int)0x80000000, 1, 32);
    // Query tiles past the band matter only where one of their rows is in a
    // sink segment of the block: one scan of the rows' segment ids by the
    // whole workgroup (every wave has the same keys, so the same has_sink)
    // marks those tiles in a bit set, eight independent loads per thread at a
    // time.
    const int ntiles = (T + BT - 1) / BT;
    const int tile_end = band_end / BT;  // the band's last tile
    if (has_sink) {
        for (int i = tid; i < (ntiles + 31) / 32; i += 256) sm.qbits[i] = 0u;
        __syncthreads();
        for (int r0 = (tile_end + 1) * BT; r0 < T; r0 += 256 * 8) {
            int sq[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = r0 + 256 * u + tid;
                sq[u] = r < T ? (a.seg ? a.seg[(size_t)b * T + r] : 1) : 0;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = r0 + 256 * u + tid;
                if (r < T && sq[u] >= sk_lo && sq[u] <= sk_hi)
                    atomicOr(&sm.qbits[(r / BT) >> 5], 1u << ((r / BT) & 31));
            }
        }
        __syncthreads();
    }
    // the tile after t0: the next band tile, then the marked tiles in order; -1 at the end
    auto next_tile = [&](int t) -> int {
        if (t + BT <= band_end) return t + BT;
        if (!has_sink) return -1;
        int k = max(t / BT + 1, tile_end + 1);
        while (k < ntiles) {
            const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)sm.qbits[k >> 5]) >> (k & 31);
            if (m != 0u) return (k + __builtin_ctz(m)) * BT;
            k = ((k >> 5) + 1) << 5;
        }
        return -1;
    };
    f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
    for (int n = 0; n < D / 32; ++n) {
        dka[n] = f32x16{};
        dva[n] = f32x16{};
    }
    for (int g = wave; g < G; g += 4) {
        const int hq = hkv * G + g;
        const size_t qhead = ((size_t)b * a.Hq + hq) * (size_t)T;
        // A tile's rows, lse, delta and segment ids are loaded into registers
        // one tile ahead: the next tile's loads are issued as soon as the
        // current tile is in LDS, and land while it is computed.
        TileRows<D> rq, ro;
        float l = 0.f, dlt = 0.f;
        int sgq = 0;
        auto fetch = [&](int t) {
            rq.load(qs + (qhead + t) * D, T - t, lane);
            ro.load((const uint16_t*)a.dout + (qhead + t) * D, T - t, lane);
            // clamped row (the tile's rows past the end are cleared when stored)
            const int tq = min(t + (lane & 31), T - 1);
            l = a.lse[qhead + tq];
            dlt = delta[qhead + tq];
            sgq = a.seg ? a.seg[(size_t)b * T + tq] : 1;
        };
        fetch(s0);
        for (int t0 = s0; t0 >= 0;) {
            // this wave's tiles (its own LDS; its reads of the previous tile are done,
            // LDS accesses of a wave complete in order)
            rq.store(ws.q, lane);
            ro.store(ws.go, lane);
            if (lane < BT) {
                const bool in = t0 + lane < T;
                ws.lse2[lane] = !in || l == kNegInf ? kNegInf : l * kLog2e;
                ws.dlt[lane] = in ? dlt : 0.f;
                ws.seg[lane] = in ? sgq : 0;
            }
            // the tile's rows all exist, are visible to some key and share one
            // segment: tseg is that segment, else 0
            const int sq0 = __builtin_amdgcn_readfirstlane(sgq);
            const int tseg =
                __ballot(lane < BT && (t0 + lane >= T || sgq != sq0 || l == kNegInf)) == 0 && sq0 > 0 ? sq0 : 0;
            const int tn = next_tile(t0);
            if (tn >= 0) fetch(tn);
            lds_reads_done();
            // S = Q' K^T from the mask (element j: query 8 (j / 4) + j % 4 + 4h of the tile)
            f32x16 sacc;
            float dl[16];
            // Whole tile visible to every valid key of the wave (the rows share
            // the key's segment and the key lies inside every row's window).
            const bool full =
                tseg > 0 && __ballot(key_ok && !((info_k & 0x7fffffff) == tseg && t0 >= my_k &&
                                                 (unsigned)(t0 + BT - 1 - my_k) < wlim)) == 0;
            if (full) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x4 l24 = lds_load128(lds_off(&ws.lse2[8 * i + 4 * h]));
                    const u32x4 dl4 = lds_load128(lds_off(&ws.dlt[8 * i + 4 * h]));
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        dl[4 * i + r] = __uint_as_float(dl4[r]);
                        sacc[4 * i + r] = key_ok ? -__uint_as_float(l24[r]) : kNegInf;
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // queries 8i + 4h + r of the tile (elements 4i + r): one read per array
                    const u32x4 sg4 = lds_load128(lds_off(&ws.seg[8 * i + 4 * h]));
                    const u32x4 l24 = lds_load128(lds_off(&ws.lse2[8 * i + 4 * h]));
                    const u32x4 dl4 = lds_load128(lds_off(&ws.dlt[8 * i + 4 * h]));
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int qi = 8 * i + 4 * h + r;
                        const int tq = t0 + qi;
                        const int sq = (int)sg4[r];
                        const float l2 = __uint_as_float(l24[r]);
                        dl[4 * i + r] = __uint_as_float(dl4[r]);
                        const bool vis = key_ok & (tq < T) & (sq > 0) & (l2 != kNegInf) &
                                         visible_full(tq - my_k, wlim, info_k, sq);
                        sacc[4 * i + r] = vis ? -l2 : kNegInf;
                    }
                }
            }
            f32x16 dpa = f32x16{};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_row<D>(ws.q, c, lane), kf[c], sacc, 0, 0, 0);
                dpa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_row<D>(ws.go, c, lane), vf[c], dpa, 0, 0, 0);
            }
            float p[16], ds[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                p[j] = __builtin_amdgcn_exp2f(sacc[j]);
                ds[j] = p[j] * (dpa[j] - dl[j]);
            }
            bf16x8 pb[2], db[2];
            pack_steps(p, pb);
            pack_steps(ds, db);
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < D / 32; ++n) {
                    dva[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_tr<D>(ws.go, m, n, lane), pb[m], dva[n], 0, 0, 0);
                    dka[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_tr<D>(ws.q, m, n, lane), db[m], dka[n], 0, 0, 0);
                }
            t0 = tn;
        }
    }
    // the four waves' sums, added in head order through LDS (the tile space,
    // free once every wave is past its walk): dk first, then dv
    auto chan = [&](int e) { return 32 * (e >> 4) + 8 * ((e & 15) >> 2) + 4 * h + (e & 3); };
    float* red = (float*)&sm;  // [4 waves][32 keys][D] fp32 (4 * 32 * D * 4 bytes fit the tiles)
    static_assert(sizeof(SmemDkvMfma<D>) >= 4 * 32 * D * 4, "reduction space");
    float gk[D / 2], gv[D / 2];  // this lane's half of the key's channels
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        __syncthreads();
#pragma unroll
        for (int n = 0; n < D / 32; ++n)
#pragma unroll
            for (int e = 0; e < 16; e += 4) {
                const f32x16& acc = pass == 0 ? dka[n] : dva[n];
                *(float4*)&red[(wave * 32 + lq) * D + chan(16 * n + e)] = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
            }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int e = 0; e < D / 2; e += 4) {
                float4 sum = *(const float4*)&red[lq * D + chan(e)];
#pragma unroll
                for (int w = 1; w < 4; ++w) {
                    const float4 x = *(const float4*)&red[(w * 32 + lq) * D + chan(e)];
                    sum.x += x.x;
                    sum.y += x.y;
                    sum.z += x.z;
                    sum.w += x.w;
                }
                float* dst = pass == 0 ? gk : gv;
                dst[e] = sum.x;
                dst[e + 1] = sum.y;
                dst[e + 2] = sum.z;
                dst[e + 3] = sum.w;
            }
        }
    }
    if (wave != 0 || !key_ok) return;
#pragma unroll
    for (int e = 0; e < D / 2; ++e) gk[e] *= 0.6931471805599453f;  // dk = dK / log2 e
    if (a.rope_cos) {
        constexpr int HALF = D / 2;
#pragma unroll
        for (int e = 0; e < D / 2; ++e) {
            const int d = chan(e);
            if (d >= HALF) continue;
            const int e2 = D == 64 ? e + 16 : e + 8;
            const float c = a.rope_cos[(size_t)my_k * HALF + d], sn = a.rope_sin[(size_t)my_k * HALF + d];
            const float x1 = gk[e], x2 = gk[e2];
            gk[e] = x1 * c + x2 * sn;
            gk[e2] = x2 * c - x1 * sn;
        }
    }
    float* ok = a.dk + krow * D;
    float* ov = a.dv + krow * D;
#pragma unroll
    for (int e = 0; e < D / 2; e += 4) {
        __builtin_nontemporal_store(f32x4{gk[e], gk[e + 1], gk[e + 2], gk[e + 3]}, (f32x4*)(ok + chan(e)));
        __builtin_nontemporal_store(f32x4{gv[e], gv[e + 1], gv[e + 2], gv[e + 3]}, (f32x4*)(ov + chan(e)));
    }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, const BwdWorkspace& w, hipStream_t s) {
    const dim3 blk(64);
    if (a.dtype == 1) {
        // bf16 operands in the fp32 buffers of the workspace: q' in q32, rotated k in k32
        uint16_t* qs = (uint16_t*)w.q32;
        const uint16_t* kr = (const uint16_t*)a.k;
        const long long nq = (long long)a.B * a.Hq * a.T * (a.D / 16);
        hipLaunchKernelGGL(bwd_prep_bf16_q_kernel, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, s, a, qs, w.delta);
        if (a.rope_cos) {
            const long long nk = (long long)a.B * a.Hkv * a.T * (a.D / 16);
            hipLaunchKernelGGL(bwd_prep_bf16_k_kernel, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, s, a,
                               (uint16_t*)w.k32);
            kr = (const uint16_t*)w.k32;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const unsigned nt = (unsigned)((a.T + BT - 1) / BT);
        const unsigned ngs = (unsigned)((a.Hq / a.Hkv + 3) / 4);
        hipLaunchKernelGGL(bwd_dq_mfma_kernel<D>, dim3(nt, (unsigned)a.Hkv * ngs, (unsigned)a.B), dim3(256), 0, s, a,
                           qs, kr, w.delta);
        hipLaunchKernelGGL(bwd_dkv_mfma_kernel<D>, dim3(nt, (unsigned)a.Hkv, (unsigned)a.B), dim3(256), 0, s, a, qs, kr,
                           w.delta);
        return hipGetLastError();
    }
    const dim3 grid_q((unsigned)a.T, (unsigned)a.Hq, (unsigned)a.B), grid_k((unsigned)a.T, (unsigned)a.Hkv, (unsigned)a.B);
    if (a.dtype == 1) {
        hipLaunchKernelGGL(bwd_prep_q_kernel<uint16_t>, grid_q, blk, 0, s, a, w.q32, w.do32, w.delta);
        hipLaunchKernelGGL(bwd_prep_kv_kernel<uint16_t>, grid_k, blk, 0, s, a, w.k32, w.v32);
    } else {
        hipLaunchKernelGGL(bwd_prep_q_kernel<float>, grid_q, blk, 0, s, a, w.q32, w.do32, w.delta);
        hipLaunchKernelGGL(bwd_prep_kv_kernel<float>, grid_k, blk, 0, s, a, w.k32, w.v32);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned nt = (unsigned)((a.T + BT - 1) / BT);
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(nt, (unsigned)a.Hq, (unsigned)a.B), blk, 0, s, a, w.q32, w.k32, w.v32,
                       w.do32, w.delta);
    hipLaunchKernelGGL(bwd_dkv_kernel<D>, dim3(nt, (unsigned)a.Hq, (unsigned)a.B), blk, 0, s, a, w.q32, w.k32,
                       w.v32, w.do32, w.delta, w.pk, w.pv);
    if (a.Hq != a.Hkv) hipLaunchKernelGGL(bwd_sum_heads_kernel, dim3(2048), dim3(256), 0, s, a, w.pk, w.pv);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_backward(const BwdArgs& a, const BwdWorkspace& w, hipStream_t s) {
    return a.D == 64 ? launch_bwd_d<64>(a, w, s) : launch_bwd_d<32>(a, w, s);
}

}  // namespace swa
