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

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, const BwdWorkspace& w, hipStream_t s) {
    const dim3 blk(64);
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
