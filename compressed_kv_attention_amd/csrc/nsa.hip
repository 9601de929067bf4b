// nsa.hip -- the selection branch of NSA, without its learned gate.
//
// [CA] "Compressed attention and the copy probe", section "Two kinds of
// columns, pooled blocks and exact recent keys", names the three branches of
// DeepSeek's Native Sparse Attention: the compressed branch (mean-pooled
// blocks), the selected branch (the top-k blocks by their compressed scores)
// and the window, mixed by a learned gate; section "What we didn't build, and
// why" leaves selection and the gate out.  This file builds the selected
// branch on the compressed variant's columns: for row t the candidates are
// the pooled blocks that have cleared the window ((j + 1) b <= t - W + 1);
// block j's score is scale <q_t, pk_j> (pk_j = mean of the block's keys before
// RoPE, rotated at its midpoint, [CA] "Pool before rotating, not after"); the
// n best blocks (the lower j on ties) are kept and one softmax runs over the
// exact keys, rotated at their positions, of all their tokens.
//
// Everything is fp32.  A preparation pass rotates the exact keys and forms the
// pooled keys; the main kernel gives each query row a lane: the row's rotated
// q in registers, a streaming top-k (8, 16 or 32 kept) of the scores of the candidate blocks
// (staged through LDS 32 blocks at a time), then attention over the chosen
// blocks' tokens, read straight from the fp32 key and value rows.
#include "swa_common.h"
#include "swa_internal.h"

namespace swa {
namespace {


template <class X>
__device__ __forceinline__ float ld_f(const X* p, size_t i);
template <>
__device__ __forceinline__ float ld_f<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_f<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

__device__ __forceinline__ void lds_store64(uint32_t addr, u32x2 v) {
#if defined(__HIP_DEVICE_COMPILE__)
    *__builtin_bit_cast(__attribute__((address_space(3))) u32x2*, addr) = v;
#else
    (void)addr;
    (void)v;
#endif
}

template <class X>
__device__ __forceinline__ void st_x(X* p, float v);
template <>
__device__ __forceinline__ void st_x<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void st_x<uint16_t>(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16_bits(v); }

// Eight consecutive elements (16-byte aligned) in fp32, and back in the
// element type (bf16 rounded to nearest even, as st_x does).
__device__ __forceinline__ void ld8(const float* p, float (&x)[8]) {
    const float4 u = ((const float4*)p)[0], v = ((const float4*)p)[1];
    x[0] = u.x, x[1] = u.y, x[2] = u.z, x[3] = u.w, x[4] = v.x, x[5] = v.y, x[6] = v.z, x[7] = v.w;
}
__device__ __forceinline__ void ld8(const uint16_t* p, float (&x)[8]) {
    const uint4 v = *(const uint4*)p;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}
__device__ __forceinline__ void st8(float* p, const float (&x)[8]) {
    ((float4*)p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    ((float4*)p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void st8(uint16_t* p, const float (&x)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = f32_to_bf16_bits(x[2 * e]) | (f32_to_bf16_bits(x[2 * e + 1]) << 16);
    *(uint4*)p = make_uint4(w[0], w[1], w[2], w[3]);
}

// Exact keys rotated at their position, in the input dtype (bf16 keys are
// rounded once after the fp32 rotation, as the key pre-pass of a prefill
// does): one thread per (row, 8 channel pairs).
template <class X>
__global__ __launch_bounds__(256) void nsa_rotate_keys_kernel(NsaArgs a, X* kr) {
    const int D = a.D, half = D / 2, per_row = half / 8;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long rows = (long long)a.B * a.Hkv * a.T;
    if (idx >= rows * per_row) return;
    const long long row = idx / per_row;
    const int i0 = (int)(idx - row * per_row) * 8;
    const int t = (int)(row % a.T);
    const int p = min(t, a.rope_len - 1);
    const X* src = (const X*)a.k + row * D;
    X* dst = kr + row * D;
    // 16-byte accesses: the 8 channels of each half and their table entries
    float x1[8], x2[8], c[8], sn[8];
    ld8(src + i0, x1);
    ld8(src + half + i0, x2);
    ld8(a.rope_cos + (size_t)p * half + i0, c);
    ld8(a.rope_sin + (size_t)p * half + i0, sn);
    float y1[8], y2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        y1[e] = x1[e] * c[e] - x2[e] * sn[e];
        y2[e] = x2[e] * c[e] + x1[e] * sn[e];
    }
    st8(dst + i0, y1);
    st8(dst + half + i0, y2);
}

// Half a row (channels [0, H) from p) in fp32.
template <int H>
__device__ __forceinline__ void load_half(const float* p, float (&x)[H]) {
#pragma unroll
    for (int i = 0; i < H / 4; ++i) {
        const float4 v = ((const float4*)p)[i];
        x[4 * i] = v.x;
        x[4 * i + 1] = v.y;
        x[4 * i + 2] = v.z;
        x[4 * i + 3] = v.w;
    }
}
template <int H>
__device__ __forceinline__ void load_half(const uint16_t* p, float (&x)[H]) {
#pragma unroll
    for (int i = 0; i < H / 8; ++i) {
        const uint4 v = ((const uint4*)p)[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[8 * i + 2 * e] = __uint_as_float(w[e] << 16);
            x[8 * i + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }
}

// Half a row as loaded (16-byte pieces), converted to fp32 where it is used.
template <class X, int H>
struct HalfRow;
template <int H>
struct HalfRow<float, H> {
    float4 v[H / 4];
    __device__ __forceinline__ void load(const float* p) {
#pragma unroll
        for (int i = 0; i < H / 4; ++i) v[i] = ((const float4*)p)[i];
    }
    __device__ __forceinline__ void to(float (&x)[H]) const {
#pragma unroll
        for (int i = 0; i < H / 4; ++i) {
            x[4 * i] = v[i].x;
            x[4 * i + 1] = v[i].y;
            x[4 * i + 2] = v[i].z;
            x[4 * i + 3] = v[i].w;
        }
    }
};
template <int H>
struct HalfRow<uint16_t, H> {
    uint4 v[H / 8];
    __device__ __forceinline__ void load(const uint16_t* p) {
#pragma unroll
        for (int i = 0; i < H / 8; ++i) v[i] = ((const uint4*)p)[i];
    }
    __device__ __forceinline__ void to(float (&x)[H]) const {
#pragma unroll
        for (int i = 0; i < H / 8; ++i) {
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[8 * i + 2 * e] = __uint_as_float(w[e] << 16);
                x[8 * i + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
            }
        }
    }
};

// Pooled keys: the mean of block j's keys before RoPE (rows added in order),
// rotated at min(j b + b/2, rope_len - 1).
template <class X>
__global__ __launch_bounds__(256) void nsa_prep_pooled_kernel(NsaArgs a, float* pk32) {
    // one thread per (pooled key, 8 channel pairs): channels i0 .. i0 + 7 and
    // their rotate-half partners, 16 bytes per access
    const int D = a.D, half = D / 2, per = half / 8;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total = (long long)a.B * a.Hkv * a.nblk * per;
    if (idx >= total) return;
    const long long key = idx / per;  // ((b * Hkv + h) * nblk + j)
    const int i0 = (int)(idx - key * per) * 8;
    const long long n = key / a.nblk;
    const int j = (int)(key - n * a.nblk);
    const X* src = (const X*)a.k + ((size_t)n * a.T + (size_t)j * a.block) * D;
    float s1[8], s2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s1[e] = s2[e] = 0.f;
#pragma unroll 4
    for (int u = 0; u < a.block; ++u) {  // rows added in order
        float x1[8], x2[8];
        ld8(src + (size_t)u * D + i0, x1);
        ld8(src + (size_t)u * D + half + i0, x2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s1[e] += x1[e];
            s2[e] += x2[e];
        }
    }
    float y1[8], y2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        y1[e] = s1[e] / (float)a.block;
        y2[e] = s2[e] / (float)a.block;
    }
    if (a.rope_cos) {
        const int p = min(j * a.block + a.block / 2, a.rope_len - 1);
        float c[8], sn[8];
        ld8(a.rope_cos + (size_t)p * half + i0, c);
        ld8(a.rope_sin + (size_t)p * half + i0, sn);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float r1 = y1[e] * c[e] - y2[e] * sn[e];
            const float r2 = y2[e] * c[e] + y1[e] * sn[e];
            y1[e] = r1;
            y2[e] = r2;
        }
    }
    st8(pk32 + key * D + i0, y1);
    st8(pk32 + key * D + half + i0, y2);
}

// One wave per 32 query rows of one head; lanes n and n + 32 share row n.
// The compressed scores of 32 pooled keys at a time come from fp32 matrix
// instructions (S^T = PK Q^T, v_mfma_f32_32x32x2_f32: lane (n, h) supplies
// channels 2i + h of row n's rotated q and of pooled key n); lane (n, h) then
// holds the scores of row n on keys 8r + 4h + {0..3}, r = 0..3, and keeps the
// best kTopK of its own candidates (candidates arrive in increasing order; a
// later one replaces only a strictly smaller score, so ties keep the lower
// block).  The two lanes of a row merge their lists (ties to the lower block)
// and attend together over the chosen blocks' tokens, each over half of the
// channels.  kTopK is 8, 16 or 32, the smallest that holds n_select.
template <class X, int D>
__device__ __forceinline__ void load_q_rotated(const NsaArgs& a, size_t qrow, int t, bool row_ok, float (&q)[D]) {
    constexpr int H = D / 2;
    if (!row_ok) {
#pragma unroll
        for (int d = 0; d < D; ++d) q[d] = 0.f;
        return;
    }
    load_half<H>((const X*)a.q + qrow * D, *(float(*)[H])&q[0]);
    load_half<H>((const X*)a.q + qrow * D + H, *(float(*)[H])&q[H]);
    if (a.rope_cos) {
        const int p = min(t, a.rope_len - 1);
        float c[H], sn[H];
        load_half<H>(a.rope_cos + (size_t)p * H, c);
        load_half<H>(a.rope_sin + (size_t)p * H, sn);
#pragma unroll
        for (int i = 0; i < H; ++i) {
            const float x1 = q[i], x2 = q[i + H];
            q[i] = x1 * c[i] - x2 * sn[i];
            q[i + H] = x2 * c[i] + x1 * sn[i];
        }
    }
}

template <class X, int D, int kTopK>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void nsa_select_kernel(NsaArgs a, const X* krot, const float* pk32) {
    constexpr int H = D / 2;   // channels per lane of a row pair
    constexpr int RS = D + 4;  // LDS row stride of the staged pooled keys (floats)
    __shared__ __align__(16) float tile[32 * RS];
    __shared__ float sc[64 * 17];  // each lane's 16 scores of the current tile
    const int lane = threadIdx.x, n = lane & 31, kk = lane >> 5;
    const int T = a.T;
    // XCD-aware numbering: dispatch sends workgroup i to XCD i % 8; each XCD
    // takes a contiguous range of (row block fastest, head, batch row), so the
    // rows one head gathers stay in that XCD's L2
    const int nrb = (T + 31) / 32;
    const long long nwg = (long long)nrb * a.Hq * a.B;
    long long lb = blockIdx.x;
    if ((nwg & 7) == 0) lb = (long long)(blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int rb = (int)(lb % nrb);
    const int hq = (int)((lb / nrb) % a.Hq);
    const int b = (int)(lb / ((long long)nrb * a.Hq));
    const int hkv = hq / (a.Hq / a.Hkv);
    const int t = rb * 32 + n;
    const bool row_ok = t < T;
    const size_t qrow = ((size_t)b * a.Hq + hq) * T + (row_ok ? t : 0);
    // the matrix operand: channels 2i + kk of row n's rotated q
    // and, for the attention over the chosen tokens, channels [H kk, H kk + H)
    // (kept from here when the lists are short, else loaded again then)
    constexpr bool kKeepQA = kTopK <= 16;
    float qB[H], qA[H];
    {
        float q[D];
        load_q_rotated<X, D>(a, qrow, t, row_ok, q);
#pragma unroll
        for (int i = 0; i < H; ++i) {
            qB[i] = kk ? q[2 * i + 1] : q[2 * i];
            if (kKeepQA) qA[i] = kk ? q[H + i] : q[i];
        }
    }
    // candidates: the pooled blocks that have cleared the window
    const int cleared = t - a.window + 1;
    const int n_vis = row_ok && cleared >= a.block ? min(cleared / a.block, a.nblk) : 0;
    int n_max = n_vis;
    for (int o = 1; o < 64; o <<= 1) n_max = max(n_max, __shfl_xor(n_max, o, 64));
    float tv[kTopK];
    int ti[kTopK];
#pragma unroll
    for (int i = 0; i < kTopK; ++i) {
        tv[i] = kNegInf;
        ti[i] = -1;
    }
    const float* pkh = pk32 + ((size_t)b * a.Hkv + hkv) * (size_t)a.nblk * D;
    const uint32_t tl = lds_off(tile);
    // Pooled keys j0 .. j0 + 31, lane (m, kk) loading channels [H kk, H kk + H)
    // of key m: every load from a clamped address, the values selected when
    // stored; the next tile's loads are issued as soon as the current tile is
    // in LDS, and land while it is scored and inserted.
    float4 xs[H / 4];
    auto fetch = [&](int j) {
        const float* src = pkh + (size_t)min(j + n, a.nblk - 1) * D + H * kk;
#pragma unroll
        for (int c4 = 0; c4 < H / 4; ++c4) xs[c4] = *(const float4*)(src + 4 * c4);
    };
    if (n_max > 0) fetch(0);
    for (int j0 = 0; j0 < n_max; j0 += 32) {
        // stage pooled keys j0 .. j0 + 31, split by channel parity (row m
        // holds the even channels, then the odd ones)
        {
            const int jj = j0 + n;
#pragma unroll
            for (int c4 = 0; c4 < H / 4; ++c4) {
                const float4 x = jj < a.nblk ? xs[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
                const int c = H * kk + 4 * c4;  // even
                lds_store64(tl + (uint32_t)(n * RS + c / 2) * 4u, u32x2{__float_as_uint(x.x), __float_as_uint(x.z)});
                lds_store64(tl + (uint32_t)(n * RS + H + c / 2) * 4u, u32x2{__float_as_uint(x.y), __float_as_uint(x.w)});
            }
        }
        if (j0 + 32 < n_max) fetch(j0 + 32);
        lds_reads_done();  // (LDS writes and reads of the wave complete in order; the wait also covers the writes)
        f32x16 acc{};
#pragma unroll
        for (int i4 = 0; i4 < H / 4; ++i4) {
            const u32x4 av = lds_load128(tl + (uint32_t)(n * RS + kk * H + 4 * i4) * 4u);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av[e]), qB[4 * i4 + e], acc, 0, 0, 0);
        }
        lds_reads_done();  // the tile is reread only after these reads
        if (j0 == 0) {
            // The first tile: the list is empty, so it is this lane's 16
            // candidates sorted (best first: larger score, or lower block on
            // equal scores) by a bitonic network, cut to k.
            float cv[16];
            int ci[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int jj = 8 * (j >> 2) + 4 * kk + (j & 3);
                const bool ok = jj < n_vis;
                cv[j] = ok ? acc[j] * a.scale : kNegInf;
                ci[j] = ok ? jj : -1;
            }
            auto better = [](float va, int ia, float vb, int ib) {
                return va > vb || (va == vb && (unsigned)ia < (unsigned)ib);
            };
#pragma unroll
            for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
                for (int st = k >> 1; st > 0; st >>= 1)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int l = i ^ st;
                        if (l <= i) continue;
                        // best first within blocks of k whose bit k is clear, worst first otherwise
                        const bool sw = (i & k) == 0 ? better(cv[l], ci[l], cv[i], ci[i])
                                                     : better(cv[i], ci[i], cv[l], ci[l]);
                        const float fv = cv[i];
                        const int fi = ci[i];
                        cv[i] = sw ? cv[l] : fv;
                        ci[i] = sw ? ci[l] : fi;
                        cv[l] = sw ? fv : cv[l];
                        ci[l] = sw ? fi : ci[l];
                    }
#pragma unroll
            for (int i = 0; i < (kTopK < 16 ? kTopK : 16); ++i) {
                tv[i] = cv[i];
                ti[i] = ci[i];
            }
            continue;
        }
        // This lane's candidates above its current threshold, as a bit mask;
        // their scores wait in LDS.  The lanes then insert together, each its
        // next candidate in increasing order, as long as any lane has one:
        // the insertion runs as often as the busiest lane needs, not once
        // for every candidate some lane takes.
        // The row's k-th best score is at least this lane's and its partner's
        // k-th best, and at least the smaller of their (k/2)-th best (together
        // they hold k scores at or above it): a candidate below that bound is
        // not among the row's k best and is not inserted (equal ones are).
        const float own_k = tv[kTopK - 1], own_h = tv[kTopK / 2 - 1];
        const float par_k = __shfl_xor(own_k, 32, 64), par_h = __shfl_xor(own_h, 32, 64);
        const float bound = fmaxf(fmaxf(own_k, par_k), fminf(own_h, par_h));
        uint32_t want = 0u;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float s = acc[j] * a.scale;
            const int jj = j0 + 8 * (j >> 2) + 4 * kk + (j & 3);
            sc[lane * 17 + j] = s;
            if (jj < n_vis && s > own_k && s >= bound) want |= 1u << j;
        }
        // Two candidates per pass, in increasing order: the second moves one
        // list place behind the first, which is the same as inserting them one
        // after the other (the second's step at place i follows the first's
        // step there and no later one of the first touches place i), with
        // half the passes and two independent chains of compare-and-swap.
        while (__builtin_amdgcn_ballot_w64(want != 0u) != 0) {
            float s1 = kNegInf, s2 = kNegInf;
            int id1 = -1, id2 = -1;
            if (want != 0u) {
                const int j = __builtin_ctz(want);
                want &= want - 1u;
                s1 = sc[lane * 17 + j];
                id1 = j0 + 8 * (j >> 2) + 4 * kk + (j & 3);
            }
            if (want != 0u) {
                const int j = __builtin_ctz(want);
                want &= want - 1u;
                s2 = sc[lane * 17 + j];
                id2 = j0 + 8 * (j >> 2) + 4 * kk + (j & 3);
            }
            // (no lane's pair reaches its list: the pass is skipped)
            if (__builtin_amdgcn_ballot_w64(s1 > tv[kTopK - 1] || s2 > tv[kTopK - 1]) == 0) continue;
            // (compare-and-swap by selects: no branch per place)
#pragma unroll
            for (int i = 0; i < kTopK; ++i) {
                const bool g1 = s1 > tv[i];
                const float v1 = tv[i];
                const int i1 = ti[i];
                tv[i] = g1 ? s1 : v1;
                ti[i] = g1 ? id1 : i1;
                s1 = g1 ? v1 : s1;
                id1 = g1 ? i1 : id1;
                const bool g2 = s2 > tv[i];
                const float v2 = tv[i];
                const int i2 = ti[i];
                tv[i] = g2 ? s2 : v2;
                ti[i] = g2 ? id2 : i2;
                s2 = g2 ? v2 : s2;
                id2 = g2 ? i2 : id2;
            }
        }
    }
    // Merge the two lists of the row (both lanes compute it): the better of
    // entry i of the kk = 0 list and entry K-1-i of the kk = 1 list, for every
    // i, is the top K as a bitonic sequence, then sorted by a bitonic network.
    // Better: the larger score, or the lower block on equal scores.
    {
        float ov[kTopK];
        int oi[kTopK];
#pragma unroll
        for (int i = 0; i < kTopK; ++i) {
            ov[i] = __shfl_xor(tv[i], 32, 64);
            oi[i] = __shfl_xor(ti[i], 32, 64);
        }
        auto better = [](float va, int ia, float vb, int ib) {
            return va > vb || (va == vb && (unsigned)ia < (unsigned)ib);
        };
        // (list A: the kk = 0 lane's, list B: the kk = 1 lane's; both lanes read
        // them from copies, since the merge overwrites tv / ti)
        float av[kTopK], bv[kTopK];
        int ai[kTopK], bi[kTopK];
#pragma unroll
        for (int i = 0; i < kTopK; ++i) {
            av[i] = kk ? ov[i] : tv[i];
            ai[i] = kk ? oi[i] : ti[i];
            bv[i] = kk ? tv[i] : ov[i];
            bi[i] = kk ? ti[i] : oi[i];
        }
#pragma unroll
        for (int i = 0; i < kTopK; ++i) {
            const bool first = better(av[i], ai[i], bv[kTopK - 1 - i], bi[kTopK - 1 - i]);
            tv[i] = first ? av[i] : bv[kTopK - 1 - i];
            ti[i] = first ? ai[i] : bi[kTopK - 1 - i];
        }
#pragma unroll
        for (int st = kTopK / 2; st >= 1; st >>= 1) {
#pragma unroll
            for (int i = 0; i < kTopK; ++i) {
                if (i & st) continue;
                const bool keep = !better(tv[i + st], ti[i + st], tv[i], ti[i]);
                const float va = tv[i], vb = tv[i + st];
                const int ia = ti[i], ib = ti[i + st];
                tv[i] = keep ? va : vb;
                ti[i] = keep ? ia : ib;
                tv[i + st] = keep ? vb : va;
                ti[i + st] = keep ? ib : ia;
            }
        }
    }
    // attention over the chosen blocks' exact tokens (online softmax); lane
    // (n, kk) holds channels [H kk, H kk + H) of row n
    if (!kKeepQA) {
        float q[D];
        load_q_rotated<X, D>(a, qrow, t, row_ok, q);
#pragma unroll
        for (int i = 0; i < H; ++i) qA[i] = kk ? q[H + i] : q[i];
    }
    const X* kh = krot + ((size_t)b * a.Hkv + hkv) * (size_t)T * D + H * kk;
    const X* vh = (const X*)a.v + ((size_t)b * a.Hkv + hkv) * (size_t)T * D + H * kk;
    float m = kNegInf, l = 0.f, o[H];
#pragma unroll
    for (int d = 0; d < H; ++d) o[d] = 0.f;
    // The chosen tokens in list order, each token's K and V half rows loaded
    // while the previous token is used.  Every lane walks the list to the
    // longest one in the wave (an entry a lane does not have reads a valid row
    // and weighs nothing), so no load sits under a divergent branch.
    const int nsel = min(a.n_select, kTopK);
    HalfRow<X, H> nk, nv;
    {
        const size_t r0 = (size_t)(nsel > 0 && ti[0] >= 0 ? ti[0] : 0) * a.block;
        nk.load(kh + r0 * D);
        nv.load(vh + r0 * D);
    }
#pragma unroll
    for (int i = 0; i < kTopK; ++i) {
        // (lists hold their valid entries first)
        if (i >= nsel || __builtin_amdgcn_ballot_w64(ti[i] >= 0) == 0) break;
        const bool vi = ti[i] >= 0;
        const int bi = vi ? ti[i] : 0;
        const int bn = (i + 1 < kTopK && i + 1 < nsel && ti[i + 1 < kTopK ? i + 1 : i] >= 0) ? ti[i + 1 < kTopK ? i + 1 : i] : 0;
        for (int u = 0; u < a.block; ++u) {
            const HalfRow<X, H> ck = nk, cv = nv;
            const size_t rn = u + 1 < a.block ? (size_t)bi * a.block + u + 1 : (size_t)bn * a.block;
            nk.load(kh + rn * D);
            nv.load(vh + rn * D);
            float kx[H], vx[H];
            ck.to(kx);
            cv.to(vx);
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < H; ++d) dot = fmaf(qA[d], kx[d], dot);
            const float other = __shfl_xor(dot, 32, 64);
            const float s = vi ? (kk ? other + dot : dot + other) * a.scale : kNegInf;
            if (s > m) {
                const float corr = expf(m - s);
                m = s;
                l *= corr;
#pragma unroll
                for (int d = 0; d < H; ++d) o[d] *= corr;
            }
            const float p = vi ? expf(s - m) : 0.f;
            l += p;
#pragma unroll
            for (int d = 0; d < H; ++d) o[d] = fmaf(p, vx[d], o[d]);
        }
    }
    if (!row_ok) return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (a.dtype == 1) {
        uint16_t* orow = (uint16_t*)a.out + qrow * D + H * kk;
#pragma unroll
        for (int d = 0; d < H; ++d) orow[d] = (uint16_t)f32_to_bf16_bits(o[d] * inv);
    } else {
        float* orow = (float*)a.out + qrow * D + H * kk;
#pragma unroll
        for (int d = 0; d < H; ++d) orow[d] = o[d] * inv;
    }
    if (kk == 0) {
        if (a.lse) a.lse[qrow] = l > 0.f ? m + logf(l) : kNegInf;
        if (a.sel) {
#pragma unroll
            for (int i = 0; i < kTopK; ++i)
                if (i < a.n_select) a.sel[qrow * a.n_select + i] = ti[i];
        }
    }
}

template <class X>
hipError_t launch_nsa_t(const NsaArgs& a, void* krot_ws, float* pk32, hipStream_t s) {
    const X* krot = (const X*)a.k;  // without RoPE the keys are read as given
    if (a.rope_cos) {
        const long long n = (long long)a.B * a.Hkv * a.T * (a.D / 16);
        hipLaunchKernelGGL(nsa_rotate_keys_kernel<X>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a,
                           (X*)krot_ws);
        krot = (const X*)krot_ws;
    }
    if (a.nblk > 0) {
        const long long n = (long long)a.B * a.Hkv * a.nblk * (a.D / 16);
        hipLaunchKernelGGL(nsa_prep_pooled_kernel<X>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, pk32);
    }
    const long long nwg = (long long)((a.T + 31) / 32) * a.Hq * a.B;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nwg), blk(64);
#define SWA_NSA(DD, KK) hipLaunchKernelGGL((nsa_select_kernel<X, DD, KK>), grid, blk, 0, s, a, krot, pk32)
    if (a.D == 64) {
        if (a.n_select <= 8) SWA_NSA(64, 8);
        else if (a.n_select <= 16) SWA_NSA(64, 16);
        else SWA_NSA(64, 32);
    } else {
        if (a.n_select <= 8) SWA_NSA(32, 8);
        else if (a.n_select <= 16) SWA_NSA(32, 16);
        else SWA_NSA(32, 32);
    }
#undef SWA_NSA
    return hipGetLastError();
}

}  // namespace

hipError_t launch_nsa_select(const NsaArgs& a, void* krot, float* pk32, hipStream_t s) {
    return a.dtype == 1 ? launch_nsa_t<uint16_t>(a, krot, pk32, s) : launch_nsa_t<float>(a, krot, pk32, s);
}

}  // namespace swa
