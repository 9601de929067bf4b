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

constexpr int NT = 32;     // pooled keys per staged tile

template <class X>
__device__ __forceinline__ float ld_f(const X* p, size_t i);
template <>
__device__ __forceinline__ float ld_f<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_f<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

// Exact keys (rotated at their position) and values in fp32: one row per
// 64-lane block, lane d < D holds channel d.
template <class X>
__global__ __launch_bounds__(64) void nsa_prep_rows_kernel(NsaArgs a, float* k32, float* v32) {
    const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x, D = a.D, d = lane % D;
    const size_t row = ((size_t)b * a.Hkv + h) * a.T + t;
    float x = ld_f((const X*)a.k, row * D + d);
    const float vv = ld_f((const X*)a.v, row * D + d);
    if (a.rope_cos) {
        const float other = __shfl_xor(x, D / 2, 64);
        const int i = d % (D / 2);
        const int p = min(t, a.rope_len - 1);
        const float c = a.rope_cos[(size_t)p * (D / 2) + i], s = a.rope_sin[(size_t)p * (D / 2) + i];
        x = d < D / 2 ? x * c - other * s : x * c + other * s;
    }
    if (lane < D) {
        k32[row * D + d] = x;
        v32[row * D + d] = vv;
    }
}

// Pooled keys: the mean of block j's keys before RoPE (rows added in order),
// rotated at min(j b + b/2, rope_len - 1).
template <class X>
__global__ __launch_bounds__(64) void nsa_prep_pooled_kernel(NsaArgs a, float* pk32) {
    const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x, D = a.D, d = lane % D;
    const size_t head = ((size_t)b * a.Hkv + h) * a.T;
    float sum = 0.f;
    for (int u = 0; u < a.block; ++u) sum += ld_f((const X*)a.k, (head + (size_t)j * a.block + u) * D + d);
    float x = sum / (float)a.block;
    if (a.rope_cos) {
        const float other = __shfl_xor(x, D / 2, 64);
        const int i = d % (D / 2);
        const int p = min(j * a.block + a.block / 2, a.rope_len - 1);
        const float c = a.rope_cos[(size_t)p * (D / 2) + i], s = a.rope_sin[(size_t)p * (D / 2) + i];
        x = d < D / 2 ? x * c - other * s : x * c + other * s;
    }
    if (lane < D) pk32[(((size_t)b * a.Hkv + h) * a.nblk + j) * D + d] = x;
}

// kTopK candidates are kept per row: 8, 16 or 32, the smallest that holds n_select.
template <class X, int D, int kTopK>
__global__ __launch_bounds__(64) void nsa_select_kernel(NsaArgs a, const float* k32, const float* v32,
                                                        const float* pk32) {
    __shared__ float tile[NT][D];
    const int lane = threadIdx.x;
    const int T = a.T;
    const int b = blockIdx.z, hq = blockIdx.y;
    const int hkv = hq / (a.Hq / a.Hkv);
    const int t = blockIdx.x * 64 + lane;
    const bool row_ok = t < T;
    const size_t qrow = ((size_t)b * a.Hq + hq) * T + (row_ok ? t : 0);
    float q[D];
#pragma unroll
    for (int d = 0; d < D; ++d) q[d] = row_ok ? ld_f((const X*)a.q, qrow * D + d) : 0.f;
    if (a.rope_cos && row_ok) {
        const int p = min(t, a.rope_len - 1);
#pragma unroll
        for (int i = 0; i < D / 2; ++i) {
            const float c = a.rope_cos[(size_t)p * (D / 2) + i], s = a.rope_sin[(size_t)p * (D / 2) + i];
            const float x1 = q[i], x2 = q[i + D / 2];
            q[i] = x1 * c - x2 * s;
            q[i + D / 2] = x2 * c + x1 * s;
        }
    }
    // candidates: the pooled blocks that have cleared the window
    const int cleared = t - a.window + 1;
    const int n_vis = row_ok && cleared >= a.block ? min(cleared / a.block, a.nblk) : 0;
    int n_max = n_vis;
    for (int o = 1; o < 64; o <<= 1) n_max = max(n_max, __shfl_xor(n_max, o, 64));
    // streaming top-kTopK, best first; a later block replaces only a strictly
    // smaller score, so equal scores keep the lower block first
    float tv[kTopK];
    int ti[kTopK];
#pragma unroll
    for (int i = 0; i < kTopK; ++i) {
        tv[i] = kNegInf;
        ti[i] = -1;
    }
    const float* pkh = pk32 + ((size_t)b * a.Hkv + hkv) * (size_t)a.nblk * D;
    for (int j0 = 0; j0 < n_max; j0 += NT) {
        __syncthreads();
        for (int e = lane; e < NT * D; e += 64) {
            const int jj = j0 + e / D;
            tile[e / D][e % D] = jj < a.nblk ? pkh[(size_t)jj * D + e % D] : 0.f;
        }
        __syncthreads();
#pragma unroll 1
        for (int u = 0; u < NT; ++u) {
            const int j = j0 + u;
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) dot = fmaf(q[d], tile[u][d], dot);
            float s = dot * a.scale;
            if (j < n_vis && s > tv[kTopK - 1]) {
                int id = j;
#pragma unroll
                for (int i = 0; i < kTopK; ++i) {
                    if (s > tv[i]) {
                        const float fs = tv[i];
                        const int is = ti[i];
                        tv[i] = s;
                        ti[i] = id;
                        s = fs;
                        id = is;
                    }
                }
            }
        }
    }
    // attention over the chosen blocks' exact tokens (online softmax)
    const float* kh = k32 + ((size_t)b * a.Hkv + hkv) * (size_t)T * D;
    const float* vh = v32 + ((size_t)b * a.Hkv + hkv) * (size_t)T * D;
    float m = kNegInf, l = 0.f, o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = 0.f;
#pragma unroll
    for (int i = 0; i < kTopK; ++i) {
        if (i >= a.n_select || ti[i] < 0) continue;
        for (int u = 0; u < a.block; ++u) {
            const size_t r = (size_t)ti[i] * a.block + u;
            const float4* kr = (const float4*)(kh + r * D);
            float dot = 0.f;
#pragma unroll
            for (int d4 = 0; d4 < D / 4; ++d4) {
                const float4 kk = kr[d4];
                dot = fmaf(q[4 * d4], kk.x, dot);
                dot = fmaf(q[4 * d4 + 1], kk.y, dot);
                dot = fmaf(q[4 * d4 + 2], kk.z, dot);
                dot = fmaf(q[4 * d4 + 3], kk.w, dot);
            }
            const float s = dot * a.scale;
            if (s > m) {
                const float corr = expf(m - s);
                m = s;
                l *= corr;
#pragma unroll
                for (int d = 0; d < D; ++d) o[d] *= corr;
            }
            const float p = expf(s - m);
            l += p;
            const float4* vr = (const float4*)(vh + r * D);
#pragma unroll
            for (int d4 = 0; d4 < D / 4; ++d4) {
                const float4 vv = vr[d4];
                o[4 * d4] = fmaf(p, vv.x, o[4 * d4]);
                o[4 * d4 + 1] = fmaf(p, vv.y, o[4 * d4 + 1]);
                o[4 * d4 + 2] = fmaf(p, vv.z, o[4 * d4 + 2]);
                o[4 * d4 + 3] = fmaf(p, vv.w, o[4 * d4 + 3]);
            }
        }
    }
    if (!row_ok) return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (a.dtype == 1) {
        uint16_t* orow = (uint16_t*)a.out + qrow * D;
#pragma unroll
        for (int d = 0; d < D; ++d) orow[d] = (uint16_t)f32_to_bf16_bits(o[d] * inv);
    } else {
        float* orow = (float*)a.out + qrow * D;
#pragma unroll
        for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
    }
    if (a.lse) a.lse[qrow] = l > 0.f ? m + logf(l) : kNegInf;
    if (a.sel) {
#pragma unroll
        for (int i = 0; i < kTopK; ++i)
            if (i < a.n_select) a.sel[qrow * a.n_select + i] = ti[i];
    }
}

template <class X>
hipError_t launch_nsa_t(const NsaArgs& a, float* k32, float* v32, float* pk32, hipStream_t s) {
    const dim3 blk(64);
    hipLaunchKernelGGL(nsa_prep_rows_kernel<X>, dim3((unsigned)a.T, (unsigned)a.Hkv, (unsigned)a.B), blk, 0, s, a,
                       k32, v32);
    if (a.nblk > 0)
        hipLaunchKernelGGL(nsa_prep_pooled_kernel<X>, dim3((unsigned)a.nblk, (unsigned)a.Hkv, (unsigned)a.B), blk, 0,
                           s, a, pk32);
    const dim3 grid((unsigned)((a.T + 63) / 64), (unsigned)a.Hq, (unsigned)a.B);
#define SWA_NSA(DD, KK) hipLaunchKernelGGL((nsa_select_kernel<X, DD, KK>), grid, blk, 0, s, a, k32, v32, pk32)
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

hipError_t launch_nsa_select(const NsaArgs& a, float* k32, float* v32, float* pk32, hipStream_t s) {
    return a.dtype == 1 ? launch_nsa_t<uint16_t>(a, k32, v32, pk32, s) : launch_nsa_t<float>(a, k32, v32, pk32, s);
}

}  // namespace swa
