// pool_rope.hip -- RoPE tables and block pooling of the compressed variant.
//
// [CA] "Compressed attention and the copy probe", section "Pool before
// rotating, not after": keys are mean-pooled over blocks of b rows BEFORE
// RoPE, values likewise, and each pooled key is then rotated once at its
// block midpoint j*b + b/2 (clamped to the last table row).  Pooled values
// are not rotated.  The rotation is rotate-half over channel pairs
// (i, i + D/2) with angle pos * theta^(-2i/D).
#include "swa_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

__global__ void rope_table_kernel(double theta, int rope_len, int D, float* cos_out, float* sin_out) {
    const int half = D / 2;
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long long)rope_len * half) return;
    const int pos = (int)(idx / half);
    const int i = (int)(idx % half);
    const double inv_freq = pow(theta, -2.0 * (double)i / (double)D);
    const double ang = (double)pos * inv_freq;
    cos_out[idx] = (float)cos(ang);
    sin_out[idx] = (float)sin(ang);
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
    if (BF16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
    return ((const float*)p)[i];
}
template <bool BF16>
__device__ __forceinline__ void store_elem(void* p, size_t i, float v) {
    if (BF16) ((uint16_t*)p)[i] = (uint16_t)f32_to_bf16_bits(v);
    else ((float*)p)[i] = v;
}

// One thread per (row group n, block j, channel pair i): channels i and i+D/2
// of the pooled key and the pooled value.
template <bool BF16>
__global__ void pool_rope_kernel(long long N, int T, int D, int block, int nblk, const void* k, const void* v,
                                 const float* cs, const float* sn, int rope_len, void* pk, void* pv) {
    const int half = D / 2;
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= N * nblk * half) return;
    const int i = (int)(idx % half);
    const long long nj = idx / half;
    const int j = (int)(nj % nblk);
    const long long n = nj / nblk;
    const size_t in_base = ((size_t)n * T + (size_t)j * block) * D;
    float k1 = 0.f, k2 = 0.f, v1 = 0.f, v2 = 0.f;
    for (int r = 0; r < block; ++r) {
        const size_t o = in_base + (size_t)r * D;
        k1 += load_elem<BF16>(k, o + i);
        k2 += load_elem<BF16>(k, o + i + half);
        v1 += load_elem<BF16>(v, o + i);
        v2 += load_elem<BF16>(v, o + i + half);
    }
    const float fb = (float)block;
    k1 /= fb;
    k2 /= fb;
    v1 /= fb;
    v2 /= fb;
    if (cs) {
        int mid = j * block + block / 2;
        if (mid > rope_len - 1) mid = rope_len - 1;
        const float c = cs[(size_t)mid * half + i];
        const float s = sn[(size_t)mid * half + i];
        const float y1 = k1 * c - k2 * s;
        const float y2 = k2 * c + k1 * s;
        k1 = y1;
        k2 = y2;
    }
    const size_t out_base = ((size_t)n * nblk + j) * D;
    store_elem<BF16>(pk, out_base + i, k1);
    store_elem<BF16>(pk, out_base + i + half, k2);
    store_elem<BF16>(pv, out_base + i, v1);
    store_elem<BF16>(pv, out_base + i + half, v2);
}

}  // namespace

hipError_t launch_rope_table(double theta, int rope_len, int D, float* c, float* sn, hipStream_t s) {
    const long long n = (long long)rope_len * (D / 2);
    const int threads = 256;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + threads - 1) / threads)), dim3(threads), 0, s, theta,
                       rope_len, D, c, sn);
    return hipGetLastError();
}

hipError_t launch_pool_rope(int B, int H, int T, int D, int block, int dtype, const void* k_pre, const void* v,
                            const float* c, const float* sn, int rope_len, void* pk, void* pv, hipStream_t s) {
    const int nblk = T / block;
    const long long N = (long long)B * H;
    const long long n = N * nblk * (D / 2);
    const int threads = 256;
    const dim3 grid((unsigned)((n + threads - 1) / threads));
    if (dtype == 1)
        hipLaunchKernelGGL((pool_rope_kernel<true>), grid, dim3(threads), 0, s, N, T, D, block, nblk, k_pre, v, c, sn,
                           rope_len, pk, pv);
    else
        hipLaunchKernelGGL((pool_rope_kernel<false>), grid, dim3(threads), 0, s, N, T, D, block, nblk, k_pre, v, c, sn,
                           rope_len, pk, pv);
    return hipGetLastError();
}

}  // namespace swa
