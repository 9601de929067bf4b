// pool_rope.hip -- the pre-passes of a prefill: RoPE tables, key rotation,
// block pooling of the compressed variant and the per-key mask metadata.
//
// [CA] "Compressed attention and the copy probe", section "Pool before
// rotating, not after": keys are mean-pooled over blocks of b rows BEFORE
// RoPE, values likewise, and each pooled key is then rotated once at its
// block midpoint j*b + b/2 (clamped to the last table row).  Pooled values
// are not rotated.  The rotation is rotate-half over channel pairs
// (i, i + D/2) with angle pos * theta^(-2i/D).
#include "swa_common.h"
#include "swa_internal.h"
#include "swa_tiles.h"

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

// Mean of b values: the fp32 sum divided by b, or multiplied by 1/b when b is
// a power of two (then the same value).
__device__ __forceinline__ void scale_by_block(float* x, int n, int block, float inv_b) {
    if (inv_b != 0.f) {
        for (int e = 0; e < n; ++e) x[e] *= inv_b;
    } else {
        const float fb = (float)block;
        for (int e = 0; e < n; ++e) x[e] /= fb;
    }
}
inline float pow2_reciprocal(int block) { return (block & (block - 1)) == 0 ? 1.0f / (float)block : 0.f; }

// Pooling with 16-byte accesses: one thread per (block j, tensor K or V,
// piece c of CH channel pairs) of a row group n: channels i0 .. i0+CH-1 and
// their rotate-half partners i0 + D/2 .. of the pooled key (rotated) or
// value.  Grid x covers one row group's pieces (the first half pools K, the
// second V), grid y the row groups.  The same arithmetic, in the same order
// per element, as the element-wise kernel below.
template <bool BF16>
__global__ __launch_bounds__(256) void pool_rope_vec_kernel(int N, int T, int D, int block, int nblk, FastDiv div_pr,
                                                            float inv_b, const void* k, const void* v, const float* cs,
                                                            const float* sn, int rope_len, void* pk, void* pv) {
    constexpr int CH = BF16 ? 8 : 4;  // elements per 16-byte piece
    constexpr int ES = BF16 ? 2 : 4;  // bytes per element
    const int half = D / 2;
    const int per_row = (int)div_pr.d;  // pieces per half row
    const uint32_t per_tensor = (uint32_t)nblk * (uint32_t)per_row;
    const uint32_t idx = blockIdx.x * 256u + threadIdx.x;
    if (idx >= 2 * per_tensor) return;
    const bool is_k = idx < per_tensor;
    const uint32_t r = is_k ? idx : idx - per_tensor;
    const int j = (int)fdiv(r, div_pr);
    const int c = (int)r - j * per_row;
    const int i0 = c * CH;
    for (int n = blockIdx.y; n < N; n += gridDim.y) {
        const char* src = (const char*)(is_k ? k : v) + (((size_t)n * T + (size_t)j * block) * D + i0) * ES;
        float x1[CH], x2[CH];
#pragma unroll
        for (int e = 0; e < CH; ++e) x1[e] = x2[e] = 0.f;
#pragma unroll 4
        for (int rr = 0; rr < block; ++rr) {
            const uint4 a = *(const uint4*)(src + (size_t)rr * D * ES);
            const uint4 b = *(const uint4*)(src + ((size_t)rr * D + half) * ES);
            const uint32_t ua[4] = {a.x, a.y, a.z, a.w}, ub[4] = {b.x, b.y, b.z, b.w};
            if constexpr (BF16) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x1[2 * i] += __uint_as_float(ua[i] << 16);
                    x1[2 * i + 1] += __uint_as_float(ua[i] & 0xffff0000u);
                    x2[2 * i] += __uint_as_float(ub[i] << 16);
                    x2[2 * i + 1] += __uint_as_float(ub[i] & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x1[i] += __uint_as_float(ua[i]);
                    x2[i] += __uint_as_float(ub[i]);
                }
            }
        }
        scale_by_block(x1, CH, block, inv_b);
        scale_by_block(x2, CH, block, inv_b);
        if (is_k && cs) {
            int mid = j * block + block / 2;
            if (mid > rope_len - 1) mid = rope_len - 1;
            const float* cr = cs + (size_t)mid * half + i0;
            const float* sr = sn + (size_t)mid * half + i0;
#pragma unroll
            for (int e = 0; e < CH; ++e) {
                const float cc = cr[e], ss = sr[e];
                const float y1 = x1[e] * cc - x2[e] * ss;
                const float y2 = x2[e] * cc + x1[e] * ss;
                x1[e] = y1;
                x2[e] = y2;
            }
        }
        char* dst = (char*)(is_k ? pk : pv) + (((size_t)n * nblk + j) * D + i0) * ES;
        uint4 w1, w2;
        if constexpr (BF16) {
            w1 = make_uint4(pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3]), pack_bf16x2(x1[4], x1[5]),
                            pack_bf16x2(x1[6], x1[7]));
            w2 = make_uint4(pack_bf16x2(x2[0], x2[1]), pack_bf16x2(x2[2], x2[3]), pack_bf16x2(x2[4], x2[5]),
                            pack_bf16x2(x2[6], x2[7]));
        } else {
            w1 = make_uint4(__float_as_uint(x1[0]), __float_as_uint(x1[1]), __float_as_uint(x1[2]), __float_as_uint(x1[3]));
            w2 = make_uint4(__float_as_uint(x2[0]), __float_as_uint(x2[1]), __float_as_uint(x2[2]), __float_as_uint(x2[3]));
        }
        *(uint4*)dst = w1;
        *(uint4*)(dst + (size_t)half * ES) = w2;
    }
}

// Pooling of one block per wave, for long blocks.  A row of K followed by its
// row of V is PPR 16-byte pieces; lane l loads piece l % PPR of rows l / PPR,
// l / PPR + RPL, ... of the block (RPL = 64 / PPR rows per step), sums them in
// fp32, and the partial sums of the RPL row groups are added across lanes
// (butterfly over lane bits log2(PPR) and up).  Lanes 0 .. PPR-1 then hold the
// block sums; each divides by b, K pieces exchange with their rotate-half
// partner piece (lane xor PPR/4) for the rotation, and every piece is stored
// once.  (The sums associate differently from a sequential loop; each pooled
// value is still one fp32 sum of b values and one rounding.)
// Grid x covers a row group's blocks (four per workgroup), grid y the row
// groups.
template <bool BF16>
__global__ __launch_bounds__(256) void pool_rope_wave_kernel(int N, int T, int D, int block, int nblk, float inv_b,
                                                            const void* k, const void* v, const float* cs,
                                                            const float* sn, int rope_len, void* pk, void* pv) {
    constexpr int CH = BF16 ? 8 : 4;  // elements per 16-byte piece
    constexpr int ES = BF16 ? 2 : 4;  // bytes per element
    const int j = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (j >= nblk) return;
    const int lane = threadIdx.x & 63;
    for (int n = blockIdx.y; n < N; n += gridDim.y) {
        const int kp = D * ES / 16;  // pieces per K row (and per V row)
        const int ppr = 2 * kp;      // pieces per K+V row pair (a power of two up to 64)
        const int rpl = 64 / ppr;    // rows per step
        const int g = lane / ppr, p = lane % ppr;
        const bool is_k = p < kp;
        const char* src = (const char*)(is_k ? k : v) + ((size_t)n * T + (size_t)j * block) * D * ES +
                          (size_t)(is_k ? p : p - kp) * 16;
        float acc[CH];
#pragma unroll
        for (int e = 0; e < CH; ++e) acc[e] = 0.f;
        for (int r = g; r < block; r += rpl) {
            const uint4 w = *(const uint4*)(src + (size_t)r * D * ES);
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
            if constexpr (BF16) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] += __uint_as_float(u[i] << 16);
                    acc[2 * i + 1] += __uint_as_float(u[i] & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += __uint_as_float(u[i]);
            }
        }
        for (int o = ppr; o < 64; o <<= 1)
#pragma unroll
            for (int e = 0; e < CH; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
        scale_by_block(acc, CH, block, inv_b);
        if (cs) {
            // the rotate-half partner piece (every lane takes part in the exchange)
            const int hp = kp / 2;  // pieces per half row
            float other[CH];
#pragma unroll
            for (int e = 0; e < CH; ++e) other[e] = __shfl_xor(acc[e], hp, 64);
            if (is_k) {
                int mid = j * block + block / 2;
                if (mid > rope_len - 1) mid = rope_len - 1;
                const bool first = p < hp;
                const int i0 = (first ? p : p - hp) * CH;
                const int half = D / 2;
#pragma unroll
                for (int e = 0; e < CH; ++e) {
                    const float c = cs[(size_t)mid * half + i0 + e];
                    const float s = sn[(size_t)mid * half + i0 + e];
                    const float k1 = first ? acc[e] : other[e], k2 = first ? other[e] : acc[e];
                    acc[e] = first ? k1 * c - k2 * s : k2 * c + k1 * s;
                }
            }
        }
        if (g == 0) {
            uint4 w;
            if constexpr (BF16) {
                w = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                               pack_bf16x2(acc[6], acc[7]));
            } else {
                w = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                               __float_as_uint(acc[3]));
            }
            char* dst = (char*)(is_k ? pk : pv) + ((size_t)n * nblk + j) * D * ES + (size_t)(is_k ? p : p - kp) * 16;
            *(uint4*)dst = w;
        }
    }
}

// One thread per (row group n, block j, channel pair i): channels i and i+D/2
// of the pooled key and the pooled value.
template <bool BF16>
__global__ void pool_rope_kernel(long long N, int T, int D, int block, int nblk, float inv_b, const void* k,
                                 const void* v, const float* cs, const float* sn, int rope_len, void* pk, void* pv) {
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
    float kv4[4] = {k1, k2, v1, v2};
    scale_by_block(kv4, 4, block, inv_b);
    k1 = kv4[0];
    k2 = kv4[1];
    v1 = kv4[2];
    v2 = kv4[3];
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

// Rotate every row t of x [N, T, D] at position t (rotate-half pairs
// (i, i + D/2)); one thread per 4 channel pairs.  The fp32 prefill rotates
// its keys with this once instead of once per query block that reads them.
__global__ void rope_rows_f32_kernel(long long rows, int T, int D, const float* x, const float* cs, const float* sn,
                                     float* y) {
    const int half = D / 2;
    const int chunks = half / 4;
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * chunks) return;
    const long long row = idx / chunks;
    const int i0 = (int)(idx % chunks) * 4;
    const int t = (int)(row % T);
    const size_t base = (size_t)row * D;
    const float4 a = *(const float4*)(x + base + i0);
    const float4 bb = *(const float4*)(x + base + half + i0);
    const float4 c = *(const float4*)(cs + (size_t)t * half + i0);
    const float4 s = *(const float4*)(sn + (size_t)t * half + i0);
    *(float4*)(y + base + i0) = make_float4(a.x * c.x - bb.x * s.x, a.y * c.y - bb.y * s.y, a.z * c.z - bb.z * s.z,
                                            a.w * c.w - bb.w * s.w);
    *(float4*)(y + base + half + i0) = make_float4(bb.x * c.x + a.x * s.x, bb.y * c.y + a.y * s.y,
                                                   bb.z * c.z + a.z * s.z, bb.w * c.w + a.w * s.w);
}

// Key rotation of one 8-pair chunk: row `row` of x [rows, D] at position
// t = row % T (rotate-half pairs (i, i + D/2)), 16-byte loads and stores.
__device__ __forceinline__ void rope_chunk_bf16(long long row, int t, int i0, int D, const uint16_t* x,
                                                const float* cs, const float* sn, uint16_t* y) {
    const int half = D / 2;
    const size_t base = (size_t)row * D;
    const uint4 w1 = *(const uint4*)(x + base + i0);
    const uint4 w2 = *(const uint4*)(x + base + half + i0);
    const float4 c0 = *(const float4*)(cs + (size_t)t * half + i0);
    const float4 c1 = *(const float4*)(cs + (size_t)t * half + i0 + 4);
    const float4 s0 = *(const float4*)(sn + (size_t)t * half + i0);
    const float4 s1 = *(const float4*)(sn + (size_t)t * half + i0 + 4);
    const uint32_t a[4] = {w1.x, w1.y, w1.z, w1.w};
    const uint32_t bb[4] = {w2.x, w2.y, w2.z, w2.w};
    const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    uint32_t o1[4], o2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float x1l = __uint_as_float(a[i] << 16), x1h = __uint_as_float(a[i] & 0xffff0000u);
        const float x2l = __uint_as_float(bb[i] << 16), x2h = __uint_as_float(bb[i] & 0xffff0000u);
        const float cl = c[2 * i], ch = c[2 * i + 1], sl = s[2 * i], sh = s[2 * i + 1];
        o1[i] = f32_to_bf16_bits(x1l * cl - x2l * sl) | (f32_to_bf16_bits(x1h * ch - x2h * sh) << 16);
        o2[i] = f32_to_bf16_bits(x2l * cl + x1l * sl) | (f32_to_bf16_bits(x2h * ch + x1h * sh) << 16);
    }
    *(uint4*)(y + base + i0) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
    *(uint4*)(y + base + half + i0) = make_uint4(o2[0], o2[1], o2[2], o2[3]);
}

// Fused pre-pass of a compressed bf16 prefill with RoPE: one read of the
// exact keys and values.  A workgroup takes a span of whole blocks of one
// (batch row, kv head); each thread rotates one 8-pair chunk of one key row
// into the rotated-key buffer (the arithmetic of rope_chunk_bf16) and leaves
// that row's pre-RoPE key and value chunks in LDS as loaded; the block means
// are then summed in fp32 from LDS row by row in order (the arithmetic of
// pool_rope_vec_kernel), and each key mean is rotated at its block midpoint.
template <int D>
__global__ __launch_bounds__(256) void pool_rotate_bf16_kernel(PoolRotArgs p) {
    constexpr int P = D / 16;    // 8-pair chunks per row
    constexpr int R = 256 / P;   // rows a workgroup can hold
    constexpr int LD = D + 8;    // LDS row stride in bf16 (padded against bank conflicts)
    constexpr int half = D / 2;
    __shared__ __align__(16) uint16_t sk[R * LD];  // pre-RoPE keys and values, as loaded
    __shared__ __align__(16) uint16_t sv[R * LD];
    const int n = blockIdx.y;  // (batch row, kv head)
    const int r0 = blockIdx.x * p.span;
    const int tid = threadIdx.x, rl = tid / P, i0 = 8 * (tid % P);
    const int row = r0 + rl;
    if (rl < p.span && row < p.T) {
        const size_t base = ((size_t)n * p.T + row) * D + i0;
        const uint4 k1 = *(const uint4*)(p.k + base), k2 = *(const uint4*)(p.k + base + half);
        const uint4 v1 = *(const uint4*)(p.v + base), v2 = *(const uint4*)(p.v + base + half);
        const float4 c0 = *(const float4*)(p.cs + (size_t)row * half + i0);
        const float4 c1 = *(const float4*)(p.cs + (size_t)row * half + i0 + 4);
        const float4 s0 = *(const float4*)(p.sn + (size_t)row * half + i0);
        const float4 s1 = *(const float4*)(p.sn + (size_t)row * half + i0 + 4);
        *(uint4*)(sk + rl * LD + i0) = k1;
        *(uint4*)(sk + rl * LD + half + i0) = k2;
        *(uint4*)(sv + rl * LD + i0) = v1;
        *(uint4*)(sv + rl * LD + half + i0) = v2;
        const uint32_t a[4] = {k1.x, k1.y, k1.z, k1.w}, bb[4] = {k2.x, k2.y, k2.z, k2.w};
        const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        uint32_t o1[4], o2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x1l = __uint_as_float(a[i] << 16), x1h = __uint_as_float(a[i] & 0xffff0000u);
            const float x2l = __uint_as_float(bb[i] << 16), x2h = __uint_as_float(bb[i] & 0xffff0000u);
            const float cl = c[2 * i], ch = c[2 * i + 1], sl = sn[2 * i], sh = sn[2 * i + 1];
            o1[i] = f32_to_bf16_bits(x1l * cl - x2l * sl) | (f32_to_bf16_bits(x1h * ch - x2h * sh) << 16);
            o2[i] = f32_to_bf16_bits(x2l * cl + x1l * sl) | (f32_to_bf16_bits(x2h * ch + x1h * sh) << 16);
        }
        *(uint4*)(p.kr + base) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
        *(uint4*)(p.kr + base + half) = make_uint4(o2[0], o2[1], o2[2], o2[3]);
    }
    __syncthreads();
    // the span's blocks: one item per (block, tensor, chunk)
    const int nb = p.span / p.block;
    const int j0 = r0 / p.block;
    for (int item = tid; item < nb * 2 * P; item += 256) {
        const int jl = item / (2 * P), rest = item - jl * 2 * P;
        const bool is_v = rest >= P;
        const int q0 = 8 * (rest - (is_v ? P : 0));
        const int j = j0 + jl;
        if (j >= p.nblk) continue;
        const uint16_t* src = (is_v ? sv : sk) + jl * p.block * LD;
        float x1[8], x2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x1[e] = x2[e] = 0.f;
        for (int rr = 0; rr < p.block; ++rr) {
            const uint4 u1 = *(const uint4*)(src + rr * LD + q0), u2 = *(const uint4*)(src + rr * LD + half + q0);
            const uint32_t w1[4] = {u1.x, u1.y, u1.z, u1.w}, w2[4] = {u2.x, u2.y, u2.z, u2.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x1[2 * i] += __uint_as_float(w1[i] << 16);
                x1[2 * i + 1] += __uint_as_float(w1[i] & 0xffff0000u);
                x2[2 * i] += __uint_as_float(w2[i] << 16);
                x2[2 * i + 1] += __uint_as_float(w2[i] & 0xffff0000u);
            }
        }
        scale_by_block(x1, 8, p.block, p.inv_b);
        scale_by_block(x2, 8, p.block, p.inv_b);
        if (!is_v) {
            int mid = j * p.block + p.block / 2;
            if (mid > p.rope_len - 1) mid = p.rope_len - 1;
            const float* cr = p.cs + (size_t)mid * half + q0;
            const float* sr = p.sn + (size_t)mid * half + q0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float cc = cr[e], ss = sr[e];
                const float y1 = x1[e] * cc - x2[e] * ss;
                const float y2 = x2[e] * cc + x1[e] * ss;
                x1[e] = y1;
                x2[e] = y2;
            }
        }
        uint16_t* dst = (is_v ? p.pv : p.pk) + ((size_t)n * p.nblk + j) * D + q0;
        *(uint4*)dst = make_uint4(pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3]), pack_bf16x2(x1[4], x1[5]),
                                  pack_bf16x2(x1[6], x1[7]));
        *(uint4*)(dst + half) = make_uint4(pack_bf16x2(x2[0], x2[1]), pack_bf16x2(x2[2], x2[3]),
                                          pack_bf16x2(x2[4], x2[5]), pack_bf16x2(x2[6], x2[7]));
    }
}

// One launch for everything a bf16 prefill prepares before attention:
//   the first blocks: key metadata, one wave per key tile of 64 keys --
//     info[b][t]     packed segment | sink << 31 of every key
//     ksub[b][2j+h]  KeySum of keys [64j + 32h, 64j + 32h + 32) ∩ [0, T)
//     tsink[b][j]    (min, max) segment of the tile's sink keys,
//                    (INT_MAX, INT_MIN) when it holds none
//   the other blocks: rotate the keys (one thread per 8-pair chunk).
// [NW section "KV Sinks for Tools: Pinning Critical Context"]: the packing
// and sink terms of the mask; the summaries let the attention kernel classify
// sub-tiles and find the tiles holding sinks without reading every key.
__global__ __launch_bounds__(256) void prefill_prep_kernel(PrepArgs p) {
    // (the metadata blocks come first: their load -> reduce -> store chain is
    // the longer one, so they start while the rotation blocks stream)
    const long long meta_blocks = p.info ? ((long long)p.B * p.ntile + 3) / 4 : 0;
    if ((long long)blockIdx.x >= meta_blocks) {
        const int chunks = p.D / 16;
        if (p.rope_rows * chunks < 0x7fffffffLL) {  // 32-bit indexing
            const uint32_t idx = ((uint32_t)blockIdx.x - (uint32_t)meta_blocks) * 256u + threadIdx.x;
            if (idx < (uint32_t)(p.rope_rows * chunks)) {
                const uint32_t row = idx / (uint32_t)chunks;  // chunks is 2 or 4
                const uint32_t t = row - fdiv(row, p.div_T) * (uint32_t)p.T;
                rope_chunk_bf16(row, (int)t, (int)(idx - row * chunks) * 8, p.D, p.x, p.cs, p.sn, p.y);
            }
        } else {
            const long long idx = ((long long)blockIdx.x - meta_blocks) * 256 + threadIdx.x;
            if (idx < p.rope_rows * chunks) {
                const long long row = idx / chunks;
                rope_chunk_bf16(row, (int)(row % p.T), (int)(idx % chunks) * 8, p.D, p.x, p.cs, p.sn, p.y);
            }
        }
        return;
    }
    const long long gt = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gt >= (long long)p.B * p.ntile) return;
    const int lane = threadIdx.x & 63;
    const int b = (int)(gt / p.ntile), j = (int)(gt % p.ntile);
    const int t = 64 * j + lane;
    const bool valid = t < p.T;
    // both loads unconditional (clamped key index) and issued together; the
    // values are selected afterwards
    const size_t ic = (size_t)b * p.T + min(t, p.T - 1);
    int sgv = 1, pfv = 0;
    if (p.seg && p.prefix) {
        sgv = p.seg[ic];
        pfv = p.prefix[ic];
    } else if (p.seg) {
        sgv = p.seg[ic];
    } else {
        pfv = p.prefix[ic];
    }
    write_key_tile_meta(b, j, lane, p.T, p.ntile, valid, sgv, pfv != 0, p.info, p.ksub, p.tsink);
}

}  // namespace

hipError_t launch_prefill_prep(const PrepArgs& p, hipStream_t s) {
    const long long meta_blocks = p.info ? ((long long)p.B * p.ntile + 3) / 4 : 0;
    const long long blocks = p.rope_blocks + meta_blocks;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(prefill_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

bool pool_rotate_fits(int D, int block) { return (D == 32 || D == 64) && block >= 1 && block <= 256 / (D / 16); }

hipError_t launch_pool_rotate_bf16(PoolRotArgs p, hipStream_t s) {
    const int R = 256 / (p.D / 16);
    p.span = p.block * (R / p.block);
    p.inv_b = pow2_reciprocal(p.block);
    const dim3 grid((unsigned)((p.T + p.span - 1) / p.span), (unsigned)p.N);
    if (p.D == 64) hipLaunchKernelGGL(pool_rotate_bf16_kernel<64>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(pool_rotate_bf16_kernel<32>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_rope_rows_f32(long long rows, int T, int D, const float* x, const float* cs, const float* sn,
                                float* y, hipStream_t s) {
    const int threads = 256;
    const long long n = rows * (D / 8);
    hipLaunchKernelGGL(rope_rows_f32_kernel, dim3((unsigned)((n + threads - 1) / threads)), dim3(threads), 0, s,
                       rows, T, D, x, cs, sn, y);
    return hipGetLastError();
}

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
    const float inv_b = pow2_reciprocal(block);
    // row groups go on grid y (at most 65535; the kernels loop over the rest)
    const unsigned gy = (unsigned)(N < 65535 ? N : 65535);
    // 16-byte pieces when a half row is a whole number of them (pointers are
    // 16-byte aligned: the entry point checks): long blocks one wave per
    // pooled row, short ones one thread per piece
    const int ch = dtype == 1 ? 8 : 4;
    const int pieces = 2 * D * (dtype == 1 ? 2 : 4) / 16;  // per K+V row pair
    const long long vec_threads = 2LL * nblk * ((D / 2) / ch);  // per row group
    if (N <= 0x7fffffff && (D / 2) % ch == 0 && block >= 8 && pieces <= 64 && (pieces & (pieces - 1)) == 0) {
        const dim3 gw((unsigned)((nblk + 3) / 4), gy);
        if (dtype == 1)
            hipLaunchKernelGGL((pool_rope_wave_kernel<true>), gw, dim3(256), 0, s, (int)N, T, D, block, nblk, inv_b,
                               k_pre, v, c, sn, rope_len, pk, pv);
        else
            hipLaunchKernelGGL((pool_rope_wave_kernel<false>), gw, dim3(256), 0, s, (int)N, T, D, block, nblk, inv_b,
                               k_pre, v, c, sn, rope_len, pk, pv);
        return hipGetLastError();
    }
    if (N <= 0x7fffffff && (D / 2) % ch == 0 && vec_threads < 0x7fffffffLL) {
        const dim3 gv((unsigned)((vec_threads + 255) / 256), gy);
        const FastDiv div_pr = make_fastdiv((uint32_t)((D / 2) / ch));
        if (dtype == 1)
            hipLaunchKernelGGL((pool_rope_vec_kernel<true>), gv, dim3(256), 0, s, (int)N, T, D, block, nblk, div_pr,
                               inv_b, k_pre, v, c, sn, rope_len, pk, pv);
        else
            hipLaunchKernelGGL((pool_rope_vec_kernel<false>), gv, dim3(256), 0, s, (int)N, T, D, block, nblk, div_pr,
                               inv_b, k_pre, v, c, sn, rope_len, pk, pv);
        return hipGetLastError();
    }
    const long long n = N * nblk * (D / 2);
    const int threads = 256;
    const dim3 grid((unsigned)((n + threads - 1) / threads));
    if (dtype == 1)
        hipLaunchKernelGGL((pool_rope_kernel<true>), grid, dim3(threads), 0, s, N, T, D, block, nblk, inv_b, k_pre, v,
                           c, sn, rope_len, pk, pv);
    else
        hipLaunchKernelGGL((pool_rope_kernel<false>), grid, dim3(threads), 0, s, N, T, D, block, nblk, inv_b, k_pre, v,
                           c, sn, rope_len, pk, pv);
    return hipGetLastError();
}

}  // namespace swa
