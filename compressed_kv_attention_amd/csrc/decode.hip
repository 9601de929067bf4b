// decode.hip -- int8 KV quantizer and the ring + sink decode step.
//
// [NS] "256-token滑动窗口+KV sink：Needle 2工具钉住机制源码分析", section
// "256-token 滑动窗口：源码走读": at decode time a key is kept when it is
// recent (q_pos - k_pos < W) or a sink; there is no packing term.  Sinks live
// in their own cache, the window in a ring of W slots (slot = pos mod W).
// The cache layout (one int8 per element plus one fp32 scale per 32
// channels) is the one the budget formula of [NW] "How the 256-Token Sliding
// Window Works with Tools as KV Sinks in Needle", section "Effective KV
// Window: Bounding the Cache Size", prices.
#include "swa_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

// Symmetric absmax/127 quantization of one 32-channel group held by 32
// consecutive lanes (one element per lane).  Returns the code; `s` receives
// the group scale.
__device__ __forceinline__ int quantize_lane(float x, float& s) {
    float amax = fabsf(x);
    amax = wave_max_xor(amax, 1, 16);
    s = amax / 127.0f;
    if (s == 0.0f) return 0;
    float r = rintf(x / s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

__global__ __launch_bounds__(256) void kv_quantize_kernel(long long total, const uint16_t* x, int8_t* xq,
                                                          float* xs) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const bool valid = i < total;
    const float f = valid ? bf16_bits_to_f32(x[i]) : 0.f;
    float s;
    const int code = quantize_lane(f, s);
    if (valid) {
        xq[i] = (int8_t)code;
        if ((threadIdx.x & 31) == 0) xs[i / 32] = s;
    }
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));

// fp32 pair -> f16 pair (round toward zero; exact for values f16 represents).
__device__ __forceinline__ half2_t cvt_pk_f16(float lo, float hi) {
    return __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// int8 codes -> f16 without conversion instructions: a code c is stored as the
// byte u = c ^ 0x80 = c + 128, and the f16 with bits 0x64uu is exactly
// 1024 + u = 1152 + c.  v_perm_b32 assembles two such halves from a word of
// codes and the constant 0x64646464 in one instruction; the 1152 offset is
// removed after the dot products (exactly, up to fp32 rounding).
constexpr uint32_t kMagic = 0x64646464u;
constexpr uint32_t kSelLo = 0x04010400u;  // [b0, 0x64, b1, 0x64]
constexpr uint32_t kSelHi = 0x04030402u;  // [b2, 0x64, b3, 0x64]
constexpr float kBias = 1152.0f;

__device__ __forceinline__ half2_t as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }
__device__ __forceinline__ float fdot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}
// Lane exchanges inside a quad (DPP quad_perm): xor 1 and xor 2.
__device__ __forceinline__ float quad_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// One workgroup per (batch row, kv head), 4 waves.  Each lane owns 16
// channels of one cache row (LPR lanes per row); rows of the sink cache and of
// the valid ring positions are dealt to the waves in chunks of NR row-steps.
// Per chunk: scores with v_dot2_f32_f16 on f16 codes, a wave-wide running max
// per head (so lanes later merge by plain sums), exp2, then O += P V with
// v_dot2_f32_f16 over pairs of rows.  Waves merge in LDS.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    constexpr int LPR = D / 16;    // lanes per row
    constexpr int RPS = 64 / LPR;  // rows per wave-step
    constexpr int NR = 4;          // row-steps per chunk (even)
    constexpr int NW = 4;          // waves
    constexpr int GROUPS = D / 32;
    __shared__ float red_m[NW][G];
    __shared__ float red_l[NW][G];
    __shared__ float red_acc[NW][G][D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x / a.Hkv;
    const int hkv = blockIdx.x % a.Hkv;
    const int W = a.W, S = a.S;
    const int pos_in = a.pos[b];
    const int pos = pos_in < 0 ? -1 : pos_in;  // a negative position appends nothing and sees only sinks
    int sl = a.sink_len ? a.sink_len[b] : S;
    sl = sl < 0 ? 0 : (sl > S ? S : sl);
    const size_t bh = (size_t)b * a.Hkv + hkv;
    int8_t* rk = a.ring_k + bh * W * D;
    int8_t* rv = a.ring_v + bh * W * D;
    float* rks = a.ring_ks + bh * W * GROUPS;
    float* rvs = a.ring_vs + bh * W * GROUPS;
    const int8_t* sk = a.sink_k ? a.sink_k + bh * S * D : nullptr;
    const int8_t* sv = a.sink_v ? a.sink_v + bh * S * D : nullptr;
    const float* sks = a.sink_ks ? a.sink_ks + bh * S * GROUPS : nullptr;
    const float* svs = a.sink_vs ? a.sink_vs + bh * S * GROUPS : nullptr;

    // 1. append the new token into slot pos % W (waves 0 and 1: K and V)
    if (a.k_new && wave < 2 && pos >= 0) {
        const uint16_t* src = (const uint16_t*)(wave == 0 ? a.k_new : a.v_new) + bh * D;
        const int slot = pos % W;
        if (lane < D) {
            float s;
            const int code = quantize_lane(bf16_bits_to_f32(src[lane]), s);
            int8_t* dst = (wave == 0 ? rk : rv) + (size_t)slot * D;
            float* dsts = (wave == 0 ? rks : rvs) + (size_t)slot * GROUPS;
            dst[lane] = (int8_t)code;
            if ((lane & 31) == 0) dsts[lane / 32] = s;
        }
    }
    __threadfence_block();
    __syncthreads();

    // 2. attend
    const int first = max(sl, pos - W + 1);
    const int n_ring = pos >= first ? pos - first + 1 : 0;
    const int n_rows = sl + n_ring;
    const int c4 = lane % LPR;     // channel chunk: channels 16*c4 .. 16*c4+15
    const int rsub = lane / LPR;   // row within a wave-step
    const float c_log2 = a.scale * kLog2e;

    // q of the G heads as f16 pairs of this lane's channels, and their sums
    uint32_t qp[G][8];
    float qsum[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)b * a.Hq + hkv * G + g) * D + 16 * c4;
        const uint4 w0 = *(const uint4*)qrow;
        const uint4 w1 = *(const uint4*)(qrow + 8);
        const uint32_t ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const half2_t h2 = cvt_pk_f16(__uint_as_float(ws[i] << 16), __uint_as_float(ws[i] & 0xffff0000u));
            qp[g][i] = __builtin_bit_cast(uint32_t, h2);
            acc += (float)h2[0] + (float)h2[1];
        }
        qsum[g] = acc * kBias;
    }

    float m_w[G], l_run[G], wsum[G], acc[G][16];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m_w[g] = kNegInf;
        l_run[g] = 0.f;
        wsum[g] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;
    }

    for (int base = wave * RPS * NR; base < n_rows; base += NW * RPS * NR) {
        uint4 kc[NR], vc[NR];
        float ksc[NR], vsc[NR];
        bool ok[NR];
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            const int r = base + t * RPS + rsub;
            ok[t] = r < n_rows;
            const int8_t* kp = rk;
            const int8_t* vp = rv;
            const float* ksp = rks;
            const float* vsp = rvs;
            int row = 0;
            if (ok[t]) {
                if (r < sl) {
                    kp = sk;
                    vp = sv;
                    ksp = sks;
                    vsp = svs;
                    row = r;
                } else {
                    row = (first + (r - sl)) % W;
                }
            }
            kc[t] = ok[t] ? *(const uint4*)(kp + (size_t)row * D + 16 * c4) : make_uint4(0, 0, 0, 0);
            vc[t] = ok[t] ? *(const uint4*)(vp + (size_t)row * D + 16 * c4) : make_uint4(0, 0, 0, 0);
            ksc[t] = ok[t] ? ksp[(size_t)row * GROUPS + c4 / 2] : 0.f;
            vsc[t] = ok[t] ? vsp[(size_t)row * GROUPS + c4 / 2] : 0.f;
        }
        // scores (log2 units)
        float sc[NR][G];
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            const uint32_t kw[4] = {kc[t].x ^ 0x80808080u, kc[t].y ^ 0x80808080u, kc[t].z ^ 0x80808080u,
                                    kc[t].w ^ 0x80808080u};
            uint32_t kh[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kh[2 * i] = __builtin_amdgcn_perm(kMagic, kw[i], kSelLo);
                kh[2 * i + 1] = __builtin_amdgcn_perm(kMagic, kw[i], kSelHi);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) d = fdot2(qp[g][i], kh[i], d);
                d = (d - qsum[g]) * ksc[t];
                d += quad_xor1(d);
                if (LPR == 4) d += quad_xor2(d);
                sc[t][g] = ok[t] ? d * c_log2 : kNegInf;
            }
        }
        // wave-wide running max per head; rescale when it grows
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float mx = sc[0][g];
#pragma unroll
            for (int t = 1; t < NR; ++t) mx = fmaxf(mx, sc[t][g]);
#pragma unroll
            for (int o = LPR; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            if (mx > m_w[g]) {  // wave-uniform
                const float corr = m_w[g] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_w[g] - mx);
                m_w[g] = mx;
                l_run[g] *= corr;
                wsum[g] *= corr;
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[g][i] *= corr;
            }
        }
        // O += P V over pairs of rows
#pragma unroll
        for (int t = 0; t < NR; t += 2) {
            const uint32_t va[4] = {vc[t].x ^ 0x80808080u, vc[t].y ^ 0x80808080u, vc[t].z ^ 0x80808080u,
                                    vc[t].w ^ 0x80808080u};
            const uint32_t vb[4] = {vc[t + 1].x ^ 0x80808080u, vc[t + 1].y ^ 0x80808080u,
                                    vc[t + 1].z ^ 0x80808080u, vc[t + 1].w ^ 0x80808080u};
            uint32_t vh[16];  // channel c: (row t, row t+1) as f16 1152 + code
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t p0 = __builtin_amdgcn_perm(vb[i], va[i], 0x05010400u);
                const uint32_t p1 = __builtin_amdgcn_perm(vb[i], va[i], 0x07030602u);
                vh[4 * i + 0] = __builtin_amdgcn_perm(kMagic, p0, kSelLo);
                vh[4 * i + 1] = __builtin_amdgcn_perm(kMagic, p0, kSelHi);
                vh[4 * i + 2] = __builtin_amdgcn_perm(kMagic, p1, kSelLo);
                vh[4 * i + 3] = __builtin_amdgcn_perm(kMagic, p1, kSelHi);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float p0 = __builtin_amdgcn_exp2f(sc[t][g] - m_w[g]);
                const float p1 = __builtin_amdgcn_exp2f(sc[t + 1][g] - m_w[g]);
                l_run[g] += p0 + p1;
                const half2_t w2 = cvt_pk_f16(p0 * vsc[t], p1 * vsc[t + 1]);
                wsum[g] += (float)w2[0] + (float)w2[1];
                const uint32_t wp = __builtin_bit_cast(uint32_t, w2);
#pragma unroll
                for (int c = 0; c < 16; ++c) acc[g][c] = fdot2(vh[c], wp, acc[g][c]);
            }
        }
    }

    // lanes holding the same channels (different rows) share the running max:
    // plain sums over the row bits of the lane index
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float bias = kBias * wsum[g];
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[g][c] -= bias;
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) {
            l_run[g] += __shfl_xor(l_run[g], o, 64);
#pragma unroll
            for (int c = 0; c < 16; ++c) acc[g][c] += __shfl_xor(acc[g][c], o, 64);
        }
    }
    if (rsub == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (c4 == 0) {
                red_m[wave][g] = m_w[g];
                red_l[wave][g] = l_run[g];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) red_acc[wave][g][16 * c4 + i] = acc[g][i];
        }
    }
    __syncthreads();
    // final merge across waves (log2 units): thread -> (g, d)
    for (int e = tid; e < G * D; e += blockDim.x) {
        const int g = e / D, d = e % D;
        float m = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) m = fmaxf(m, red_m[w][g]);
        float l = 0.f, o = 0.f;
        if (m != kNegInf) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = red_m[w][g] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(red_m[w][g] - m);
                l += red_l[w][g] * f;
                o += red_acc[w][g][d] * f;
            }
        }
        const float val = l > 0.f ? o / l : 0.f;
        ((uint16_t*)a.out)[((size_t)b * a.Hq + hkv * G + g) * D + d] = (uint16_t)f32_to_bf16_bits(val);
    }
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t s) {
    const int G = a.Hq / a.Hkv;
    const dim3 grid(a.B * a.Hkv), block(256);
    switch (G) {
        case 1: hipLaunchKernelGGL((decode_kernel<D, 1>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((decode_kernel<D, 2>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((decode_kernel<D, 4>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((decode_kernel<D, 8>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_quantize(long long N, int D, const void* x, int8_t* xq, float* xs, hipStream_t s) {
    const long long total = N * D;
    const int threads = 256;
    hipLaunchKernelGGL(kv_quantize_kernel, dim3((unsigned)((total + threads - 1) / threads)), dim3(threads), 0, s,
                       total, (const uint16_t*)x, xq, xs);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    if (a.D == 64) return launch_decode_d<64>(a, s);
    return launch_decode_d<32>(a, s);
}

}  // namespace swa
