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

// Dot of 16 int8 codes (packed in a uint4) with 16 fp32 values.
__device__ __forceinline__ float dot16_i8(const uint4& k, const float* q) {
    const uint32_t w[4] = {k.x, k.y, k.z, k.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int code = (int)(int8_t)((w[i] >> (8 * j)) & 0xffu);
            acc = fmaf(q[4 * i + j], (float)code, acc);
        }
    }
    return acc;
}

// One workgroup per (batch row, kv head).  Each lane owns 16 channels of one
// cache row (LPR lanes per row); the rows of the sink cache and of the valid
// ring positions are dealt to the waves in chunks of NR rows per lane, with
// one online-softmax update per chunk.  Partial (max, sum, acc) states are
// merged across lanes with shuffles and across waves in LDS.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    constexpr int LPR = D / 16;      // lanes per row
    constexpr int RPW = 64 / LPR;    // rows per wave step
    constexpr int NR = 4;            // row steps per chunk
    constexpr int NW = 4;            // waves
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
    const int c = lane % LPR;      // channel chunk: channels 16c .. 16c+15
    const int rsub = lane / LPR;   // row within a wave step
    float qv[G][16];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)b * a.Hq + hkv * G + g) * D + 16 * c;
        const uint4 w0 = *(const uint4*)qrow;
        const uint4 w1 = *(const uint4*)(qrow + 8);
        const uint32_t ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            qv[g][2 * i] = __uint_as_float(ws[i] << 16);
            qv[g][2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
        }
    }
    float m_run[G], l_run[G], acc[G][16];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m_run[g] = kNegInf;
        l_run[g] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;
    }

    for (int base = wave * RPW * NR; base < n_rows; base += NW * RPW * NR) {
        uint4 kc[NR], vc[NR];
        float ksc[NR], vsc[NR];
        bool ok[NR];
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            const int r = base + t * RPW + rsub;
            ok[t] = r < n_rows;
            kc[t] = make_uint4(0, 0, 0, 0);
            vc[t] = make_uint4(0, 0, 0, 0);
            ksc[t] = 0.f;
            vsc[t] = 0.f;
            if (ok[t]) {
                const int8_t* kp;
                const int8_t* vp;
                const float* ksp;
                const float* vsp;
                if (r < sl) {
                    kp = sk + (size_t)r * D;
                    vp = sv + (size_t)r * D;
                    ksp = sks + (size_t)r * GROUPS;
                    vsp = svs + (size_t)r * GROUPS;
                } else {
                    const int slot = (first + (r - sl)) % W;
                    kp = rk + (size_t)slot * D;
                    vp = rv + (size_t)slot * D;
                    ksp = rks + (size_t)slot * GROUPS;
                    vsp = rvs + (size_t)slot * GROUPS;
                }
                kc[t] = *(const uint4*)(kp + 16 * c);
                vc[t] = *(const uint4*)(vp + 16 * c);
                ksc[t] = ksp[c / 2];
                vsc[t] = vsp[c / 2];
            }
        }
        float sc[NR][G];
#pragma unroll
        for (int t = 0; t < NR; ++t) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = dot16_i8(kc[t], qv[g]) * ksc[t];
#pragma unroll
                for (int o = 1; o < LPR; o <<= 1) d += __shfl_xor(d, o, 64);
                sc[t][g] = ok[t] ? d * a.scale : kNegInf;
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float mx = sc[0][g];
#pragma unroll
            for (int t = 1; t < NR; ++t) mx = fmaxf(mx, sc[t][g]);
            const float m_new = fmaxf(m_run[g], mx);
            if (m_new == kNegInf) continue;
            const float corr = __expf(m_run[g] - m_new);
            m_run[g] = m_new;
            l_run[g] *= corr;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[g][i] *= corr;
#pragma unroll
            for (int t = 0; t < NR; ++t) {
                const float p = __expf(sc[t][g] - m_new);
                l_run[g] += p;
                const float pv = p * vsc[t];
                const uint32_t w[4] = {vc[t].x, vc[t].y, vc[t].z, vc[t].w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[g][4 * i + j] = fmaf(pv, (float)(int)(int8_t)((w[i] >> (8 * j)) & 0xffu), acc[g][4 * i + j]);
            }
        }
    }

    // merge lanes that hold the same channels (different rows): xor over row bits
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) {
            const float m_o = __shfl_xor(m_run[g], o, 64);
            const float l_o = __shfl_xor(l_run[g], o, 64);
            const float m_new = fmaxf(m_run[g], m_o);
            const float c_self = m_new == kNegInf ? 0.f : __expf(m_run[g] - m_new);
            const float c_other = m_new == kNegInf ? 0.f : __expf(m_o - m_new);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float a_o = __shfl_xor(acc[g][i], o, 64);
                acc[g][i] = acc[g][i] * c_self + a_o * c_other;
            }
            l_run[g] = l_run[g] * c_self + l_o * c_other;
            m_run[g] = m_new;
        }
    }
    if (rsub == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (c == 0) {
                red_m[wave][g] = m_run[g];
                red_l[wave][g] = l_run[g];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) red_acc[wave][g][16 * c + i] = acc[g][i];
        }
    }
    __syncthreads();
    // final merge across waves: thread -> (g, d)
    for (int e = tid; e < G * D; e += blockDim.x) {
        const int g = e / D, d = e % D;
        float m = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) m = fmaxf(m, red_m[w][g]);
        float l = 0.f, o = 0.f;
        if (m != kNegInf) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = __expf(red_m[w][g] - m);
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
