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

// One workgroup per (batch row, kv head, GW of the G query heads), 4 waves;
// the G/GW workgroups of a kv head are numbered consecutively on one XCD so
// they share its L2.  Each lane owns 16 channels of one cache row (LPR lanes
// per row); rows (sinks, then the valid ring positions) are dealt to the waves
// in chunks of NR row-steps.  Per chunk: scores with v_dot2_f32_f16 on f16
// codes, a running max per row group that is raised lazily (only when a score
// exceeds it by 2^8), exp2, then O += P V with v_dot2_f32_f16 over pairs of
// rows.  Lanes and waves merge their partial (max, sum, output) in LDS.
//
// The appended token is quantized by every workgroup into LDS and attended
// from there (the ring slot it is written to is never read back in the same
// call), so the workgroups of a kv head need no ordering between them.
template <int D, int GW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void decode_kernel(DecodeArgs a) {
    constexpr int LPR = D / 16;    // lanes per row
    constexpr int RPS = 64 / LPR;  // rows per wave-step
    constexpr int NR = 4;          // row-steps per chunk (even)
    constexpr int NW = 4;          // waves
    constexpr int GROUPS = D / 32;
    constexpr float kGrow = 8.0f;  // lazy rescale threshold (log2 units)
    __shared__ float part_m[NW][64][GW];
    __shared__ float part_l[NW][64][GW];
    __shared__ float part_acc[NW][64][GW][17];  // 16 channels, padded
    __shared__ __align__(16) int8_t new_codes[2][D];  // appended K and V codes
    __shared__ float new_scale[2][GROUPS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = a.Hq / a.Hkv;
    const int nsub = G / GW;
    const int nblocks = gridDim.x;
    int lb = blockIdx.x;
    if ((nblocks & 7) == 0) lb = (blockIdx.x & 7) * (nblocks >> 3) + (blockIdx.x >> 3);
    const int hs = lb % nsub;
    const int b = (lb / nsub) / a.Hkv;
    const int hkv = (lb / nsub) % a.Hkv;
    const int h0 = hkv * G + hs * GW;  // first query head of this workgroup
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
    const bool append = a.k_new != nullptr && pos >= 0;
    const int c4 = lane % LPR;     // channel chunk: channels 16*c4 .. 16*c4+15
    const int rsub = lane / LPR;   // row within a wave-step

    // 1. quantize the new token (wave 0: K, wave 1: V) into LDS; the first
    // workgroup of the kv head also writes it into ring slot pos % W
    if (append && wave < 2) {
        const uint16_t* src = (const uint16_t*)(wave == 0 ? a.k_new : a.v_new) + bh * D;
        const bool in = lane < D;
        float sc;
        const int code = quantize_lane(in ? bf16_bits_to_f32(src[in ? lane : 0]) : 0.f, sc);
        if (in) {
            new_codes[wave][lane] = (int8_t)code;
            if ((lane & 31) == 0) new_scale[wave][lane / 32] = sc;
            if (hs == 0) {
                const int slot = pos % W;
                ((wave == 0 ? rk : rv) + (size_t)slot * D)[lane] = (int8_t)code;
                if ((lane & 31) == 0) (wave == 0 ? rks : rvs)[(size_t)slot * GROUPS + lane / 32] = sc;
            }
        }
    }
    __syncthreads();

    // 2. attend: sink rows [0, sl), ring positions [first, pos]
    const int first = max(sl, pos - W + 1);
    const int n_ring = pos >= first ? pos - first + 1 : 0;
    const int n_rows = sl + n_ring;
    const int r_new = (append && n_ring > 0) ? n_rows - 1 : 0x7fffffff;  // row held in registers
    const int first_slot = first >= 0 ? first % W : 0;
    const float c_log2 = a.scale * kLog2e;

    // q of the GW heads as f16 pairs of this lane's channels; their sums times
    // the code offset start each dot product
    uint32_t qp[GW][8];
    float qbias[GW];
#pragma unroll
    for (int g = 0; g < GW; ++g) {
        const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)b * a.Hq + h0 + g) * D + 16 * c4;
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
        qbias[g] = -acc * kBias;
    }

    float m_ref[GW], l_run[GW], wsum[GW], acc[GW][16];
#pragma unroll
    for (int g = 0; g < GW; ++g) {
        m_ref[g] = kNegInf;
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
            kc[t] = vc[t] = make_uint4(0, 0, 0, 0);
            ksc[t] = vsc[t] = 0.f;
            if (r == r_new) {  // the appended token
                kc[t] = *(const uint4*)&new_codes[0][16 * c4];
                vc[t] = *(const uint4*)&new_codes[1][16 * c4];
                ksc[t] = new_scale[0][c4 / 2];
                vsc[t] = new_scale[1][c4 / 2];
            } else if (ok[t]) {
                const int8_t* kp = rk;
                const int8_t* vp = rv;
                const float* ksp = rks;
                const float* vsp = rvs;
                int row;
                if (r < sl) {
                    kp = sk;
                    vp = sv;
                    ksp = sks;
                    vsp = svs;
                    row = r;
                } else {
                    row = first_slot + (r - sl);
                    row = row >= W ? row - W : row;
                }
                kc[t] = *(const uint4*)(kp + (size_t)row * D + 16 * c4);
                vc[t] = *(const uint4*)(vp + (size_t)row * D + 16 * c4);
                ksc[t] = ksp[(size_t)row * GROUPS + c4 / 2];
                vsc[t] = vsp[(size_t)row * GROUPS + c4 / 2];
            }
        }
        // scores (log2 units); every lane of a row ends with the row's score
        float sc[NR][GW];
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
            const float ks = ksc[t] * c_log2;
#pragma unroll
            for (int g = 0; g < GW; ++g) {
                float d = qbias[g];
#pragma unroll
                for (int i = 0; i < 8; ++i) d = fdot2(qp[g][i], kh[i], d);
                d *= ks;
                d += quad_xor1(d);
                if (LPR == 4) d += quad_xor2(d);
                sc[t][g] = ok[t] ? d : kNegInf;
            }
        }
        // raise the reference max of a row group only when a score outgrows it
        // by more than 2^8 (the first valid row always does)
        float cmax[GW];
        bool grow = false;
#pragma unroll
        for (int g = 0; g < GW; ++g) {
            cmax[g] = sc[0][g];
#pragma unroll
            for (int t = 1; t < NR; ++t) cmax[g] = fmaxf(cmax[g], sc[t][g]);
            grow |= cmax[g] > m_ref[g] + kGrow;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int g = 0; g < GW; ++g) {
                const bool up = cmax[g] > m_ref[g] + kGrow;
                const float corr =
                    up ? (m_ref[g] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_ref[g] - cmax[g])) : 1.f;
                m_ref[g] = up ? cmax[g] : m_ref[g];
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
            for (int g = 0; g < GW; ++g) {
                const float p0 = ok[t] ? __builtin_amdgcn_exp2f(sc[t][g] - m_ref[g]) : 0.f;
                const float p1 = ok[t + 1] ? __builtin_amdgcn_exp2f(sc[t + 1][g] - m_ref[g]) : 0.f;
                l_run[g] += p0 + p1;
                const half2_t w2 = cvt_pk_f16(p0 * vsc[t], p1 * vsc[t + 1]);
                const uint32_t wp = __builtin_bit_cast(uint32_t, w2);
                wsum[g] = fdot2(wp, 0x3c003c00u, wsum[g]);  // exact sum of the two f16 weights
#pragma unroll
                for (int c = 0; c < 16; ++c) acc[g][c] = fdot2(vh[c], wp, acc[g][c]);
            }
        }
    }

    // 3. merge: every lane leaves (max, sum, 16 outputs) per head in LDS; the
    // rows of a lane quad carry identical max and sum
#pragma unroll
    for (int g = 0; g < GW; ++g) {
        const float bias = kBias * wsum[g];
        part_m[wave][lane][g] = m_ref[g];
        part_l[wave][lane][g] = l_run[g];
#pragma unroll
        for (int i = 0; i < 16; ++i) part_acc[wave][lane][g][i] = acc[g][i] - bias;
    }
    __syncthreads();
    // thread -> (head g, channel d): combine the NW * RPS partials of its channel chunk
    for (int e = tid; e < GW * D; e += 64 * NW) {
        const int g = e / D, d = e % D;
        const int cc = d / 16, i = d % 16;
        float m = kNegInf;
        for (int w = 0; w < NW; ++w)
            for (int r = 0; r < RPS; ++r) m = fmaxf(m, part_m[w][r * LPR + cc][g]);
        float l = 0.f, o = 0.f;
        if (m != kNegInf) {
            for (int w = 0; w < NW; ++w)
                for (int r = 0; r < RPS; ++r) {
                    const int ln = r * LPR + cc;
                    const float mm = part_m[w][ln][g];
                    const float f = mm == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mm - m);
                    l += part_l[w][ln][g] * f;
                    o += part_acc[w][ln][g][i] * f;
                }
        }
        const float val = l > 0.f ? o / l : 0.f;
        ((uint16_t*)a.out)[((size_t)b * a.Hq + h0 + g) * D + d] = (uint16_t)f32_to_bf16_bits(val);
    }
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t s) {
    const int G = a.Hq / a.Hkv;
    const int gw = G >= 2 ? 2 : 1;
    const long long nblocks = (long long)a.B * a.Hkv * (G / gw);
    if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nblocks), block(256);
    if (gw == 2)
        hipLaunchKernelGGL((decode_kernel<D, 2>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((decode_kernel<D, 1>), grid, block, 0, s, a);
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
