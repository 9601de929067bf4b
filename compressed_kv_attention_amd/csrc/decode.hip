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

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// DPP quad permutations: xor 2 within a quad, and a broadcast of quad lane r.
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) { return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) { return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); }
template <int R>
__device__ __forceinline__ float quad_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), R * 0x55, 0xF, 0xF, false));
}

// Four int8 codes -> four f16 values 1152 + code (see kMagic).
__device__ __forceinline__ half4_t codes_to_h4(uint32_t w) {
    const uint32_t u = w ^ 0x80808080u;
    const uint32_t lo = __builtin_amdgcn_perm(kMagic, u, kSelLo);
    const uint32_t hi = __builtin_amdgcn_perm(kMagic, u, kSelHi);
    return __builtin_bit_cast(half4_t, make_uint2(lo, hi));
}

// v_mfma_f32_4x4x4f16 runs 16 independent 4x4x4 blocks; block b is lanes
// 4b..4b+3 and, with c = lane % 4, computes
//   C(lane 4b+c, reg r) += sum_e A(lane 4b+r, e) * B(lane 4b+c, e).
// Decode uses it twice per chunk of 64 cache rows, one row per lane:
//   scores: A = K row of lane 4b+r (4 channels per instruction), B = q of
//           head c  ->  C(4b+c, r) = score of head c on key 4b+r;
//   P V:    A = weights of head r on keys 4b+e (exactly the layout the scores
//           came out in), B = V codes of keys 4b+e at channel 4i+c (a 4x4
//           byte transpose inside the quad)  ->  C(4b+c, r) = partial output
//           of head r at channel 4i+c over the quad's keys.
// So every softmax quantity of lane 4b+c belongs to head c and keys 4b..4b+3.
template <int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(DecodeArgs a) {
    constexpr int NI = D / 4;       // 4-channel instructions per row
    constexpr int GROUPS = D / 32;  // scale groups per row
    constexpr int NW = 2;           // waves
    constexpr int CH = 64;          // rows per chunk (one per lane)
    constexpr float kGrow = 8.0f;   // lazy rescale threshold (log2 units)
    __shared__ float part_acc[NW][64][NI * 4 + 1];
    __shared__ float part_ws[NW][64][GROUPS];
    __shared__ float part_l[NW][64];
    __shared__ float part_m[NW][4];
    __shared__ __align__(16) int8_t new_codes[2][D];  // appended K and V codes
    __shared__ float new_scale[2][GROUPS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 3;  // head of this lane's softmax quantities
    const int G = a.Hq / a.Hkv;
    const int nsub = (G + 3) / 4;
    const int hs = blockIdx.x % nsub;
    const int b = (blockIdx.x / nsub) / a.Hkv;
    const int hkv = (blockIdx.x / nsub) % a.Hkv;
    const int h0 = hkv * G + hs * 4;            // first query head of this workgroup
    const int nh = min(4, G - hs * 4);          // heads served (padding heads have q = 0)
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
    const int8_t* sk = a.sink_k ? a.sink_k + bh * S * D : rk;  // (never read when sl == 0)
    const int8_t* sv = a.sink_v ? a.sink_v + bh * S * D : rv;
    const float* sks = a.sink_ks ? a.sink_ks + bh * S * GROUPS : rks;
    const float* svs = a.sink_vs ? a.sink_vs + bh * S * GROUPS : rvs;
    const bool append = a.k_new != nullptr && pos >= 0;

    // rows: sinks [0, sl), then ring positions [first, pos]; with an append
    // the last of them (position pos) comes from LDS
    const int first = max(sl, pos - W + 1);
    const int n_ring = pos >= first ? pos - first + 1 : 0;
    const int n_rows = sl + n_ring;
    const int r_new = (append && n_ring > 0) ? n_rows - 1 : -1;
    const int first_slot = first >= 0 ? first % W : 0;
    const float c_log2 = a.scale * kLog2e;

    // Row r of the walk -> cache row; rows past the end read row 0 of the
    // ring (valid memory) and are masked, so every chunk issues the same loads.
    uint4 kr[NI / 4], vr[NI / 4];
    float2 ksc, vsc;
    auto row_of = [&](int base, bool& sink) {
        const int r = base + lane;
        const bool ok = r < n_rows && r != r_new;
        sink = ok && r < sl;
        int row = first_slot + (r - sl);
        row = row >= W ? row - W : row;
        return ok ? (sink ? r : row) : 0;
    };
    auto load_k = [&](int base) {
        bool sink;
        const int row = row_of(base, sink);
        const int8_t* kp = (sink ? sk : rk) + (size_t)row * D;
#pragma unroll
        for (int j = 0; j < NI / 4; ++j) kr[j] = *(const uint4*)(kp + 16 * j);
        const float* ksp = (sink ? sks : rks) + (size_t)row * GROUPS;
        ksc.x = ksp[0];
        ksc.y = GROUPS > 1 ? ksp[GROUPS - 1] : 0.f;
    };
    auto load_v = [&](int base) {
        bool sink;
        const int row = row_of(base, sink);
        const int8_t* vp = (sink ? sv : rv) + (size_t)row * D;
#pragma unroll
        for (int j = 0; j < NI / 4; ++j) vr[j] = *(const uint4*)(vp + 16 * j);
        const float* vsp = (sink ? svs : rvs) + (size_t)row * GROUPS;
        vsc.x = vsp[0];
        vsc.y = GROUPS > 1 ? vsp[GROUPS - 1] : 0.f;
    };
    int base = wave * CH;
    load_k(base);
    load_v(base);

    // q of head c as the B operand: 4 channels per instruction, f16
    half4_t qb[NI];
    float qbias[GROUPS];
    {
        const bool live = c < nh;
        const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)b * a.Hq + h0 + (live ? c : 0)) * D;
#pragma unroll
        for (int g = 0; g < GROUPS; ++g) qbias[g] = 0.f;
#pragma unroll
        for (int j = 0; j < NI / 2; ++j) {
            const uint4 w = live ? *(const uint4*)(qrow + 8 * j) : make_uint4(0, 0, 0, 0);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const half2_t lo = cvt_pk_f16(__uint_as_float(ws[2 * h] << 16), __uint_as_float(ws[2 * h] & 0xffff0000u));
                const half2_t hi =
                    cvt_pk_f16(__uint_as_float(ws[2 * h + 1] << 16), __uint_as_float(ws[2 * h + 1] & 0xffff0000u));
                qb[2 * j + h] = half4_t{lo[0], lo[1], hi[0], hi[1]};
                qbias[(8 * j) / 32] += (float)lo[0] + (float)lo[1] + (float)hi[0] + (float)hi[1];
            }
        }
#pragma unroll
        for (int g = 0; g < GROUPS; ++g) qbias[g] *= -kBias;
    }

    // quantize the new token (wave 0: K, wave 1: V) into LDS; the first
    // workgroup of the kv head also writes it into ring slot pos % W
    if (append) {
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

    // lane-dependent byte selectors of the quad transpose
    const uint32_t sel1 = (c < 2) ? 0x05040100u : 0x03020706u;
    const uint32_t sel2 = (c & 1) ? 0x03070105u : 0x06020400u;

    f32x4_t acc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_h[4] = {kNegInf, kNegInf, kNegInf, kNegInf};  // reference max per head (wave-uniform)
    float m_c = kNegInf;                                  // = m_h[c]
    float l_c = 0.f;                                      // row sum of head c (this lane's keys)
    float ws_c[GROUPS];                                   // sum of f16 weights of head c per group
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) ws_c[g] = 0.f;

    while (base < n_rows) {
        if (r_new >= base && r_new < base + CH && lane == r_new - base) {  // the appended token
#pragma unroll
            for (int j = 0; j < NI / 4; ++j) {
                kr[j] = *(const uint4*)&new_codes[0][16 * j];
                vr[j] = *(const uint4*)&new_codes[1][16 * j];
            }
            ksc = make_float2(new_scale[0][0], new_scale[0][GROUPS - 1]);
            vsc = make_float2(new_scale[1][0], new_scale[1][GROUPS - 1]);
        }
        // scores: C_g(4b+c, r) = sum over group g of q_c * (1152 + code) - 1152 * sum q_c
        f32x4_t s0 = f32x4_t{qbias[0], qbias[0], qbias[0], qbias[0]};
        f32x4_t s1 = f32x4_t{qbias[GROUPS - 1], qbias[GROUPS - 1], qbias[GROUPS - 1], qbias[GROUPS - 1]};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint4 w4 = kr[i / 4];
            const uint32_t w = (i % 4 == 0) ? w4.x : (i % 4 == 1) ? w4.y : (i % 4 == 2) ? w4.z : w4.w;
            if (i < 8)
                s0 = __builtin_amdgcn_mfma_f32_4x4x4f16(codes_to_h4(w), qb[i], s0, 0, 0, 0);
            else
                s1 = __builtin_amdgcn_mfma_f32_4x4x4f16(codes_to_h4(w), qb[i], s1, 0, 0, 0);
        }
        // per-key scales of the quad's keys (key 4b + r sits in quad lane r)
        const float ks0[4] = {quad_bcast<0>(ksc.x), quad_bcast<1>(ksc.x), quad_bcast<2>(ksc.x), quad_bcast<3>(ksc.x)};
        const float vs0[4] = {quad_bcast<0>(vsc.x), quad_bcast<1>(vsc.x), quad_bcast<2>(vsc.x), quad_bcast<3>(vsc.x)};
        float ks1[4], vs1[4];
        if (GROUPS > 1) {
            ks1[0] = quad_bcast<0>(ksc.y);
            ks1[1] = quad_bcast<1>(ksc.y);
            ks1[2] = quad_bcast<2>(ksc.y);
            ks1[3] = quad_bcast<3>(ksc.y);
            vs1[0] = quad_bcast<0>(vsc.y);
            vs1[1] = quad_bcast<1>(vsc.y);
            vs1[2] = quad_bcast<2>(vsc.y);
            vs1[3] = quad_bcast<3>(vsc.y);
        }
        load_k(base + NW * CH);  // the next chunk's K rows load while this chunk finishes
        const int kq = base + (lane & ~3);  // walk index of the quad's key 0
        float sc[4];
        bool grow = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = s0[r] * ks0[r];
            if (GROUPS > 1) v = __builtin_fmaf(s1[r], ks1[r], v);
            sc[r] = (kq + r < n_rows) ? v * c_log2 : kNegInf;
            grow |= sc[r] > m_c + kGrow;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            // new reference max of every head: the max over the wave's lanes of that head
            float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
#pragma unroll
            for (int o = 4; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            float corr[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float mx_h = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), h));
                const bool up = mx_h > m_h[h] + kGrow;
                corr[h] = up ? (m_h[h] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_h[h] - mx_h)) : 1.f;
                m_h[h] = up ? mx_h : m_h[h];
            }
            m_c = c == 0 ? m_h[0] : c == 1 ? m_h[1] : c == 2 ? m_h[2] : m_h[3];
            const float corr_c = c == 0 ? corr[0] : c == 1 ? corr[1] : c == 2 ? corr[2] : corr[3];
            l_c *= corr_c;
#pragma unroll
            for (int g = 0; g < GROUPS; ++g) ws_c[g] *= corr_c;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][r] *= corr[r];
        }
        // weights of head c on the quad's keys, scaled per V group, as the A operand
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = (kq + r < n_rows) ? __builtin_amdgcn_exp2f(sc[r] - m_c) : 0.f;
            l_c += p[r];
        }
        const half2_t a0l = cvt_pk_f16(p[0] * vs0[0], p[1] * vs0[1]);
        const half2_t a0h = cvt_pk_f16(p[2] * vs0[2], p[3] * vs0[3]);
        const half4_t pa0 = half4_t{a0l[0], a0l[1], a0h[0], a0h[1]};
        ws_c[0] = fdot2(__builtin_bit_cast(uint32_t, a0l), 0x3c003c00u, ws_c[0]);
        ws_c[0] = fdot2(__builtin_bit_cast(uint32_t, a0h), 0x3c003c00u, ws_c[0]);
        half4_t pa1 = pa0;
        if (GROUPS > 1) {
            const half2_t a1l = cvt_pk_f16(p[0] * vs1[0], p[1] * vs1[1]);
            const half2_t a1h = cvt_pk_f16(p[2] * vs1[2], p[3] * vs1[3]);
            pa1 = half4_t{a1l[0], a1l[1], a1h[0], a1h[1]};
            ws_c[GROUPS - 1] = fdot2(__builtin_bit_cast(uint32_t, a1l), 0x3c003c00u, ws_c[GROUPS - 1]);
            ws_c[GROUPS - 1] = fdot2(__builtin_bit_cast(uint32_t, a1h), 0x3c003c00u, ws_c[GROUPS - 1]);
        }
        // O += P V: V codes of the quad's keys at channel 4i + c
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint4 w4 = vr[i / 4];
            const uint32_t w = (i % 4 == 0) ? w4.x : (i % 4 == 1) ? w4.y : (i % 4 == 2) ? w4.z : w4.w;
            const uint32_t t = __builtin_amdgcn_perm(dpp_xor2(w), w, sel1);
            const uint32_t col = __builtin_amdgcn_perm(dpp_xor1(t), t, sel2);
            acc[i] = __builtin_amdgcn_mfma_f32_4x4x4f16(i < 8 ? pa0 : pa1, codes_to_h4(col), acc[i], 0, 0, 0);
        }
        base += NW * CH;
        load_v(base);
    }

    // merge: lanes of one head and channel (16 quads) and the two waves
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) part_acc[wave][lane][4 * i + r] = acc[i][r];
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) part_ws[wave][lane][g] = ws_c[g];
    part_l[wave][lane] = l_c;
    if (lane < 4) part_m[wave][lane] = m_c;
    __syncthreads();
    for (int e = tid; e < 4 * D; e += 64 * NW) {
        const int h = e / D, d = e % D;
        if (h >= nh) continue;
        const int i = d / 4, cc = d % 4, g = d / 32;
        float m = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) m = fmaxf(m, part_m[w][h]);
        float l = 0.f, o = 0.f;
        if (m != kNegInf) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float mw = part_m[w][h];
                if (mw == kNegInf) continue;
                float ow = 0.f, wsw = 0.f, lw = 0.f;
#pragma unroll
                for (int q4 = 0; q4 < 16; ++q4) {
                    ow += part_acc[w][4 * q4 + cc][4 * i + h];
                    wsw += part_ws[w][4 * q4 + h][g];
                    lw += part_l[w][4 * q4 + h];
                }
                const float f = __builtin_amdgcn_exp2f(mw - m);
                o += (ow - kBias * wsw) * f;
                l += lw * f;
            }
        }
        const float val = l > 0.f ? o / l : 0.f;
        ((uint16_t*)a.out)[((size_t)b * a.Hq + h0 + h) * D + d] = (uint16_t)f32_to_bf16_bits(val);
    }
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t s) {
    const int G = a.Hq / a.Hkv;
    const long long nblocks = (long long)a.B * a.Hkv * ((G + 3) / 4);
    if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_kernel<D>), dim3((unsigned)nblocks), dim3(128), 0, s, a);
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
