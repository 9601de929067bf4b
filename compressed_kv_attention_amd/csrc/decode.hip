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
#include <mutex>

#include "swa_common.h"
#include "swa_internal.h"

// Optional phase-time accounting for profiling builds; no code in normal builds.
#ifndef SWA_TRACE_DECL
#define SWA_TRACE_DECL
#define SWA_TRACE(slot)
#endif

namespace swa {
namespace {


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
// fp32 pair -> f16 pair, round to nearest even (one v_cvt_pk_f16_f32): the
// weight operands, whose rounding errors then carry no bias.
__device__ __forceinline__ half2_t cvt_pk_f16_rne(float lo, float hi) {
    return half2_t{(_Float16)lo, (_Float16)hi};
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
// (Every lane of a quad permutation has a source, so the "old" operand is
// never used; passing the source itself avoids materialising one.)
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) { return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) { return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false); }

// Four int8 codes -> four f16 values 1152 + code (see kMagic).
__device__ __forceinline__ half4_t codes_to_h4(uint32_t w) {
    const uint32_t u = w ^ 0x80808080u;
    const uint32_t lo = __builtin_amdgcn_perm(kMagic, u, kSelLo);
    const uint32_t hi = __builtin_amdgcn_perm(kMagic, u, kSelHi);
    return __builtin_bit_cast(half4_t, make_uint2(lo, hi));
}

// q and the appended token are read by global loads the compiler does not
// track either (they are issued before a chunk's direct loads and waited for
// with vm_wait_upto); tie() marks the point after that wait from which their
// registers may be read.
template <class X>
__device__ __forceinline__ void tie(X& x) {
    asm volatile("" : "+v"(x));
}
__device__ __forceinline__ u32x4 gload_b128_untracked(const void* p) {
    u32x4 r;
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p) : "memory");
    return r;
}
__device__ __forceinline__ uint32_t gload_b32_untracked(const void* p) {
    uint32_t r;
    asm volatile("global_load_dword %0, %1, off" : "=v"(r) : "v"(p) : "memory");
    return r;
}
__device__ __forceinline__ uint32_t gload_u16_untracked(const void* p) {
    uint32_t r;
    asm volatile("global_load_ushort %0, %1, off" : "=v"(r) : "v"(p) : "memory");
    return r;
}

// One wave's LDS copy of a chunk of 64 cache rows: K and V codes (row-major,
// 16-byte pieces of row r stored XOR-swizzled by (r >> 1) so that one row per
// lane reads without bank conflicts) and the group scales.
template <int D>
struct DecBuf {
    int8_t k[64 * D];
    int8_t v[64 * D];
    float ks[64 * (D / 32)];
    float vs[64 * (D / 32)];
};

template <int D, int NW, int NBUF>
struct DecSmem {
    // chunks in flight, per wave; after its walk a wave leaves its per-head
    // outputs (before normalisation, [4][D] floats) in its own first buffer
    DecBuf<D> buf[NW][NBUF];
    float part_m[NW][4], part_l[NW][4];
    int last;  // this workgroup is the last of its unit to finish (split-K)
    static_assert(sizeof(DecBuf<D>) >= 4 * D * sizeof(float), "partials fit a chunk buffer");
    __device__ float* part_o(int w) { return (float*)&buf[w][0]; }
};


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
//
// A workgroup of NW waves serves one (batch row, kv head, up to 4 query
// heads); the waves take the chunks of the walk in turn and merge at the end.
// Rows reach LDS by DMA in coalesced 16-rows-per-instruction pieces into one
// chunk buffer per wave, whose K part (rows and scales) and V part are each
// refilled with the next chunk as soon as they have been read; each lane
// then reads its own row.  The walk
// is cut into chunks of 64 rows that lie wholly in the sink cache or wholly
// in the ring (one base pointer per chunk).
//
// The appended token is quantized in registers while the first chunks load
// (the first wave of the kv head also stores it into ring slot pos % W,
// which the walk over positions [first, pos - 1] never reads); it joins the
// final merge as one more exact softmax partial, so the walk needs no
// per-lane special case.
//
// Compressed mode (COMP): the sink cache is the cache of pooled blocks, of
// which the first floor((pos - W + 1) / b) -- those that have cleared the
// window -- are walked, and the ring holds the window from position
// max(0, pos - W + 1).  The appending wave also adds the new token's pre-RoPE
// key and its value to the frontier sums of the block in progress and, when
// the token completes its block, stores the block's mean (the key rotated at
// the block midpoint) quantized into the block's pooled slot; that slot is
// not walked before position pos + W.
template <int D, int NW, bool COMP>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(3))) void decode_kernel(DecodeArgs a) {
    constexpr int NI = D / 4;       // 4-channel instructions per row
    constexpr int GROUPS = D / 32;  // scale groups per row
    constexpr int NBUF = 1;         // chunk buffers per wave (K and V parts refilled separately)
    constexpr int CH = 64;          // rows per chunk (one per lane)
    constexpr int CPR = D / 16;     // 16-byte pieces per row
    constexpr int RPI = 64 / CPR;   // rows per DMA instruction
    constexpr int NKI = CH / RPI;   // DMA instructions per chunk for K (and for V)
    constexpr int NDMA_PART = NKI + GROUPS;     // DMA instructions per chunk part (K or V)
    constexpr int NDMA = 2 * NDMA_PART;         // DMA instructions per chunk
    constexpr float kGrow = 8.0f;   // lazy rescale threshold (log2 units)
    constexpr int kNoExp = -100000; // "no V scale seen yet"
    __shared__ __align__(16) DecSmem<D, NW, NBUF> sm;
    SWA_TRACE_DECL

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 3;  // head of this lane's softmax quantities
    const int G = a.Hq / a.Hkv;
    const int nsub = (G + 3) / 4;
    // workgroup -> (unit = (batch row, kv head, group of 4 query heads), split)
    const int splits = a.num_splits;
    const int sp = blockIdx.x % splits;
    const int unit = blockIdx.x / splits;
    const int hs = unit % nsub;
    const int b = (unit / nsub) / a.Hkv;
    const int hkv = (unit / nsub) % a.Hkv;
    const int h0 = hkv * G + hs * 4;    // first query head of this wave
    const int nh = min(4, G - hs * 4);  // heads served (padding heads have q = 0)
    const int W = a.W, S = a.S;
    const int pos_in = a.pos[b];
    const int pos = pos_in < 0 ? -1 : pos_in;  // a negative position appends nothing and sees only sinks
    int sl;
    if constexpr (COMP) {
        // pooled blocks that have cleared the window: (j + 1) * b <= pos - W + 1
        const int cleared = pos - W + 1;
        sl = cleared >= a.block ? min(cleared / a.block, S) : 0;
    } else {
        sl = a.sink_len ? a.sink_len[b] : S;
        sl = sl < 0 ? 0 : (sl > S ? S : sl);
    }
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
    // the last of them (position pos) is merged from registers at the end
    const int first = COMP ? max(0, pos - W + 1) : max(sl, pos - W + 1);
    const int n_ring = pos >= first ? pos - first + 1 : 0;
    const bool has_new = append && n_ring > 0;
    const int n_ring_mem = n_ring - (has_new ? 1 : 0);  // ring rows read from the cache
    const int first_slot = first >= 0 ? first % W : 0;
    // This split's share of the walk over the sl + n_ring_mem cached rows:
    // rows [r0, r1), whole 16-row pieces, cut into its sink part [s0, s1) and
    // its ring part [g0, g1) (ring rows counted from position `first`).
    int r0 = 0, r1 = sl + n_ring_mem;
    if (splits > 1) {
        const int per = (((r1 + splits - 1) / splits) + 15) & ~15;
        r0 = min(sp * per, r1);
        r1 = min(r0 + per, r1);
    }
    const int s0 = min(r0, sl), s1 = min(r1, sl);
    const int g0 = max(r0, sl) - sl, g1 = max(r1, sl) - sl;
    const int nc_s = (s1 - s0 + CH - 1) / CH;
    const int n_chunks = nc_s + (g1 - g0 + CH - 1) / CH;
    const float c_log2_all = a.scale * kLog2e;
    // Step ci of the walk reads chunk ci (sinks first, then the ring), so the
    // two waves of a workgroup read neighbouring chunks at the same time;
    // steps past the end read nothing useful.  (Starting the workgroups at
    // different chunks, to spread their first requests, measured slower.)
    auto chunk_of = [&](int ci) { return ci; };
    // this wave's steps: kk -> walk step wave + NW * kk
    const int n_steps = n_chunks > wave ? (n_chunks - wave + NW - 1) / NW : 0;
    auto first_row_of = [&](int cj) { return cj < nc_s ? s0 + cj * CH : g0 + (cj - nc_s) * CH; };
    auto rows_of = [&](int cj) { return min(CH, (cj < nc_s ? s1 : g1) - first_row_of(cj)); };
    auto chunk_rows = [&](int ci) { return rows_of(chunk_of(ci)); };

    // per-head maxima over the wave's lanes of head c (lane bits 2..5), made
    // wave-uniform (every quad holds the same four rows' scales)
    auto all_blocks_umax = [](uint32_t x) {
        x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x124, 0xF, 0xF, false));
        x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x128, 0xF, 0xF, false));
        const auto s16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        x = max(s16[0], s16[1]);
        const auto s32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return __builtin_amdgcn_readfirstlane(max(s32[0], s32[1]));
    };
    // per-head sums over the wave's lanes of head c (lane bits 2..5)
    auto all_blocks = [](float x) {
        x += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x124, 0xF, 0xF, false));
        x += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x128, 0xF, 0xF, false));
        auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
        auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
    };

    // q of head c (padding heads read head 0 and are zeroed below) and the
    // appended token's elements of this lane; issued before the cache rows so
    // they arrive first
    const bool live = c < nh;
    u32x4 qraw[NI / 2];
    {
        const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)b * a.Hq + h0 + (live ? c : 0)) * D;
#pragma unroll
        for (int j = 0; j < NI / 2; ++j) qraw[j] = gload_b128_untracked(qrow + 8 * j);
    }
    const uint16_t* kn_src = append ? (const uint16_t*)a.k_new + bh * D : (const uint16_t*)a.q;
    const uint16_t* vn_src = append ? (const uint16_t*)a.v_new + bh * D : (const uint16_t*)a.q;
    uint32_t xk = gload_u16_untracked(kn_src + lane % D), xv = gload_u16_untracked(vn_src + lane % D);
    // compressed mode: the pre-RoPE key and the frontier sums of this lane's
    // channel (every (batch row, kv head) has them, so the loads stay in bounds)
    uint32_t xkp = 0, xfk = 0, xfv = 0;
    if constexpr (COMP) {
        xkp = gload_u16_untracked((const uint16_t*)a.k_pre + bh * D + lane % D);
        xfk = gload_b32_untracked(a.front_k + bh * D + lane % D);
        xfv = gload_b32_untracked(a.front_v + bh * D + lane % D);
    }

    // DMA of chunk ci into buffer bi: NKI instructions each for K and V (RPI
    // rows of CPR pieces), GROUPS each for the two scale arrays.  Rows past a
    // chunk's last valid row repeat its first row; a chunk past the end reads
    // row 0 of the ring and is never used.
    auto issue = [&](int ci, int bi, int part) {
        const int cj = chunk_of(ci);
        const bool sink = cj < nc_s;
        const int valid = rows_of(cj);
        const int j0 = valid > 0 ? first_row_of(cj) : 0;
        const int8_t* kb = sink ? sk : rk;
        const int8_t* vb = sink ? sv : rv;
        const float* ksb = sink ? sks : rks;
        const float* vsb = sink ? svs : rvs;
        auto row_of = [&](int rr) {  // (selects, no branches: the wait counts stay static)
            const int rs = j0 + (rr < valid ? rr : 0);
            int rg = first_slot + rs;
            rg = rg >= W ? rg - W : rg;
            const int row = sink ? rs : rg;
            return valid > 0 ? row : 0;
        };
        DecBuf<D>& B = sm.buf[wave][bi];
        // part 0: the K rows and K scales, part 1: the V rows and V scales
        // (each tensor's part of a chunk requested back to back measured
        // faster than interleaved K and V pieces)
        {
            const int t = part;
#pragma unroll
            for (int j = 0; j < NKI; ++j) {
                const int rr = j * RPI + lane / CPR;
                const int pc = lane % CPR;
                if (t == 0) {
                    const int lc = pc ^ ((rr >> 1) & (CPR - 1));  // logical piece stored at slot pc
                    dma16_nt(kb, (uint32_t)row_of(rr) * D + 16 * lc, lds_off(&B.k[j * 1024]));
                } else {
                    // (V stays row-major for D = 64: it is read with transposing reads)
                    const int lv = D == 64 ? pc : pc ^ ((rr >> 1) & (CPR - 1));
                    dma16_nt(vb, (uint32_t)row_of(rr) * D + 16 * lv, lds_off(&B.v[j * 1024]));
                }
            }
#pragma unroll
            for (int j = 0; j < GROUPS; ++j) {
                const int f = 64 * j + lane;
                const uint32_t off = (uint32_t)row_of(f / GROUPS) * GROUPS + f % GROUPS;
                if (t == 0) dma4(ksb, off * 4, lds_off(&B.ks[64 * j]));
                else dma4(vsb, off * 4, lds_off(&B.vs[64 * j]));
            }
        }
    };
    // the first chunk now, the rest once q is ready: the first requests of
    // all waves then reach memory ahead of everything else
    issue(wave, 0, 0);
    issue(wave, 0, 1);

    // q of head c as the B operand: 4 channels per instruction, f16 (q and
    // the new token were loaded before the NDMA DMA instructions of chunk 0)
    vm_wait_upto<NDMA>();
#pragma unroll
    for (int j = 0; j < NI / 2; ++j) tie(qraw[j]);
    tie(xk);
    tie(xv);
    tie(xkp);
    tie(xfk);
    tie(xfv);
    // q is scaled by a power of two (per head, exact) that brings its largest
    // magnitude into [2^13, 2^14): the f16 operand then neither overflows nor
    // drops the low bits of small values (bf16 carries 8 significant bits, f16
    // 11).  The factor comes out again through this lane's c_log2.
    uint32_t qmax = 0;
#pragma unroll
    for (int j = 0; j < NI / 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w = live ? qraw[j][e] : 0u;
            qmax = max(qmax, max(w & 0x7fffu, (w >> 16) & 0x7fffu));
        }
    const int qsh = qmax == 0 ? 0 : 140 - (int)(qmax >> 7);  // 2^(e - 127) * 2^(140 - e) = 2^13
    const float c_log2 = __builtin_amdgcn_ldexpf(c_log2_all, -qsh);
    auto q16 = [&](uint32_t bits) { return __builtin_amdgcn_ldexpf(__uint_as_float(bits), qsh); };
    half4_t qb[NI];
    float qbias[GROUPS];
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) qbias[g] = 0.f;
#pragma unroll
    for (int j = 0; j < NI / 2; ++j) {
        const u32x4 w = qraw[j];
        const uint32_t ws[4] = {live ? w[0] : 0u, live ? w[1] : 0u, live ? w[2] : 0u, live ? w[3] : 0u};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const half2_t lo = cvt_pk_f16(q16(ws[2 * h] << 16), q16(ws[2 * h] & 0xffff0000u));
            const half2_t hi = cvt_pk_f16(q16(ws[2 * h + 1] << 16), q16(ws[2 * h + 1] & 0xffff0000u));
            qb[2 * j + h] = half4_t{lo[0], lo[1], hi[0], hi[1]};
            qbias[(8 * j) / 32] += (float)lo[0] + (float)lo[1] + (float)hi[0] + (float)hi[1];
        }
    }
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) qbias[g] *= -kBias;

    // the appended token: lane l quantizes channel l of K and V; its score on
    // head c comes from lane 4b + c over channels 4b .. 4b+3 (the codes of
    // the quad's lanes, whose group scale this lane shares)
    float s_new = kNegInf;  // score of head c (log2 units), uniform per head
    float v_new = 0.f;      // dequantized V of channel `lane`
    int ck = 0, cv = 0;     // its codes and scales (stored into the ring at the end)
    float sck = 0.f, scv = 0.f;
    if (append) {
        ck = quantize_lane(bf16_bits_to_f32((uint16_t)xk), sck);
        cv = quantize_lane(bf16_bits_to_f32((uint16_t)xv), scv);
        v_new = (float)cv * scv;
        if (has_new) {
            // every lane forms the whole dot product of its head's q with the
            // dequantized new key, reading channel ch's value from lane ch
            const float kd = (float)ck * sck;  // dequantized K of channel `lane`
            float d = 0.f;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    d = __builtin_fmaf((float)qb[i][e],
                                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kd), 4 * i + e)), d);
            s_new = d * c_log2;
        }
    }
    SWA_TRACE(0);

    // lane-dependent byte selectors of the quad transpose
    const uint32_t sel1 = (c < 2) ? 0x05040100u : 0x03020706u;
    const uint32_t sel2 = (c & 1) ? 0x03070105u : 0x06020400u;
    const uint32_t swz = (lane >> 1) & (CPR - 1);

    // D = 64: lane l accumulates O of all four heads (reg r = head r) at
    // channel l, in two halves (quads 0-7 and 8-15 of each chunk) that are
    // added at the end.  D = 32: acc[i] holds the per-quad partials of
    // channels 4i + c, summed over the quads at the end.
    constexpr int NACC = D == 64 ? 2 : NI;
    f32x4_t acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // D = 64 transposing V reads: lane l of 16-lane group g names 8 bytes of
    // row 8t + (l % 16) / 2 at channels 16g + 8 (l % 2) .. +7
    const uint32_t vt_lane = 64 * ((lane & 15) >> 1) + 16 * (lane >> 4) + 8 * (lane & 1);
    float m_h[4] = {kNegInf, kNegInf, kNegInf, kNegInf};  // reference max per head (wave-uniform)
    float m_c = kNegInf;                                  // = m_h[c]
    float l_c = 0.f;                                      // row sum of head c (this lane's keys)
    float ws_c[GROUPS];                                   // sum of f16 weights of head c per group
    int ve[GROUPS];                                       // V-scale exponent per group (wave-uniform)
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) {
        ws_c[g] = 0.f;
        ve[g] = kNoExp;
    }

    for (int kk = 0; kk < n_steps; ++kk) {
        const int bi = kk % NBUF;
        const int ci = wave + NW * kk;
        // The K part of this chunk has landed once at most NDMA_PART loads are
        // outstanding (its V part was requested after it).  The two parts are
        // read and refilled separately, so the next chunk's K streams in while
        // this chunk's V arrives and its scores are computed.
        vm_wait_upto<NDMA_PART>();
        SWA_TRACE(1);
        const DecBuf<D>& B = sm.buf[wave][bi];
        const int nvalid = chunk_rows(ci);
        // this lane's row: K and V pieces in logical order
        u32x4 kr[CPR], vr[CPR];
        const uint32_t kbase = lds_off(&B.k[0]) + 16 * CPR * lane;
        const uint32_t vbase = lds_off(&B.v[0]) + 16 * CPR * lane;
#pragma unroll
        for (int m = 0; m < CPR; ++m) kr[m] = lds_load128(kbase + 16 * (m ^ swz));
        // the group scales of the quad's four keys (rows 4b .. 4b+3), [key][group]
        u32x4 ksw[GROUPS], vsw[GROUPS];
        const uint32_t qoff = 16 * GROUPS * (lane >> 2);
#pragma unroll
        for (int g = 0; g < GROUPS; ++g) ksw[g] = lds_load128(lds_off(&B.ks[0]) + qoff + 16 * g);
        SWA_TRACE(2);
        // the K buffers are free again once these reads have completed
        lds_reads_done();
        const bool more = kk + 1 < n_steps;
        if (more) issue(ci + NW, bi, 0);

        // scores: C_g(4b+c, r) = sum over group g of q_c * (1152 + code) - 1152 * sum q_c
        // (the two group chains alternate so consecutive MFMAs are independent)
        f32x4_t s0 = f32x4_t{qbias[0], qbias[0], qbias[0], qbias[0]};
        f32x4_t s1 = f32x4_t{qbias[GROUPS - 1], qbias[GROUPS - 1], qbias[GROUPS - 1], qbias[GROUPS - 1]};
#pragma unroll
        for (int i0 = 0; i0 < 8; ++i0) {
#pragma unroll
            for (int gi = 0; gi < GROUPS; ++gi) {
                const int i = i0 + 8 * gi;
                const uint32_t w = kr[i / 4][i % 4];
                if (gi == 0)
                    s0 = __builtin_amdgcn_mfma_f32_4x4x4f16(codes_to_h4(w), qb[i], s0, 0, 0, 0);
                else
                    s1 = __builtin_amdgcn_mfma_f32_4x4x4f16(codes_to_h4(w), qb[i], s1, 0, 0, 0);
            }
        }
        // per-key scales of the quad's keys: key 4b + r, group g at word r * GROUPS + g
        float ks0[4], vs0[4], ks1[4] = {0.f, 0.f, 0.f, 0.f}, vs1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int w0 = r * GROUPS;
            ks0[r] = __uint_as_float(ksw[w0 / 4][w0 % 4]);
            if (GROUPS > 1) ks1[r] = __uint_as_float(ksw[(w0 + 1) / 4][(w0 + 1) % 4]);
        }
        const int kq = lane & ~3;  // chunk row of the quad's key 0
        float sc[4];
        bool grow = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = s0[r] * ks0[r];
            if (GROUPS > 1) v = __builtin_fmaf(s1[r], ks1[r], v);
            sc[r] = (kq + r < nvalid) ? v * c_log2 : kNegInf;
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
            for (int i = 0; i < NACC; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][r] *= corr[r];
        }
        // weights of head c on the quad's keys
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = (kq + r < nvalid) ? __builtin_amdgcn_exp2f(sc[r] - m_c) : 0.f;
            l_c += p[r];
        }
        // the V part of this chunk: outstanding after it, at most the next K part
        if (more) vm_wait_upto<NDMA_PART>();
        else vm_wait_upto<0>();
        u32x2 vt[8];  // D = 64: read t -> V codes of rows 8t .. 8t+7 at channel `lane`
        if constexpr (D == 64) {
#pragma unroll
            for (int t = 0; t < 8; ++t) vt[t] = lds_load_tr8(lds_off(&B.v[0]) + vt_lane + 512 * t);
        } else {
#pragma unroll
            for (int m = 0; m < CPR; ++m) vr[m] = lds_load128(vbase + 16 * (m ^ swz));
        }
#pragma unroll
        for (int g = 0; g < GROUPS; ++g) vsw[g] = lds_load128(lds_off(&B.vs[0]) + qoff + 16 * g);
        lds_reads_done();
        if (more) issue(ci + NW, bi, 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // rows past the chunk's end carry no weight; their scale words (slots
            // that may never have been written) are not used
            const int w0 = r * GROUPS;
            const bool ok = kq + r < nvalid;
            vs0[r] = ok ? __uint_as_float(vsw[w0 / 4][w0 % 4]) : 0.f;
            if (GROUPS > 1) vs1[r] = ok ? __uint_as_float(vsw[(w0 + 1) / 4][(w0 + 1) % 4]) : 0.f;
        }
        // The weight operand p * s_v is an f16 number: it is formed relative to
        // a power of two 2^ve[g] at least as large as every V scale of group g
        // seen so far (p <= 2^8, so the operand stays below 2^8), and the
        // accumulators are rescaled exactly when a chunk raises ve[g].
        {
            const uint32_t m0 = all_blocks_umax(max(max(__float_as_uint(vs0[0]), __float_as_uint(vs0[1])),
                                                    max(__float_as_uint(vs0[2]), __float_as_uint(vs0[3]))));
            const uint32_t m1 = GROUPS > 1 ? all_blocks_umax(max(max(__float_as_uint(vs1[0]), __float_as_uint(vs1[1])),
                                                                 max(__float_as_uint(vs1[2]), __float_as_uint(vs1[3]))))
                                           : 0u;
            const int e0 = m0 ? (int)(m0 >> 23) - 126 : kNoExp;  // scales < 2^e (finite, non-negative)
            const int e1 = m1 ? (int)(m1 >> 23) - 126 : kNoExp;
            if (e0 > ve[0] || (GROUPS > 1 && e1 > ve[GROUPS - 1])) {
                float f[GROUPS];
                const int en[2] = {max(e0, ve[0]), max(e1, ve[GROUPS - 1])};
#pragma unroll
                for (int g = 0; g < GROUPS; ++g) {
                    f[g] = ve[g] == kNoExp ? 1.f : __builtin_amdgcn_ldexpf(1.f, ve[g] - en[g]);
                    ve[g] = en[g];
                    ws_c[g] *= f[g];
                }
                const float fl = (D == 64 && lane >= 32) ? f[GROUPS - 1] : f[0];
#pragma unroll
                for (int i = 0; i < NACC; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][r] *= fl;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                vs0[r] = __builtin_amdgcn_ldexpf(vs0[r], -ve[0]);
                if (GROUPS > 1) vs1[r] = __builtin_amdgcn_ldexpf(vs1[r], -ve[GROUPS - 1]);
            }
        }
        // ... scaled per V group, as the A operand of P V
        const half2_t a0l = cvt_pk_f16_rne(p[0] * vs0[0], p[1] * vs0[1]);
        const half2_t a0h = cvt_pk_f16_rne(p[2] * vs0[2], p[3] * vs0[3]);
        const half4_t pa0 = half4_t{a0l[0], a0l[1], a0h[0], a0h[1]};
        ws_c[0] = fdot2(__builtin_bit_cast(uint32_t, a0l), 0x3c003c00u, ws_c[0]);
        ws_c[0] = fdot2(__builtin_bit_cast(uint32_t, a0h), 0x3c003c00u, ws_c[0]);
        half4_t pa1 = pa0;
        if (GROUPS > 1) {
            const half2_t a1l = cvt_pk_f16_rne(p[0] * vs1[0], p[1] * vs1[1]);
            const half2_t a1h = cvt_pk_f16_rne(p[2] * vs1[2], p[3] * vs1[3]);
            pa1 = half4_t{a1l[0], a1l[1], a1h[0], a1h[1]};
            ws_c[GROUPS - 1] = fdot2(__builtin_bit_cast(uint32_t, a1l), 0x3c003c00u, ws_c[GROUPS - 1]);
            ws_c[GROUPS - 1] = fdot2(__builtin_bit_cast(uint32_t, a1h), 0x3c003c00u, ws_c[GROUPS - 1]);
        }
        if constexpr (D == 64) {
            // O += P V with blocks = channel quads: block b (lanes 4b..4b+3)
            // computes O[head r][channel 4b + c] over one key quad whose
            // weights every block of its half takes by broadcast (CBSZ = 3:
            // blocks 0-7 read block ABID, blocks 8-15 block 8 + ABID).  The
            // halves need different V group scales, so one lane exchange
            // builds the two A operands: for quads 0-7, lanes 0-31 keep their
            // group-0 weights and lanes 32-63 receive the group-1 weights of
            // lanes 0-31; for quads 8-15 the other way round.
            const u32x2 w0 = __builtin_bit_cast(u32x2, pa0), w1 = __builtin_bit_cast(u32x2, pa1);
            const auto e0 = __builtin_amdgcn_permlane32_swap(w0[0], w1[0], false, false);
            const auto e1 = __builtin_amdgcn_permlane32_swap(w0[1], w1[1], false, false);
            const half4_t a_lo = __builtin_bit_cast(half4_t, make_uint2(e0[0], e1[0]));  // quads 0-7
            const half4_t a_hi = __builtin_bit_cast(half4_t, make_uint2(e0[1], e1[1]));  // quads 8-15
#define SWA_PV(Q)                                                                                          \
    acc[0] = __builtin_amdgcn_mfma_f32_4x4x4f16(a_lo, codes_to_h4(vt[(Q) / 2][(Q) % 2]), acc[0], 3, Q, 0);   \
    acc[1] = __builtin_amdgcn_mfma_f32_4x4x4f16(a_hi, codes_to_h4(vt[4 + (Q) / 2][(Q) % 2]), acc[1], 3, Q, 0);
            SWA_PV(0) SWA_PV(1) SWA_PV(2) SWA_PV(3) SWA_PV(4) SWA_PV(5) SWA_PV(6) SWA_PV(7)
#undef SWA_PV
        } else {
            // O += P V: V codes of the quad's keys at channel 4i + c
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const uint32_t w = vr[i / 4][i % 4];
                const uint32_t t = __builtin_amdgcn_perm(dpp_xor2(w), w, sel1);
                const uint32_t col = __builtin_amdgcn_perm(dpp_xor1(t), t, sel2);
                acc[i] = __builtin_amdgcn_mfma_f32_4x4x4f16(i < 8 ? pa0 : pa1, codes_to_h4(col), acc[i], 0, 0, 0);
            }
        }
        SWA_TRACE(3);
    }
    // every DMA has landed (also unused prologue chunks) before LDS is reused
    // or the wave ends
    vm_wait_upto<0>();

    // D = 32: sum the 16 blocks' partial outputs.  Two halving exchanges
    // (lane bits 5 and 4) leave each lane NJ = NI / 4 channel steps per head;
    // row rotations by 4 and 8 add the four blocks of each 16-lane row.  Lane
    // l then holds the totals of channels 4 i + c with i = j + NJ * (l >> 4).
    // D = 64 needs no reduction: lane l already holds channel l.
    constexpr int NJ = NI / 4;
    float o2[NJ][4];
    if constexpr (D == 64) {
#pragma unroll
        for (int r = 0; r < 4; ++r) o2[0][r] = acc[0][r] + acc[1][r];
    } else {
        float o1[NI / 2][4];
#pragma unroll
        for (int j = 0; j < NI / 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[j][r]),
                                                                __float_as_uint(acc[j + NI / 2][r]), false, false);
                o1[j][r] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(o1[j][r]),
                                                                __float_as_uint(o1[j + NJ][r]), false, false);
                float x = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                x += __int_as_float(
                    __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x124, 0xF, 0xF, false));
                x += __int_as_float(
                    __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x128, 0xF, 0xF, false));
                o2[j][r] = x;
            }
    }
    const float l_tot = all_blocks(l_c);
    float ws_tot[GROUPS];
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) ws_tot[g] = all_blocks(ws_c[g]);

    // the first wave of the kv head stores the new token into its ring slot
    if (append && hs == 0 && sp == 0 && wave == 0 && lane < D) {
        const int slot = pos % W;
        (rk + (size_t)slot * D)[lane] = (int8_t)ck;
        (rv + (size_t)slot * D)[lane] = (int8_t)cv;
        if ((lane & 31) == 0) {
            rks[(size_t)slot * GROUPS + lane / 32] = sck;
            rvs[(size_t)slot * GROUPS + lane / 32] = scv;
        }
    }
    if constexpr (COMP) {
        if (append && hs == 0 && sp == 0 && wave == 0) {
            const int ch = lane % D;
            const int blk = a.block;
            const bool restart = pos % blk == 0;
            const float fk = (restart ? 0.f : __uint_as_float(xfk)) + bf16_bits_to_f32((uint16_t)xkp);
            const float fv = (restart ? 0.f : __uint_as_float(xfv)) + bf16_bits_to_f32((uint16_t)xv);
            if (lane < D) {
                a.front_k[bh * D + ch] = fk;
                a.front_v[bh * D + ch] = fv;
            }
            const int j = pos / blk;
            if (pos % blk == blk - 1 && j < S) {
                // the completed block: mean of its pre-RoPE keys rotated at the
                // block midpoint (rotate-half pairing: channel ch with ch ^ D/2)
                const float mk = fk / (float)blk, mv = fv / (float)blk;
                const float other = __shfl_xor(mk, D / 2, 64);
                float rk = mk;
                if (a.rope_cos) {
                    const int mid = min(j * blk + blk / 2, a.rope_len - 1);
                    const int i = ch % (D / 2);
                    const float cs = a.rope_cos[(size_t)mid * (D / 2) + i], sn = a.rope_sin[(size_t)mid * (D / 2) + i];
                    rk = ch < D / 2 ? __builtin_fmaf(mk, cs, -other * sn) : __builtin_fmaf(mk, cs, other * sn);
                }
                float spk, spv;
                const int cpk = quantize_lane(rk, spk), cpv = quantize_lane(mv, spv);
                const size_t row = bh * S + j;
                if (lane < D) {
                    a.pool_k[row * D + ch] = (int8_t)cpk;
                    a.pool_v[row * D + ch] = (int8_t)cpv;
                    if ((lane & 31) == 0) {
                        a.pool_ks[row * GROUPS + lane / 32] = spk;
                        a.pool_vs[row * GROUPS + lane / 32] = spv;
                    }
                }
            }
        }
    }
    SWA_TRACE(4);

    // Merge of the waves: each leaves its per-head partial in LDS, in final
    // units: (acc - 1152 * sum of f16 weights) * 2^ve[g] over max m_c.
    {
        float ws_r[4][GROUPS];  // the f16 weight sums of each head r (lanes 0..3 hold heads 0..3)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int g = 0; g < GROUPS; ++g)
                ws_r[r][g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ws_tot[g]), r));
        if constexpr (D == 64) {
            const int g = lane >> 5;
            const int e = g ? ve[GROUPS - 1] : ve[0];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sm.part_o(wave)[r * D + lane] =
                    e == kNoExp ? 0.f
                                : __builtin_amdgcn_ldexpf(o2[0][r] - kBias * (g ? ws_r[r][GROUPS - 1] : ws_r[r][0]), e);
        } else {
            const int i_out = (lane >> 2) % NJ;
            const bool writer = ((lane >> 2) & 3) < NJ;
            const int ch = 4 * (i_out + NJ * (lane >> 4)) + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float o = o2[0][r];
#pragma unroll
                for (int j = 1; j < NJ; ++j) o = i_out == j ? o2[j][r] : o;
                o = ve[0] == kNoExp ? 0.f : __builtin_amdgcn_ldexpf(o - kBias * ws_r[r][0], ve[0]);
                if (writer) sm.part_o(wave)[r * D + ch] = o;
            }
        }
        if (lane < 4) {
            sm.part_m[wave][lane] = m_c;
            sm.part_l[wave][lane] = l_tot;
        }
    }
    __syncthreads();
    const float sn[4] = {__int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_new), 0)),
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_new), 1)),
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_new), 2)),
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_new), 3))};
    // One softmax partial (m, l, o) merged with the appended token -> output.
    auto finish = [&](int r, int d, float sr, float vn, float m, float l, float o) {
        const float mm = fmaxf(m, sr);
        float num = 0.f, den = 0.f;
        if (mm != kNegInf) {  // exp2(-inf - mm) is 0 for a finite mm: empty parts drop out
            const float fn = __builtin_amdgcn_exp2f(sr - mm), fo = __builtin_amdgcn_exp2f(m - mm);
            num = fn * vn + fo * o;
            den = fn + fo * l;
        }
        const float val = den > 0.f ? num * __builtin_amdgcn_rcpf(den) : 0.f;
        ((uint16_t*)a.out)[((size_t)b * a.Hq + h0 + r) * D + d] = (uint16_t)f32_to_bf16_bits(val);
    };
    // Partials of split-K, [unit][split][head] (m, l) and [unit][split][head][D] o.
    const size_t pbase = ((size_t)unit * splits) * 4;
    auto st = [](float* p, float v) {
        __hip_atomic_store((uint32_t*)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // (4 * D is a multiple of the block size; with D = 64 each iteration is one
    // head per wave and lane = channel, so the head's merge factors are uniform
    // and the lane's own v_new is the channel's)
    for (int e = tid; e < 4 * D; e += 64 * NW) {
        const int r = e / D, d = e % D;
        const float vn = D == 64 ? v_new : __shfl(v_new, d, 64);  // before any lane leaves the loop body
        float m = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) m = fmaxf(m, sm.part_m[w][r]);
        float o = 0.f, l = 0.f;
        if (m != kNegInf) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = __builtin_amdgcn_exp2f(sm.part_m[w][r] - m);
                o += f * sm.part_o(w)[r * D + d];
                l += f * sm.part_l[w][r];
            }
        }
        if (splits == 1) {
            if (r < nh) finish(r, d, r == 0 ? sn[0] : r == 1 ? sn[1] : r == 2 ? sn[2] : sn[3], vn, m, l, o);
        } else {
            const size_t row = pbase + (size_t)sp * 4 + r;
            st(a.part_o + row * D + d, o);
            if (d == 0) {
                st(a.part_ml + 2 * row, m);
                st(a.part_ml + 2 * row + 1, l);
            }
        }
    }
    if (splits == 1) return;

    // Split-K combine: the last workgroup of the unit to finish merges every
    // split's partial (in split order, so the result does not depend on which
    // workgroup is last) and sets the unit's counter back to zero.
    // The L2 caches of the XCDs are not coherent with one another, and a
    // device-scope fence writes back and invalidates a whole L2: done by
    // every workgroup, that costs more than the walk itself.  So the partials
    // travel only through device-scope atomic stores and loads, which write
    // through and read past the L2, and the ordering is made explicit: every
    // store of the workgroup has completed before its arrival is counted, and
    // the last workgroup reads only after its count came back.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
        const int prev = __hip_atomic_fetch_add(a.counters + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.last = prev == splits - 1;
    }
    __syncthreads();
    if (!sm.last) return;
    auto ld = [](const float* p) {
        return __uint_as_float(__hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    };
    for (int e = tid; e < 4 * D; e += 64 * NW) {
        const int r = e / D, d = e % D;
        const float vn = D == 64 ? v_new : __shfl(v_new, d, 64);
        if (r >= nh) continue;
        // the partials in batches of 8 splits whose loads are in flight
        // together, each batch merged into the running (m, l, o)
        float m = kNegInf, o = 0.f, l = 0.f;
        for (int q0 = 0; q0 < splits; q0 += 8) {
            float mq[8], lq[8], oq[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const size_t row = pbase + (size_t)min(q0 + j, splits - 1) * 4 + r;
                mq[j] = ld(a.part_ml + 2 * row);
                lq[j] = ld(a.part_ml + 2 * row + 1);
                oq[j] = ld(a.part_o + row * D + d);
            }
            float mb = m;
#pragma unroll
            for (int j = 0; j < 8; ++j) mb = q0 + j < splits ? fmaxf(mb, mq[j]) : mb;
            if (mb != kNegInf) {  // (exp2 of -inf is 0: empty partials drop out)
                const float f = __builtin_amdgcn_exp2f(m - mb);
                o *= f;
                l *= f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float fj = q0 + j < splits ? __builtin_amdgcn_exp2f(mq[j] - mb) : 0.f;
                    o += fj * oq[j];
                    l += fj * lq[j];
                }
                m = mb;
            }
        }
        finish(r, d, r == 0 ? sn[0] : r == 1 ? sn[1] : r == 2 ? sn[2] : sn[3], vn, m, l, o);
    }
    if (tid == 0) __hip_atomic_store(a.counters + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    SWA_TRACE(5);
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t s) {
    const int G = a.Hq / a.Hkv;
    const long long nblocks = (long long)a.B * a.Hkv * ((G + 3) / 4) * a.num_splits;
    if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const bool wide = decode_waves(a.B, a.Hq, a.Hkv) == 8;
    if (a.block > 0) {
        if (wide) hipLaunchKernelGGL((decode_kernel<D, 8, true>), dim3((unsigned)nblocks), dim3(512), 0, s, a);
        else hipLaunchKernelGGL((decode_kernel<D, 2, true>), dim3((unsigned)nblocks), dim3(128), 0, s, a);
    } else {
        if (wide) hipLaunchKernelGGL((decode_kernel<D, 8, false>), dim3((unsigned)nblocks), dim3(512), 0, s, a);
        else hipLaunchKernelGGL((decode_kernel<D, 2, false>), dim3((unsigned)nblocks), dim3(128), 0, s, a);
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

// ---- split-K state without caller memory --------------------------------
// For callers that cannot allocate (HIP graph capture, tight serving loops):
// the split-K counters and partials live in this file-scope device array, one
// copy per GPU, held until the process ends.  Every call on a GPU shares it,
// so calls that overlap in time on one GPU race.  Its counters are zero at
// load time, are cleared once more by the first call on each device, and
// every completed call leaves them zero again.
namespace {
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ void zero_words_kernel(uint32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}
}  // namespace

hipError_t launch_decode_noalloc(DecodeArgs a, const DecodeWorkspace& wl, hipStream_t s) {
    if (wl.total > kNoAllocScratchBytes) return hipErrorInvalidValue;
    char* base = nullptr;
    if (wl.total > 0) {
        int dev = -1;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (g_scratch_ptr[dev] == nullptr) {
            // this device's copy of the array: its address, taken once with the
            // device current (the array's host-side name is not an address)
            void* ptr = nullptr;
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, s, (uint32_t*)ptr,
                               kNoAllocScratchBytes / sizeof(uint32_t));
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            g_scratch_ptr[dev] = ptr;
        }
        base = (char*)g_scratch_ptr[dev];
        a.counters = (int*)(base + wl.counters);
        a.part_ml = (float*)(base + wl.part_ml);
        a.part_o = (float*)(base + wl.part_o);
    }
    return launch_decode(a, s);
}

}  // namespace swa
