// swa_common.h -- small device helpers shared by the gfx950 kernels of libswa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

constexpr int kMaxT = 131072;      // longest sequence the prefill kernels accept
constexpr int kDebugMaxT = 16384;  // longest sequence swa_debug_visibility accepts

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Wave64 butterfly reductions (all lanes get the result).
__device__ __forceinline__ float wave_max_xor(float v, int first, int last) {
    for (int o = first; o <= last; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Symmetric absmax/127 quantization of one 32-channel group held by 32
// consecutive lanes (one element per lane), the int8 cache layout that the
// budget formula of [NW] "How the 256-Token Sliding Window Works with Tools
// as KV Sinks in Needle" ("Effective KV Window") prices: scale = amax / 127
// in fp32, code = round-half-even(x / scale) clamped to +-127, a zero group
// gives scale 0 and codes 0.  Returns the code; `s` receives the group scale.
__device__ __forceinline__ int quantize_lane(float x, float& s) {
    float amax = fabsf(x);
    amax = wave_max_xor(amax, 1, 16);
    s = amax / 127.0f;
    if (s == 0.0f) return 0;
    float r = rintf(x / s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}
__device__ __forceinline__ int wave_imin_xor(int v, int first, int last) {
    for (int o = first; o <= last; o <<= 1) v = min(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ int wave_imax_xor(int v, int first, int last) {
    for (int o = first; o <= last; o <<= 1) v = max(v, __shfl_xor(v, o, 64));
    return v;
}

// Whole-wave min / max without LDS: DPP steps within each row of 16 lanes
// (xor 1, xor 2, rotate 4, rotate 8), then the row-pair and half-wave swaps.
// Every lane gets the result.
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int x) {
    return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
}
template <bool MAX>
__device__ __forceinline__ int wave_reduce_i32(int x) {
    auto op = [](int u, int v) { return MAX ? max(u, v) : min(u, v); };
    x = op(x, dpp_i32<0xB1>(x));
    x = op(x, dpp_i32<0x4E>(x));
    x = op(x, dpp_i32<0x124>(x));
    x = op(x, dpp_i32<0x128>(x));
    const auto s16 = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    x = op((int)s16[0], (int)s16[1]);
    const auto s32 = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return op((int)s32[0], (int)s32[1]);
}
__device__ __forceinline__ int wave_min_i32(int x) { return wave_reduce_i32<false>(x); }
__device__ __forceinline__ int wave_max_i32(int x) { return wave_reduce_i32<true>(x); }

// ---- LDS staging ---------------------------------------------------------
// Cache and key tiles move global -> LDS by direct loads issued from inline
// asm, which the compiler does not see: seen, they would make it wait for
// every load in flight before any LDS read (it cannot tell buffers apart).
// A wave waits for its own direct loads with an explicit vmcnt wait.  Every
// LDS read is an ordinary load that the compiler schedules, waits for and
// orders against the matrix instructions under its own hazard rules.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// LDS byte address of a pointer into __shared__ memory (device pass only; the
// host pass never runs device functions).
__device__ __forceinline__ uint32_t lds_off(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(uint32_t, (__attribute__((address_space(3))) const char*)p);
#else
    (void)p;
    return 0u;
#endif
}
__device__ __forceinline__ u32x4 lds_load128(uint32_t addr) {
#if defined(__HIP_DEVICE_COMPILE__)
    return *__builtin_bit_cast(__attribute__((address_space(3))) const u32x4*, addr);
#else
    (void)addr;
    return u32x4{};
#endif
}
// ds_read_b64_tr_b16: in each 16-lane group, lane j gets element j of the
// four 16-bit rows the group's lanes address (row i from lanes 4i..4i+3).
__device__ __forceinline__ u32x2 lds_load_tr16(uint32_t addr) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(__builtin_bit_cast(__attribute__((address_space(3))) s16x4*, addr)));
#else
    (void)addr;
    return u32x2{};
#endif
}
// ds_read_b64_tr_b8: in each 16-lane group, lanes 2r and 2r+1 each name 8
// bytes that together form row r (16 bytes) of an 8 x 16 byte matrix; lane j
// gets column j (rows 0..7, one byte each, row 0 in the lowest byte).
__device__ __forceinline__ u32x2 lds_load_tr8(uint32_t addr) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(__builtin_bit_cast(__attribute__((address_space(3))) i32x2*, addr)));
#else
    (void)addr;
    return u32x2{};
#endif
}
// Direct global -> LDS loads: lane l's 16 (or 4) bytes at base + voff land at
// LDS byte lds + 16 l (or 4 l).  base and lds must be wave-uniform.  M0 holds
// the LDS address; the compiler reserves M0 and does not keep values in it
// across these statements in the kernels here (none of their own code reads
// M0, which a host test checks on the generated assembly).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// (readfirstlane makes the uniformity explicit, so the operands always get
// scalar registers; it costs nothing on values already held in them)
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t u = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (const void*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(uniform_ptr(base)),
                 "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}
// The same with the non-temporal hint, for data that one launch reads once
// (a decode step's cache rows): they need not displace reused lines.
__device__ __forceinline__ void dma16_nt(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(uniform_ptr(base)),
                 "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(uniform_ptr(base)),
                 "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}
#pragma clang diagnostic pop
// All LDS reads issued so far have completed (before a direct load may
// overwrite what they read); the compiler sees the wait.
__device__ __forceinline__ void lds_reads_done() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited for
    asm volatile("" ::: "memory");
}
// Wait until at most N of this wave's vector-memory loads are outstanding
// (direct loads included).  A compiler barrier for memory accesses: no LDS
// read moves above it.
template <int N>
__device__ __forceinline__ void vm_wait_upto() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace swa
