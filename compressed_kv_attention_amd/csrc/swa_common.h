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

}  // namespace swa
