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

}  // namespace swa
