// swa_internal.h -- kernel argument blocks and launchers behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swa_common.h"

namespace swa {

// Division by a divisor fixed at launch: q = (mulhi(n, mul) + n) >> shift with
// shift = ceil(log2 d) and mul = floor(2^32 (2^shift - d) / d) + 1, exact for
// every n < 2^31 (the round-up multiply-and-shift method of Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994).
struct FastDiv {
    uint32_t d, mul, shift;
};
inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    f.shift = 0;
    while ((1ull << f.shift) < d) ++f.shift;
    f.mul = (uint32_t)((((1ull << 32) * ((1ull << f.shift) - d)) / d) + 1);
    return f;
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    return (__umulhi(n, f.mul) + n) >> f.shift;
}

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* pk;  // pooled keys (compressed mode)
    const void* pv;
    const int32_t* seg;
    const uint8_t* prefix;
    // key metadata of a bf16 plain prefill with segment ids or sink flags
    // (all NULL otherwise), written by the prep pass:
    const int32_t* kinfo;  // [B][T] packed key info (segment | sink << 31)
    const int32_t* ksub;   // [B][2 * ntile][4] KeySum of each 32-key sub-tile
    const int32_t* tsink;  // [B][ntile][2] segment range of each 64-key tile's sinks
    int ntile;             // ceil(T / 64)
    const float* rope_cos;
    const float* rope_sin;
    void* out;
    float* lse;
    int B, Hq, Hkv, T, D;
    int window;
    int block;  // compress block, 0 = plain
    int nblk;   // T / block
    int rope_len;
    float scale;
    // workgroup geometry of the MFMA kernel: heads per workgroup and 32-row
    // blocks per workgroup (hpw * rbs waves)
    int hpw, rbs;
    // divisors of the bf16 kernel's workgroup numbering (set by its launcher):
    // query blocks, head groups per batch row (Hkv * G / hpw), head groups per
    // kv head (G / hpw), hpw, and the compress block
    FastDiv div_nqb, div_hg, div_groups, div_hpw, div_block;
};

// Geometry the bf16 MFMA kernel uses for a given GQA group size: 4 waves per
// workgroup, hpw heads (the largest divisor of G that is at most 4) times rbs
// 32-row blocks (hpw * rbs = 4).  With G >= 4 every wave of a workgroup has
// the same rows, hence the same mask and the same amount of work.
constexpr int kMfmaWaves = 4;
struct MfmaGeom {
    int hpw, rbs;
};
inline MfmaGeom mfma_geometry(int G) {
    MfmaGeom g;
    g.hpw = G >= 4 ? 4 : G;
    while (G % g.hpw) --g.hpw;
    g.rbs = kMfmaWaves / g.hpw;
    return g;
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_debug_visibility(const PrefillArgs& a, bool mfma_geometry, uint8_t* mask, int32_t* count,
                                   hipStream_t s);
hipError_t launch_rope_table(double theta, int rope_len, int D, float* c, float* sn, hipStream_t s);
hipError_t launch_pool_rope(int B, int H, int T, int D, int block, int dtype, const void* k_pre,
                            const void* v, const float* c, const float* sn, int rope_len, void* pk,
                            void* pv, hipStream_t s);
// Arguments of the bf16 prep pass (key rotation and key metadata in one
// launch); either part may be empty (rope_blocks == 0, or info == NULL).
struct PrepArgs {
    long long rope_blocks;  // ceil(rope_rows * D / 16 / 256)
    long long rope_rows;    // B * Hkv * T
    int B, T, D, ntile;
    FastDiv div_T;          // T, for rows * D / 16 < 2^31 (else 64-bit indexing)
    const uint16_t* x;  // keys to rotate [rope_rows, D]
    const float* cs;
    const float* sn;
    uint16_t* y;  // rotated keys
    const int32_t* seg;
    const uint8_t* prefix;
    int32_t* info;  // [B][T]
    int32_t* ksub;  // [B][2 * ntile][4]
    int32_t* tsink; // [B][ntile][2]
};
hipError_t launch_prefill_prep(const PrepArgs& p, hipStream_t s);
hipError_t launch_rope_rows_f32(long long rows, int T, int D, const float* x, const float* cs, const float* sn,
                                float* y, hipStream_t s);
hipError_t launch_kv_quantize(long long N, int D, const void* x, int8_t* xq, float* xs, hipStream_t s);

struct DecodeArgs {
    const void* q;
    const void* k_new;
    const void* v_new;
    int8_t* ring_k;
    int8_t* ring_v;
    float* ring_ks;
    float* ring_vs;
    const int8_t* sink_k;
    const int8_t* sink_v;
    const float* sink_ks;
    const float* sink_vs;
    const int32_t* pos;
    const int32_t* sink_len;
    void* out;
    float* partial;  // workspace for split-K partials (num_splits > 1)
    int B, Hq, Hkv, D, W, S;
    int num_splits;
    float scale;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

}  // namespace swa
