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
    // Split sources (bf16 kernel only; zero and null otherwise): the query
    // rows start at q_first, so q, out and lse hold rows q_first .. T - 1 of
    // each head; with k2 set, key rows from kv_split on come from k2 / v2,
    // which hold rows kv_split .. T - 1 of each kv head.  Both are multiples
    // of 64.
    int q_first = 0;
    int kv_split = 0;
    const void* k2 = nullptr;
    const void* v2 = nullptr;
};

// Geometry the bf16 MFMA kernel uses for a given GQA group size: 4 waves per
// workgroup, hpw heads (the largest divisor of G that is at most 4) times rbs
// 64-row blocks (hpw * rbs = 4).  With G >= 4 every wave of a workgroup has
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
// The bf16 kernel's own visibility: the same walk and masks, written out as
// mask [B, T, Tk] (zeroed first; may be null) and count [B, T].
hipError_t launch_prefill_bf16_dump(const PrefillArgs& a, uint8_t* mask, int32_t* count, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_debug_visibility(const PrefillArgs& a, bool mfma_geometry, uint8_t* mask, int32_t* count,
                                   hipStream_t s);
hipError_t launch_rope_table(double theta, int rope_len, int D, float* c, float* sn, hipStream_t s);
hipError_t launch_pool_rope(int B, int H, int T, int D, int block, int dtype, const void* k_pre,
                            const void* v, const float* c, const float* sn, int rope_len, void* pk,
                            void* pv, hipStream_t s);
// The fused pre-pass of a compressed bf16 prefill with RoPE: rotated exact
// keys and the pooled keys (rotated at their block midpoints) and values from
// one read of k and v.  Blocks of up to 256 / (D / 16) rows (pool_rotate_fits).
struct PoolRotArgs {
    int N, T, D, block, nblk, rope_len;
    int span;     // rows per workgroup (whole blocks; set by the launcher)
    float inv_b;  // 1 / block when a power of two, else 0 (set by the launcher)
    const uint16_t* k;
    const uint16_t* v;
    const float* cs;
    const float* sn;
    uint16_t* kr;  // rotated keys [N, T, D]
    uint16_t* pk;  // [N, nblk, D]
    uint16_t* pv;
};
bool pool_rotate_fits(int D, int block);
hipError_t launch_pool_rotate_bf16(PoolRotArgs p, hipStream_t s);
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
    // split-K state (num_splits > 1), in the caller's workspace: one arrival
    // counter per (batch row, kv head, group of 4 query heads) -- zero between
    // calls -- and each split's softmax partials: (m, l) and o[D] per head
    int* counters;
    float* part_ml;
    float* part_o;
    int B, Hq, Hkv, D, W, S;
    int num_splits;  // >= 1 (the entry point resolves 0 = automatic)
    float scale;
    // Compressed mode (block > 0): the sink arrays are the pooled-block cache
    // (capacity S rows, written through pool_* when a block completes),
    // k_pre [B][Hkv][D] bf16 is the appended key before rotation, front_k /
    // front_v [B][Hkv][D] fp32 hold the running sums of the block in progress,
    // and rope_cos / rope_sin [rope_len][D/2] (or NULL: no rotation) rotate a
    // pooled key at its block midpoint.
    int block;
    const void* k_pre;
    float* front_k;
    float* front_v;
    int8_t* pool_k;
    int8_t* pool_v;
    float* pool_ks;
    float* pool_vs;
    const float* rope_cos;
    const float* rope_sin;
    int rope_len;
};
// Workspace of a decode with `splits` parts: [counters][partial m, l][partial o],
// each part 256-byte aligned; 0 bytes when splits == 1.
struct DecodeWorkspace {
    size_t counters, part_ml, part_o, total;
};
inline DecodeWorkspace decode_workspace_layout(int B, int Hq, int Hkv, int D, int splits) {
    DecodeWorkspace w{0, 0, 0, 0};
    if (splits <= 1 || B <= 0 || Hkv <= 0) return w;
    auto r256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t units = (size_t)B * Hkv * ((Hq / Hkv + 3) / 4);
    w.counters = 0;
    w.part_ml = r256(units * sizeof(int));
    w.part_o = w.part_ml + r256(units * splits * 4 * 2 * sizeof(float));
    w.total = w.part_o + r256(units * splits * 4 * (size_t)D * sizeof(float));
    return w;
}
// Waves per decode workgroup.  A batch with at least 512 (batch row, kv head,
// group of 4 query heads) units fills the chip with two-wave workgroups, each
// wave walking every other 64-row chunk.  Smaller batches take eight waves
// per workgroup, so a unit's chunks are walked side by side instead of one
// after another and its waves merge through LDS.
inline int decode_waves(int B, int Hq, int Hkv) {
    const long long units = (long long)B * Hkv * ((Hq / Hkv + 3) / 4);
    return units >= 512 ? 2 : 8;
}
// Split count the library picks for num_splits == 0: one, unless a unit's
// walk would leave its eight waves more than two chunks each; then enough
// splits for two chunks per wave, within 1024 workgroups.  (A split-K
// combine costs about four dependent memory round trips, more than the walk
// of two chunks.)
inline int decode_auto_splits(int B, int Hq, int Hkv, int W, int S) {
    const long long units = (long long)B * Hkv * ((Hq / Hkv + 3) / 4);
    if (units <= 0 || decode_waves(B, Hq, Hkv) != 8) return 1;
    const long long chunks = ((long long)S + W + 63) / 64;
    long long s = (chunks + 15) / 16;
    const long long max_by_grid = 1024 / units;
    if (s > max_by_grid) s = max_by_grid;
    return (int)(s < 1 ? 1 : s);
}
constexpr int kMaxDecodeSplits = 256;

// Backward of the plain-mode prefill: the caller's tensors and the fp32
// staging (q and k rotated when a table is given, dO, and Delta = rowsum(dO o)).
struct BwdArgs {
    const void* q;     // [B][Hq][T][D], dtype
    const void* k;     // [B][Hkv][T][D], dtype
    const void* v;
    const void* out;   // [B][Hq][T][D], dtype (the forward's output)
    const void* dout;  // [B][Hq][T][D], dtype
    const float* lse;  // [B][Hq][T] (the forward's row log-sum-exp)
    const int32_t* seg;
    const uint8_t* prefix;
    const float* rope_cos;  // [T][D/2] or NULL
    const float* rope_sin;
    float* dq;  // [B][Hq][T][D]
    float* dk;  // [B][Hkv][T][D]
    float* dv;
    int B, Hq, Hkv, T, D, window;
    int dtype;  // 0 fp32, 1 bf16
    float scale;
};
struct BwdWorkspace {
    float* q32;
    float* k32;
    float* v32;
    float* do32;
    float* delta;
    float* pk;  // per-query-head dk / dv shares [B][Hq][T][D] (GQA groups of more than one head)
    float* pv;
};
hipError_t launch_prefill_backward(const BwdArgs& a, const BwdWorkspace& w, hipStream_t s);

// NSA selection branch: the caller's tensors (q, k, v before RoPE).
struct NsaArgs {
    const void* q;  // [B][Hq][T][D], dtype
    const void* k;  // [B][Hkv][T][D], dtype
    const void* v;
    const float* rope_cos;  // [rope_len][D/2] or NULL
    const float* rope_sin;
    void* out;       // [B][Hq][T][D], dtype
    float* lse;      // [B][Hq][T] or NULL
    int32_t* sel;    // [B][Hq][T][n_select] or NULL
    int B, Hq, Hkv, T, D, window, block, nblk, n_select, rope_len;
    int dtype;  // 0 fp32, 1 bf16
    float scale;
};
// Preparation (the exact keys rotated, in the input dtype, when a table is
// given; fp32 pooled keys) and the selection kernel; krot [B][Hkv][T][D],
// pk32 [B][Hkv][nblk][D].
hipError_t launch_nsa_select(const NsaArgs& a, void* krot, float* pk32, hipStream_t s);

// Chunked prefill: the caller's tensors and the staged sequence length
// Tv = S + W - 1 + Tc (sink rows, ring rows before the chunk, the chunk).
struct ChunkArgs {
    const void* q;  // [B][Hq][Tc][D] bf16
    const void* k;  // [B][Hkv][Tc][D] bf16
    const void* v;
    int8_t* ring_k;
    int8_t* ring_v;
    float* ring_ks;
    float* ring_vs;
    const int8_t* sink_k;
    const int8_t* sink_v;
    const float* sink_ks;
    const float* sink_vs;
    const int32_t* pos0;
    const int32_t* sink_len;
    void* out;  // [B][Hq][Tc][D] bf16
    int B, Hq, Hkv, D, W, S, Tc;
    int C;   // cached rows of the key sequence: S + W - 1 rounded up to 64
    int Tv;  // C + Tc
    // the prefill's key metadata of the Tv keys (as its pre-pass writes it)
    int32_t* info;
    int32_t* ksub;
    int32_t* tsink;
    int ntile;  // ceil(Tv / 64)
};
// Stage the cached rows of K/V (sink and ring rows dequantized, padding zero),
// the segment and prefix arrays of the whole key sequence and the prefill's
// key metadata of it.
hipError_t launch_chunk_stage(const ChunkArgs& a, void* k_stage, void* v_stage, int32_t* seg, uint8_t* prefix,
                              hipStream_t s);
// Quantize the chunk's last min(W, Tc) tokens into the ring.
hipError_t launch_chunk_finish(const ChunkArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// Largest split-K state swa_attn_decode_noalloc holds (its device array).
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
// The decode launch with the split-K state in the library's device array
// instead of caller memory; fails with hipErrorInvalidValue when wl.total
// exceeds kNoAllocScratchBytes.
hipError_t launch_decode_noalloc(DecodeArgs a, const DecodeWorkspace& wl, hipStream_t s);

}  // namespace swa
