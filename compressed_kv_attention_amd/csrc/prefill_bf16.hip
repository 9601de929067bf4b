// prefill_bf16.hip -- bf16 prefill attention on gfx950 MFMA.
//
// Computes softmax attention under the packing & causal & (recent | sink)
// mask of [NW] "How the 256-Token Sliding Window Works with Tools as KV Sinks
// in Needle" (section "KV Sinks for Tools: Pinning Critical Context"), and the
// compressed-column variant of [CA] "Compressed attention and the copy probe"
// (sections "Two kinds of columns, pooled blocks and exact recent keys" and
// "Pool before rotating, not after").
//
// Work decomposition.  A workgroup of 4 waves owns one (batch, kv head) pair
// and 32 * rbs query rows for hpw query heads of that kv head's GQA group
// (hpw * rbs = 4); each wave owns 32 rows of one head.  The heads of a group
// share every K/V tile staged in LDS.  Workgroups are numbered so that each XCD
// (and its L2) gets a contiguous run of query blocks of the same (batch, kv
// head), which read overlapping key tiles.
//
// Staging.  Key tiles of 64 keys go from global memory straight into LDS
// (global_load_lds, 16 bytes per lane, no registers), two buffers deep: while
// tile t is computed, tile t+1 is in flight.  K and V are stored row-major
// with an XOR swizzle of their 16-byte chunks chosen so that the MFMA operand
// reads hit distinct banks; V is read column-wise with ds_read_b64_tr_b16.
// With RoPE, q is rotated here as it is loaded; the keys arrive already
// rotated (the library rotates them once, in a pre-pass).
//
// Per tile each wave works on two 32-key sub-tiles:
//   S^T = K Q^T      4 x v_mfma_f32_32x32x16_bf16 (keys are the M rows)
//   online softmax   per query = per lane column, so the running max, sum
//                    and rescale are lane-local (one xor-32 exchange for max);
//                    the output is rescaled only when a row max grows by more
//                    than 2^8 (the stale max is used consistently otherwise)
//   O^T += V^T P^T   2 x 2 MFMAs; P^T comes straight from the S^T registers
// Sub-tiles the mask hides completely are skipped, sub-tiles it shows
// completely skip the element predicate (swa_tiles.h).
//
// DUMP instantiations run the same walk, sub-tile classification, lane gate
// and masks, but write the pairs they would let through (and each row's
// visible count) instead of computing attention: the tests check this
// kernel's own mask bit for bit.
#include "swa_common.h"
#include "swa_internal.h"
#include "swa_tiles.h"

// Optional phase-time accounting for profiling builds; no code in normal builds.
#ifndef SWA_TRACE_DECL
#define SWA_TRACE_DECL
#define SWA_TRACE(slot)
#endif

namespace swa {
namespace {

constexpr int BN = 64;   // keys per LDS tile
constexpr int SUB = 32;  // keys per MFMA sub-tile
constexpr int NBUF = 2;  // LDS tile buffers: the tile computed and the next one
constexpr int kSinkWords = (kMaxT / BN + 31) / 32;
constexpr float kRescaleSum = 256.0f;  // the reference max moves when a weight sum passes 2^8

// Wait for all of this wave's global loads (direct-to-LDS ones included) and
// LDS accesses, then the workgroup barrier.  The wait is the builtin, not asm,
// so that the compiler knows every earlier load has completed and inserts no
// wait of its own on the tiles in flight later.
__device__ __forceinline__ void wait_all_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int D>
struct SmemBf16 {
    uint16_t k[NBUF][BN * D];     // K tiles, row-major, 16-byte chunks swizzled
    uint16_t v[NBUF][BN * D];     // V tiles, row-major, 16-byte chunks swizzled
    int kinfo[NBUF][BN];          // packed segment | sink << 31 of the tile's keys
    int ksum[NBUF][BN / SUB][4];  // KeySum of each sub-tile (from the prep pass)
    uint32_t sink_bits[kSinkWords];
};

// Swizzled position (in 16-byte chunks) of chunk c of key row k.  K: rows that
// share LDS banks get different chunk orders, so the 32 rows one MFMA operand
// read touches are conflict free.  V: the four rows one transpose read covers
// per half-wave fall into different bank halves.  Both swizzles depend only on
// the low bits of k, so rows 32 apart differ by a constant offset.
template <int D>
__device__ __forceinline__ int k_chunk(int k, int c) {
    constexpr int CPR = D / 8;  // chunks per row
    return k * CPR + (c ^ ((k * CPR / 16) % CPR));
}
template <int D>
__device__ __forceinline__ int v_chunk(int k, int c) {
    constexpr int CPR = D / 8;
    return k * CPR + (D == 64 ? (c ^ (((k >> 1) & 1) * 4)) : c);
}

// Per-lane byte offsets, within a key tile, of the rows and chunks this
// lane's wave moves: wave w issues loads ld = w, w + kMfmaWaves, ...; load ld
// covers key rows [ld * ROWS, ld * ROWS + ROWS) and lane l moves 16 bytes of
// row ld * ROWS + l / CPR.  The lane writes LDS chunk ld * 64 + l; it picks the
// logical chunk whose swizzled position that is.
template <int D>
struct TileLoads {
    static constexpr int CPR = D / 8;                       // 16-byte chunks per row
    static constexpr int ROWS = 64 / CPR;                   // key rows per wave instruction
    static constexpr int LOADS = BN / ROWS / kMfmaWaves;    // instructions per wave per tile
    // Offsets of the wave's first load; load i sits i * kMfmaWaves * ROWS rows
    // further (a multiple of 32 rows, which keeps the swizzle unchanged).
    uint32_t koff, voff;
    __device__ __forceinline__ void init(int wave, int lane) {
        const int kr = wave * ROWS + lane / CPR;
        const int pc = lane % CPR;
        const int ck = pc ^ ((kr * CPR / 16) % CPR);
        const int cv = D == 64 ? (pc ^ (((kr >> 1) & 1) * 4)) : pc;
        koff = (uint32_t)(kr * D + 8 * ck) * 2;
        voff = (uint32_t)(kr * D + 8 * cv) * 2;
        static_assert((kMfmaWaves * ROWS) % 32 == 0 || LOADS == 1, "swizzle period");
    }
};

// The wave that stages the sub-tile summaries (wave 0 stages the key info).
constexpr int kMetaWave = 1 % kMfmaWaves;

// Per-wave base addresses of the (batch row, kv head) a workgroup works on,
// computed once: each tile then only adds its offset.
struct TileBases {
    const char* k;      // exact keys: row 0 of this head
    const char* v;
    const char* k2;     // split keys: row kv_split of this head (or null)
    const char* v2;
    const char* pk;     // pooled keys (compressed mode)
    const char* pv;
    const char* info;   // packed key info of this batch row (or null)
    const char* ksub;   // sub-tile summaries of this batch row
};
template <int D, bool SPLIT>
__device__ __forceinline__ TileBases tile_bases(const PrefillArgs& a, int b, int hkv) {
    TileBases t;
    const size_t head = (size_t)b * a.Hkv + hkv;
    const size_t t1 = (size_t)(SPLIT ? a.kv_split : a.T);  // rows per head of the first source
    t.k = (const char*)((const uint16_t*)a.k + head * t1 * D);
    t.v = (const char*)((const uint16_t*)a.v + head * t1 * D);
    const size_t t2 = (size_t)(a.T - a.kv_split);
    t.k2 = SPLIT ? (const char*)((const uint16_t*)a.k2 + head * t2 * D) : nullptr;
    t.v2 = SPLIT ? (const char*)((const uint16_t*)a.v2 + head * t2 * D) : nullptr;
    t.pk = a.pk ? (const char*)((const uint16_t*)a.pk + head * (size_t)a.nblk * D) : nullptr;
    t.pv = a.pv ? (const char*)((const uint16_t*)a.pv + head * (size_t)a.nblk * D) : nullptr;
    t.info = a.kinfo ? (const char*)(a.kinfo + (size_t)b * a.T) : nullptr;
    t.ksub = a.ksub ? (const char*)(a.ksub + (size_t)b * 2 * a.ntile * 4) : nullptr;
    return t;
}

// Issue the global->LDS loads of one tile into buffer `buf`: wave w moves
// 1 KB of K and 1 KB of V (64 lanes x 16 bytes) per instruction; with key
// metadata, wave 0 also moves the keys' packed info and kMetaWave the two
// sub-tile summaries.  Rows past the last key load the last key's row
// (finite data, masked later).
template <int D, bool DUMP, bool SPLIT>
__device__ __forceinline__ void issue_tile(const PrefillArgs& a, const TileBases& tb, SmemBf16<D>& sm, uint32_t koff,
                                           uint32_t voff, int buf, int kind, int tile, int wave, int lane) {
    using TL = TileLoads<D>;
    constexpr uint32_t kStep = kMfmaWaves * TL::ROWS * D * 2;  // bytes between a wave's loads
    const bool pooled = kind == COL_POOLED;
    const int nkeys = pooled ? a.nblk : a.T;
    const int k0 = tile * BN;
    // uniform base pointers (the tile's first row) plus 32-bit per-lane offsets
    const size_t toff = (size_t)k0 * D * 2;
    const char* kb = (pooled ? tb.pk : tb.k) + toff;
    const char* vb = (pooled ? tb.pv : tb.v) + toff;
    if (SPLIT && !pooled && k0 >= a.kv_split) {  // a tile of the second source (kv_split is a multiple of BN)
        const size_t off2 = (size_t)(k0 - a.kv_split) * D * 2;
        kb = tb.k2 + off2;
        vb = tb.v2 + off2;
    }
    if (DUMP) {
        // the mask alone: no K or V (the visibility dump is given no tensors)
    } else if (k0 + BN <= nkeys) {
#pragma unroll
        for (int i = 0; i < TL::LOADS; ++i) {
            const int ld = wave + kMfmaWaves * i;
            dma16(kb, koff + i * kStep, lds_off(&sm.k[buf][ld * 64 * 8]));
            dma16(vb, voff + i * kStep, lds_off(&sm.v[buf][ld * 64 * 8]));
        }
    } else {  // the last tile: rows past the end repeat the last key
#pragma unroll
        for (int i = 0; i < TL::LOADS; ++i) {
            const int ld = wave + kMfmaWaves * i;
            const int kr = ld * TL::ROWS + lane / TL::CPR;
            const uint32_t back = (uint32_t)(kr - min(kr, nkeys - 1 - k0)) * D * 2;
            dma16(kb, koff + i * kStep - back, lds_off(&sm.k[buf][ld * 64 * 8]));
            dma16(vb, voff + i * kStep - back, lds_off(&sm.v[buf][ld * 64 * 8]));
        }
    }
    if (!pooled && tb.info) {
        if (wave == 0) {
            const uint32_t gk = (uint32_t)min(k0 + lane, a.T - 1);
            dma4(tb.info, gk * 4, lds_off(&sm.kinfo[buf][0]));
        }
        if (wave == kMetaWave && lane < 2 * 4)
            dma4(tb.ksub, (uint32_t)(2 * tile * 4 + lane) * 4, lds_off(&sm.ksum[buf][0][0]));
    }
}

// RoPE table rows q0 .. q0 + 31 (clamped to the table) of cos and of sin,
// staged by direct loads into the second V buffer as [2][32][D/2] floats
// (exactly that buffer's 128 D bytes): when every wave of a workgroup rotates
// the same 32 query rows, the workgroup reads their table rows once.  The
// buffer is free until the walk's second tile is issued into it.
template <int D>
__device__ __forceinline__ void issue_rope_rows(const PrefillArgs& a, SmemBf16<D>& sm, int q0, int wave, int lane) {
    constexpr int PPR = D / 8;               // 16-byte pieces per table row (D/2 floats)
    constexpr int NI = 2 * 32 * PPR / 64;    // 1 KB instructions for both tables
    static_assert(NI * 1024 == (int)sizeof(sm.v[1]), "table rows fill the second V buffer");
    const uint32_t dst = lds_off(&sm.v[1][0]);
    for (int i = wave; i < NI; i += kMfmaWaves) {
        const int id = (i % (NI / 2)) * 64 + lane;  // piece within one table's 32 rows
        const int row = min(q0 + id / PPR, a.rope_len - 1);
        dma16(i < NI / 2 ? (const void*)a.rope_cos : (const void*)a.rope_sin,
              (uint32_t)(row * (D / 2) * 4 + (id % PPR) * 16), dst + i * 1024);
    }
}

__device__ __forceinline__ int lds_load32(uint32_t addr) {
#if defined(__HIP_DEVICE_COMPILE__)
    return *__builtin_bit_cast(__attribute__((address_space(3))) const int*, addr);
#else
    (void)addr;
    return 0;
#endif
}
__device__ __forceinline__ void lds_store64(uint32_t addr, u32x2 v) {
#if defined(__HIP_DEVICE_COMPILE__)
    *__builtin_bit_cast(__attribute__((address_space(3))) u32x2*, addr) = v;
#else
    (void)addr;
    (void)v;
#endif
}

__device__ __forceinline__ void unpack8(const uint4& x, float* f) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint4 pack8(const float* f) {
    uint4 r;
    r.x = cvt_pk_bf16(f[0], f[1]);
    r.y = cvt_pk_bf16(f[2], f[3]);
    r.z = cvt_pk_bf16(f[4], f[5]);
    r.w = cvt_pk_bf16(f[6], f[7]);
    return r;
}

// Rotate-half RoPE of 8 channel pairs: x1 holds channels d..d+7 (< D/2), x2
// holds d+D/2..d+D/2+7; c/s hold the table entries of channels d..d+7.  The
// rotated values are multiplied by `mul` before their one rounding to bf16.
__device__ __forceinline__ void rotate8(uint4& x1, uint4& x2, const float4& c0, const float4& c1, const float4& s0,
                                        const float4& s1, float mul) {
    float a[8], bb[8];
    unpack8(x1, a);
    unpack8(x2, bb);
    const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    float y1[8], y2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        y1[i] = (a[i] * c[i] - bb[i] * s[i]) * mul;
        y2[i] = (bb[i] * c[i] + a[i] * s[i]) * mul;
    }
    x1 = pack8(y1);
    x2 = pack8(y2);
}

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

// V^T operand of O^T += V^T P^T for keys [kb, kb + 16) of a tile
// sub-tile and channels [32n, 32n + 32): lane (channel d = l % 32, half h)
// needs the 8 keys 16m + 4h + {0..3} and 16m + 8 + 4h + {0..3} of channel d.
// Two transpose reads (hi = 0, 1): within each 16-lane group, source lane
// j = 4r + a points at key K_r, channels base + 4a .. +3; output lane 4a' + b'
// then holds channel base + lane%16 of keys K_0..K_3.  This is the lane's byte
// offset for kb = 0; keys kb (a multiple of 16) sit kb * D * 2 bytes further.
template <int D>
__device__ __forceinline__ uint32_t vt_lane_off(int n, int hi, int lane) {
    const int g = lane >> 4;  // 16-lane group
    const int h = g >> 1;     // keys half
    const int j = lane & 15;
    const int r = j >> 2, a4 = j & 3;
    const int ch = 32 * n + 16 * (g & 1) + 4 * a4;  // first channel this source lane points at
    const int c = ch >> 3, half = (ch >> 2) & 1;
    return (uint32_t)(v_chunk<D>(8 * hi + 4 * h + r, c) * 16 + 8 * half);
}
// K operand of S^T = K Q^T, chunk c (channels 16c + 8h .. +7) of key lq of a
// sub-tile at keys [0, 32); sub-tile st sits st * SUB * D * 2 bytes further.
template <int D>
__device__ __forceinline__ uint32_t k_lane_off(int c, int lane) {
    return (uint32_t)(k_chunk<D>(lane & 31, 2 * c + (lane >> 5)) * 16);
}


struct DumpOut {
    uint8_t* mask;   // [B, T, Tk] visibility (zeroed by the launcher), or null
    int32_t* count;  // [B, T] visible columns per row
};

template <int D, bool ROPE, bool COMPRESSED, bool DUMP, bool SPLIT>
__global__ __launch_bounds__(64 * kMfmaWaves) __attribute__((amdgpu_waves_per_eu(4, 8))) void prefill_bf16_kernel(
    PrefillArgs a, DumpOut dump) {
    static_assert(D == 32 || D == 64, "head dim");
    __shared__ __align__(16) SmemBf16<D> sm;
    SWA_TRACE_DECL
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int lq = lane & 31;

    const int T = a.T;
    const int G = (int)a.div_groups.d * a.hpw;  // GQA group size
    const int wg_rows = 32 * a.rbs;
    // XCD-aware numbering: dispatch sends workgroup i to XCD i % 8; give each
    // XCD a contiguous range of logical blocks (query block fastest).
    const int nblocks = gridDim.x;
    int lb = blockIdx.x;
    if ((nblocks & 7) == 0) lb = (blockIdx.x & 7) * (nblocks >> 3) + (blockIdx.x >> 3);
    const int bh = (int)fdiv((uint32_t)lb, a.div_nqb);  // batch row * head groups + head group
    // The dispatcher fills an XCD's 32 CUs one workgroup each in turn, so a CU
    // receives blocks 32 apart in this numbering.  Reversing the query-block
    // order of every other run of max(32, nqb) blocks pairs late query blocks
    // (costly: more keys visible) with early ones on every CU; the decision is
    // taken per (batch row, head group), so the map stays one to one.
    const int nqb = (int)a.div_nqb.d;
    int qb = lb - bh * nqb;
    const int run = nqb >= 32 ? bh : (bh * nqb) >> 5;  // run of the group's first block
    if (run & 1) qb = nqb - 1 - qb;
    const int b = (int)fdiv((uint32_t)bh, a.div_hg);
    const int hg = bh - b * (int)a.div_hg.d;
    const int hkv = (int)fdiv((uint32_t)hg, a.div_groups);
    const int hsub = hg - hkv * (int)a.div_groups.d;
    const int q_first = SPLIT ? a.q_first : 0;
    const int q0 = q_first + qb * wg_rows;
    const int q1 = min(q0 + wg_rows - 1, T - 1);
    const int wrb = (int)fdiv((uint32_t)wave, a.div_hpw);  // row block of this wave
    const int my_h = hkv * G + hsub * a.hpw + (wave - wrb * a.hpw);
    const int r0 = q0 + 32 * wrb;
    const bool wave_active = wave < a.hpw * a.rbs && r0 < T;
    const int my_q = r0 + lq;
    const bool row_ok = my_q < T;
    // q, out and lse hold rows q_first .. T - 1 of each head
    const int Tq = T - q_first;
    const size_t qhead = ((size_t)b * a.Hq + my_h) * Tq;
    constexpr bool plain = !COMPRESSED;
    // scale * log2 e, folded into q (one rounding of q to bf16)
    const float c_log2 = a.scale * kLog2e;

    // Tile plan.  The band comes first in the walk, so the first tile's loads
    // start at once; every global load of the prologue is issued before any of
    // them is waited for.
    const TilePlan plan = plan_tiles(q0, q1, a.window, a.block, a.nblk, a.prefix != nullptr, BN);
    TileIter it;
    it.init(plan, sm.sink_bits, BN);
    int kc = 0, tc = 0;  // tile being computed
    const bool have0 = it.next(kc, tc);
    SWA_TRACE(11);
    // The rows' segment ids and the sink-tile summaries first (the first
    // values the prologue waits for), then the tile, table and q loads.  The
    // loads are unconditional, from clamped addresses, with the values
    // selected afterwards: a load under a divergent branch is waited for where
    // the branch ends.  (Sink tiles before the band: tiles whose sinks belong
    // to a segment of the workgroup's rows; the prep pass gives each tile's
    // sink segment range, and every wave loads the rows' segment ids, at most
    // 128 rows, itself.)
    // (each branch only loads into a variable given its default before it, so
    // that no value is waited for until it is used)
    const int32_t* seg_row = a.seg ? a.seg + (size_t)b * T : nullptr;
    int seg_ld = 1;
    if (seg_row) seg_ld = seg_row[min(my_q, T - 1)];
    const int n_sink_tiles = plan.sink_keys / BN;
    const bool scan = n_sink_tiles > 0;
    int s0v = 1, s1v = 1;
    int2 tv = make_int2(0x7fffffff, (int)0x80000000);
    if (scan) {
        if (seg_row) {
            s0v = seg_row[min(q0 + lane, q1)];
            s1v = seg_row[min(q0 + 64 + lane, q1)];
        }
        tv = *(const int2*)(a.tsink + ((size_t)b * a.ntile + min(lane, n_sink_tiles - 1)) * 2);
    }
    TileLoads<D> tl;
    tl.init(wave, lane);
    const TileBases tb = tile_bases<D, SPLIT>(a, b, hkv);
    if (have0) issue_tile<D, DUMP, SPLIT>(a, tb, sm, tl.koff, tl.voff, 0, kc, tc, wave, lane);
    // one 32-row block per workgroup: the table rows go through LDS, once
    const bool tab_lds = ROPE && a.rbs == 1;
    if (tab_lds) issue_rope_rows<D>(a, sm, q0, wave, lane);
    SWA_TRACE(6);

    // q.  Without the table rows in LDS, the wave's 32 rows come by direct
    // loads into its quarter of K/V buffer 1 (free until the walk's second
    // tile): whole rows per instruction, the 16-byte chunks of row r stored
    // XOR-swizzled by r so that the operand reads below (a row per lane) spread
    // over the banks.  With the table rows there, each lane reads its own.
    constexpr int QCPR = D / 8;       // 16-byte chunks per q row
    constexpr int QRPI = 64 / QCPR;   // q rows per direct-load instruction
    const bool q_lds = !DUMP && !tab_lds;
    const uint32_t q_lds_base =
        lds_off(wave < 2 ? &sm.k[1][0] : &sm.v[1][0]) + (uint32_t)(wave & 1) * 32u * D * 2u;
    uint4 raw[D / 16];
    if (q_lds) {
        if (wave_active) {
            const void* qbase = (const uint16_t*)a.q + (qhead + (r0 - q_first)) * D;
#pragma unroll
            for (int i = 0; i < 32 / QRPI; ++i) {
                const int r = i * QRPI + lane / QCPR, pc = lane % QCPR;
                const int rr = min(r, T - 1 - r0);  // rows past the end repeat the last row
                // (non-temporal: each q row is read by this workgroup alone)
                dma16_nt(qbase, (uint32_t)(rr * D * 2 + (pc ^ (r % QCPR)) * 16), q_lds_base + 1024u * i);
            }
        }
#pragma unroll
        for (int c = 0; c < D / 16; ++c) raw[c] = make_uint4(0, 0, 0, 0);
    } else {
        const uint16_t* qrow = (const uint16_t*)a.q + (qhead + (row_ok ? my_q - q_first : 0)) * D;
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
            raw[c] = (!DUMP && row_ok) ? *(const uint4*)(qrow + 16 * c + 8 * h) : make_uint4(0, 0, 0, 0);
    }
    float4 rc[D / 32][2], rsn[D / 32][2];
    if (ROPE && !tab_lds && row_ok) {
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
            const int d0 = 16 * c + 8 * h;
            const float* cs = a.rope_cos + (size_t)my_q * (D / 2) + d0;
            const float* sn = a.rope_sin + (size_t)my_q * (D / 2) + d0;
            rc[c][0] = *(const float4*)cs;
            rc[c][1] = *(const float4*)(cs + 4);
            rsn[c][0] = *(const float4*)sn;
            rsn[c][1] = *(const float4*)(sn + 4);
        }
    }
    const int seg_q = row_ok ? seg_ld : 0;


    SWA_TRACE(7);
    const bool row_vis = row_ok && (!plain || seg_q > 0);  // padding rows see nothing
    const unsigned wlim = window_limit(a.window);
    RowSum rs;
    rs.r0 = r0;
    rs.r1 = min(r0 + 31, T - 1);
    rs.smin = __builtin_amdgcn_readfirstlane(wave_min_i32(row_ok ? seg_q : 0x7fffffff));
    rs.smax = __builtin_amdgcn_readfirstlane(wave_max_i32(row_ok ? seg_q : (int)0x80000000));
    // every row of the wave lies in segment rs.smin or rs.smax (or is padding)
    const bool two_seg =
        __builtin_amdgcn_ballot_w64(row_ok && seg_q > 0 && seg_q != rs.smin && seg_q != rs.smax) == 0;

    int n_sink_sel = 0;  // sink tiles the walk visits
    if (scan) {
        const int rseg0 = q0 + lane <= q1 ? s0v : 0x7fffffff;
        const int rseg1 = q0 + 64 + lane <= q1 ? s1v : 0x7fffffff;
        int2 tsk = lane < n_sink_tiles ? tv : make_int2(0x7fffffff, (int)0x80000000);
        const int lo = max(1, wave_min_i32(min(rseg0, rseg1)));
        const int hi = wave_max_i32(max(rseg0 == 0x7fffffff ? (int)0x80000000 : rseg0,
                                         rseg1 == 0x7fffffff ? (int)0x80000000 : rseg1));
        for (int t0 = 0; t0 < n_sink_tiles; t0 += 64) {
            if (t0 > 0) {
                tsk = make_int2(0x7fffffff, (int)0x80000000);
                if (t0 + lane < n_sink_tiles) tsk = *(const int2*)(a.tsink + ((size_t)b * a.ntile + t0 + lane) * 2);
            }
            const uint64_t hit = __ballot(tsk.x <= hi && tsk.y >= lo);
            n_sink_sel += __builtin_popcountll(hit);
            if (wave == 0 && lane == 0) {
                sm.sink_bits[t0 / 32] = (uint32_t)hit;
                if (t0 / 32 + 1 < kSinkWords) sm.sink_bits[t0 / 32 + 1] = (uint32_t)(hit >> 32);
            }
        }
    }
    SWA_TRACE(8);
    // Reference max, in the units of the scaled scores u = s * scale * log2 e
    // (q carries the factor): weights are exp2(u - base).  base is 0 and
    // m_set false until a row's first visible sub-tile sets it.  nbase holds
    // -base in all 16 places for rows that see anything (-inf for rows that
    // see nothing): the initial accumulator of fully visible sub-tiles, so
    // the MFMA itself leaves u - base and the exponent reads it directly.
    float base = 0.f;
    bool m_set = false;
    float l_run = 0.f;
    f32x16 nbase;
#pragma unroll
    for (int j = 0; j < 16; ++j) nbase[j] = row_vis ? -0.f : kNegInf;
    // (kept in 16 registers: the compiler would otherwise hold one value and
    // copy it into 16 registers before every fully visible sub-tile)
    asm volatile("" : "+v"(nbase));
    f32x16 o[D / 32];
#pragma unroll
    for (int n = 0; n < D / 32; ++n) o[n] = f32x16{};
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t ones2 = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);

    // Workgroups with more tiles to walk than a plain window band issue first
    // on their SIMDs: when every workgroup is resident at once, the call
    // ends with its longest walks (query blocks that see a sink prefix or
    // many pooled blocks), and the lighter ones beside them can wait.
    {
        const int n_band = plan.band_hi >= plan.band_lo ? plan.band_hi - plan.band_lo + 1 : 0;
        const int n_walk = n_band + plan.n_pooled + n_sink_sel;
        const int n_typ = a.window > 0 ? (wg_rows + a.window - 1 + BN - 1) / BN + 1 : 0;
        const int extra = a.window > 0 ? n_walk - n_typ : 0;
        if (extra >= 3) __builtin_amdgcn_s_setprio(3);
        else if (extra == 2) __builtin_amdgcn_s_setprio(2);
        else if (extra == 1) __builtin_amdgcn_s_setprio(1);
    }
    // tile 0 (and the staged table rows) must have landed
    wait_all_barrier();
    if (q_lds) {
        // the wave's q rows (row lq, chunks 2c + h), then the K/V buffer 1 is
        // free again once every wave has read its rows
        if (wave_active && row_ok) {
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
                raw[c] = __builtin_bit_cast(
                    uint4, lds_load128(q_lds_base + (uint32_t)(lq * QCPR + ((2 * c + h) ^ (lq % QCPR))) * 16u));
            if (ROPE) {
#pragma unroll
                for (int c = 0; c < D / 32; ++c)
                    rotate8(raw[c], raw[c + D / 32], rc[c][0], rc[c][1], rsn[c][0], rsn[c][1], c_log2);
            }
        }
        lds_reads_done();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
    if (tab_lds) {
        const uint32_t tab = lds_off(&sm.v[1][0]);
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
            const uint32_t o = (uint32_t)(lq * (D / 2) + 16 * c + 8 * h) * 4;
            const u32x4 c0 = lds_load128(tab + o), c1 = lds_load128(tab + o + 16);
            const u32x4 s0 = lds_load128(tab + 64 * D + o), s1 = lds_load128(tab + 64 * D + o + 16);
            rc[c][0] = __builtin_bit_cast(float4, c0);
            rc[c][1] = __builtin_bit_cast(float4, c1);
            rsn[c][0] = __builtin_bit_cast(float4, s0);
            rsn[c][1] = __builtin_bit_cast(float4, s1);
        }
        if (row_ok) {
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
                rotate8(raw[c], raw[c + D / 32], rc[c][0], rc[c][1], rsn[c][0], rsn[c][1], c_log2);
        }
        // every wave has read the rows before the walk's second tile overwrites them
        lds_reads_done();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
    // without RoPE q is scaled here (with RoPE, by the rotation)
    if (!ROPE && !DUMP) {
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            float f[8];
            unpack8(raw[c], f);
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] *= c_log2;
            raw[c] = pack8(f);
        }
    }
    // Q^T operand: lane holds row my_q, channels 16c + 8h .. +7 for each c.
    bf16x8 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qf[c] = __builtin_bit_cast(bf16x8, raw[c]);
    SWA_TRACE(0);

    // LDS addresses of the operand reads in the buffer being computed; they
    // move by +-kTileBytes from one tile to the next.
    constexpr uint32_t kTileBytes = BN * D * 2;
    uint32_t k_addr[D / 16], v_addr[D / 32][2];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) k_addr[c] = lds_off(&sm.k[0][0]) + k_lane_off<D>(c, lane);
#pragma unroll
    for (int n = 0; n < D / 32; ++n) {
        v_addr[n][0] = lds_off(&sm.v[0][0]) + vt_lane_off<D>(n, 0, lane);
        v_addr[n][1] = lds_off(&sm.v[0][0]) + vt_lane_off<D>(n, 1, lane);
    }
    int buf_step = (int)kTileBytes;
    const uint32_t info_lds = lds_off(&sm.kinfo[0][0]);
    // Fast classification of exact sub-tiles: a sub-tile starting at key k0
    // is FULL for this wave when its keys all lie in the segment every row of
    // the wave belongs to (fast_seg; -2 when the rows are not all in one real
    // segment) and either fpos_lo <= k0 <= fpos_hi (every pair causal and
    // inside the window) or every key is a sink and k0 <= fpos_hi (every pair
    // causal; sinks stay visible at any distance).
    const int fpos_lo = a.window != 0 ? max(rs.r1 - a.window + 1, 0) : 0;
    const int fpos_hi = rs.r0 - (SUB - 1);
    const int fast_seg = !plain ? 1 : (rs.smin == rs.smax && rs.smin > 0 ? rs.smin : -2);
    const bool fpos_any = fpos_hi >= fpos_lo;
    const uint32_t sum_lds = lds_off(&sm.ksum[0][0][0]);
    int cnt = 0;  // DUMP: visible columns of this lane's row (its key half)
    const bool dump_writer = DUMP && hkv == 0 && (my_h % G) == 0 && dump.mask != nullptr;
    const int Tk = COMPRESSED ? a.nblk + T : T;
    int cur = 0;
    bool have = have0;
    while (have) {
        // the next tile loads into the other buffer (free since the last barrier)
        const int nxt = cur ^ 1;
        int kn = 0, tn = 0;
        const bool have_next = it.next(kn, tn);
        if (have_next) issue_tile<D, DUMP, SPLIT>(a, tb, sm, tl.koff, tl.voff, nxt, kn, tn, wave, lane);
        SWA_TRACE(1);

        if (wave_active) {
            const bool pooled = COMPRESSED && kc == COL_POOLED;
            const int nkeys = pooled ? a.nblk : T;
            int cls_st[BN / SUB];
            bool gate_st[BN / SUB];
            // sub-tile summaries (staged with the tile); without key metadata
            // every key is in segment 1 and none is a sink
            KeySum ks_cur[BN / SUB];
#pragma unroll
            for (int st = 0; st < BN / SUB; ++st) ks_cur[st] = make_key_sum(true, 1, false, false);
            if (!pooled && a.ksub) {
#pragma unroll
                for (int st = 0; st < BN / SUB; ++st) {
                    const u32x4 kv = lds_load128(sum_lds + (cur * (BN / SUB) + st) * 16);
                    ks_cur[st].smin = __builtin_amdgcn_readfirstlane((int)kv[0]);
                    ks_cur[st].smax = __builtin_amdgcn_readfirstlane((int)kv[1]);
                    ks_cur[st].any_sink = __builtin_amdgcn_readfirstlane((int)kv[2]);
                    ks_cur[st].all_sink = __builtin_amdgcn_readfirstlane((int)kv[3]);
                }
            }
#pragma unroll
            for (int st = 0; st < BN / SUB; ++st) {
                const int k0 = tc * BN + st * SUB;
                int cls;
                unsigned wl = wlim;
                const KeySum& ks = ks_cur[st];
                // (fully visible by the fast test or as pooled blocks: then every
                // row that sees anything sees every key, and the lane gate is the
                // row's own visibility, already in nbase)
                bool splat = false;
                if (pooled) {
                    cls = classify_pooled(rs, k0, SUB, a.window, a.block, a.nblk);
                    splat = cls == TILE_FULL;
                } else if ((!plain || (ks.smin == ks.smax && ks.smin > 0 &&
                                       (ks.smin == fast_seg || (two_seg && (ks.smin == rs.smin || ks.smin == rs.smax))))) &&
                           ((fpos_any && (unsigned)(k0 - fpos_lo) <= (unsigned)(fpos_hi - fpos_lo)) ||
                            (plain && ks.all_sink != 0 && k0 <= fpos_hi))) {
                    // (rows of a two-segment wave that are not in the keys'
                    // segment are left out by the lane gate)
                    cls = TILE_FULL;
                    splat = !plain || ks.smin == fast_seg;
                } else {
                    cls = classify_exact(rs, ks, k0, SUB, nkeys, a.window, plain, wl);
                }
                cls = __builtin_amdgcn_readfirstlane(cls);
                wl = __builtin_amdgcn_readfirstlane(wl);
                cls_st[st] = cls;
                if (cls == TILE_SKIP) continue;
                // Rows outside the sub-tile's segment (and padding rows) take no
                // weight from it: their max ignores it and their exponent base
                // is +inf, so every weight is exactly 0.
                gate_st[st] =
                    (pooled || cls == TILE_PARTIAL) ? row_vis : lane_gate(row_vis, plain, seg_q, ks);

                // Element j of the score block holds key k0 + off(j) + 4h with
                // off(j) = 8(j/4) + j%4.  The mask enters as the accumulator's
                // initial value: 0 where the pair is visible, -inf where it is not.
                const int kb = k0 + 4 * h;  // key of element 0
                // The accumulator's initial value: -base where the pair is visible
                // (and the row passes the lane gate), -inf where it is not.
                const bool gate = gate_st[st];
                auto make_bias = [&]() {
                    const uint32_t nb = __float_as_uint(-base);
                    f32x16 bias;
                    if (cls == TILE_FULL) {
                        // every pair of the sub-tile, for the rows the lane gate lets through
                        const float v = gate ? __uint_as_float(nb) : kNegInf;
#pragma unroll
                        for (int j = 0; j < 16; ++j) bias[j] = v;
                    } else if (cls == TILE_PARTIAL_POS) {
                        // Element j is visible iff its key offset off(j) lies in
                        // [d0 - wl + 1, d0]: a mask over offsets 0..31, then one
                        // bit extract and one bit select per element.
                        const int d0 = my_q - kb;
                        // (bounds past 2^20 act as no bound: |d0| stays far below it)
                        const int lo = max(d0 + 1 - (int)min(wl, 1u << 20), 0);
                        const int hi = min(d0, 31);
                        uint32_t vis = 0u;
                        if (hi >= lo && gate) vis = (hi == 31 ? 0xffffffffu : (2u << hi) - 1u) & ~((1u << lo) - 1u);
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)vis, 8 * (j >> 2) + (j & 3), 1);
                            bias[j] = __uint_as_float((m & nb) | (~m & 0xff800000u));
                        }
                    } else if (pooled) {
                        // pooled blocks visible to this row (recomputed here, where
                        // it is rarely needed, rather than held in a register)
                        int plim = my_q - a.window + 1;
                        asm volatile("" : "+v"(plim));  // keep it here, not hoisted
                        const int pooled_n =
                            plim < a.block ? 0 : min((int)fdiv((uint32_t)plim, a.div_block), a.nblk);
                        const int lim = row_vis ? pooled_n - kb : -1;
#pragma unroll
                        for (int j = 0; j < 16; ++j)
                            bias[j] = (8 * (j >> 2) + (j & 3)) < lim ? __uint_as_float(nb) : kNegInf;
                    } else if (!plain) {
                        // (unreachable: exact keys of the compressed variant are
                        // never PARTIAL, having neither segments nor sinks)
#pragma unroll
                        for (int j = 0; j < 16; ++j) bias[j] = kNegInf;
                    } else if (two_seg) {
                        // The wave's rows lie in at most two segments (rs.smin,
                        // rs.smax): a ballot over the sub-tile's 32 key infos
                        // gives the keys of each segment and the sink keys as
                        // bit masks over key offsets; the row then takes
                        // (its segment) & ((causal & in window) | (causal & sink)).
                        const int kinf = lds_load32(info_lds + (uint32_t)(cur * BN + st * SUB + lq) * 4u);
                        const int kseg = kinf & 0x7fffffff;
                        const uint32_t m_lo = (uint32_t)__builtin_amdgcn_ballot_w64(kseg == rs.smin);
                        const uint32_t m_hi = (uint32_t)__builtin_amdgcn_ballot_w64(kseg == rs.smax);
                        const uint32_t m_sink = (uint32_t)__builtin_amdgcn_ballot_w64(kinf < 0);
                        const uint32_t m_seg = seg_q == rs.smin ? m_lo : m_hi;
                        // offsets relative to kb = k0 + 4h; causal: off <= d0,
                        // window: off >= d0 + 1 - wlim (bounds past 2^20 act as none)
                        const int d0 = my_q - kb;
                        const int hi = min(d0, 31);
                        const int lo = max(d0 + 1 - (int)min(wlim, 1u << 20), 0);
                        const uint32_t causal = hi < 0 ? 0u : (hi == 31 ? 0xffffffffu : (2u << hi) - 1u);
                        const uint32_t recent = lo > 31 ? 0u : causal & ~((1u << lo) - 1u);
                        uint32_t vis = (m_seg >> (4 * h)) & (recent | ((m_sink >> (4 * h)) & causal));
                        vis = row_vis ? vis : 0u;
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)vis, 8 * (j >> 2) + (j & 3), 1);
                            bias[j] = __uint_as_float((m & nb) | (~m & 0xff800000u));
                        }
                    } else {
                        const int d0 = my_q - kb;
                        u32x4 inf[4];
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4)
                            inf[g4] = lds_load128(info_lds + cur * BN * 4 + (st * SUB + 8 * g4 + 4 * h) * 4);
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const bool vis =
                                    row_vis & visible_full(d0 - (8 * g4 + r), wlim, (int)inf[g4][r], seg_q);
                                bias[4 * g4 + r] = vis ? __uint_as_float(nb) : kNegInf;
                            }
                        }
                    }
                    return bias;
                };
                if constexpr (DUMP) {
                    // the pairs this sub-tile lets through for this row: its
                    // mask, where the lane gate lets the row take weight at all
                    // (the mask is formed by every lane: it may take ballots)
                    const f32x16 bias = splat ? nbase : make_bias();
                    if (!gate_st[st]) continue;
                    uint8_t* mrow = dump_writer ? dump.mask + ((size_t)b * T + my_q) * Tk : nullptr;
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = kb + 8 * (j >> 2) + (j & 3);
                        if (bias[j] != kNegInf && key < nkeys) {
                            ++cnt;
                            if (mrow) mrow[(COMPRESSED && !pooled ? a.nblk : 0) + key] = 1;
                        }
                    }
                    continue;
                }

                u32x4 kr[D / 16];
#pragma unroll
                for (int c = 0; c < D / 16; ++c) kr[c] = lds_load128(k_addr[c] + st * SUB * D * 2);
                // sacc = u - base (visible pairs) or -inf
                f32x16 sacc;
                if (splat)
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kr[0]), qf[0], nbase, 0, 0,
                                                                   0);
                else
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kr[0]), qf[0], make_bias(),
                                                                   0, 0, 0);
#pragma unroll
                for (int c = 1; c < D / 16; ++c)
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kr[c]), qf[c], sacc, 0, 0,
                                                                   0);
                // Largest sacc of the row over both key halves (-inf where the row
                // sees nothing of this sub-tile).
                auto sub_max = [&]() {
                    // (compiler-generated max: sacc holds MFMA results, and only the
                    // compiler inserts the wait a VALU read of them needs)
                    float mx = sacc[0];
#pragma unroll
                    for (int j = 1; j < 16; ++j) mx = __builtin_fmaxf(mx, sacc[j]);
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false,
                                                                     false);
                    return __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                };
                // Raise each row's reference by the sub-tile's excess over it (the
                // whole max for a row's first visible sub-tile), rescaling what has
                // been accumulated and the sub-tile's scores against the new one.
                auto raise_base = [&]() {
                    const float mx = sub_max();
                    const float up = mx == kNegInf ? 0.f : (m_set ? __builtin_fmaxf(mx, 0.f) : mx);
                    const float corr = m_set ? __builtin_amdgcn_exp2f(-up) : 1.f;
                    m_set = m_set || mx != kNegInf;
                    base += up;
                    l_run *= corr;
#pragma unroll
                    for (int n = 0; n < D / 32; ++n) o[n] *= corr;
#pragma unroll
                    for (int j = 0; j < 16; ++j) sacc[j] -= up;
#pragma unroll
                    for (int j = 0; j < 16; ++j) nbase[j] = row_vis ? -base : kNegInf;
                    asm volatile("" : "+v"(nbase));
                };
                // bf16 weights exp2(u - base) and the sum of exactly those weights
                // over this lane's keys (hidden pairs give exactly 0).
                uint32_t pw[8];
                auto weights = [&]() {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        pw[i] = cvt_pk_bf16(__builtin_amdgcn_exp2f(sacc[2 * i]), __builtin_amdgcn_exp2f(sacc[2 * i + 1]));
                    float ps = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[i]), ones2, ps, false);
                    return ps;
                };
                // Rows with no reference yet take this sub-tile's max.
                if (__builtin_amdgcn_ballot_w64(gate && !m_set) != 0) raise_base();
                float psum = weights();
                // The reference is lazy: it moves only when some row's scores
                // outgrow it by more than 2^8.  Any weight above 2^8 lifts its
                // lane's sum above 2^8, so the sum is the test; the rare case
                // recomputes the weights against the true max.
                if (__builtin_amdgcn_ballot_w64(psum > kRescaleSum) != 0) {
                    raise_base();
                    psum = weights();
                }
                l_run += psum;
                // V^T operands of the sub-tile's 32 keys
                u32x2 vlo[2][D / 32], vhi[2][D / 32];
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int n = 0; n < D / 32; ++n) {
                        vlo[m][n] = lds_load_tr16(v_addr[n][0] + (st * SUB + 16 * m) * D * 2);
                        vhi[m][n] = lds_load_tr16(v_addr[n][1] + (st * SUB + 16 * m) * D * 2);
                    }
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    u32x4 vw[D / 32];
#pragma unroll
                    for (int n = 0; n < D / 32; ++n) {
                        vw[n] = u32x4{vlo[m][n][0], vlo[m][n][1], vhi[m][n][0], vhi[m][n][1]};
                    }
                    const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pw[4 * m], pw[4 * m + 1], pw[4 * m + 2],
                                                                            pw[4 * m + 3]));
#pragma unroll
                    for (int n = 0; n < D / 32; ++n)
                        o[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw[n]), pb, o[n], 0,
                                                                       0, 0);
                }
            }
        }
        SWA_TRACE(2);

        // tile `nxt` must have landed before the barrier
        wait_all_barrier();
        SWA_TRACE(4);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) k_addr[c] += buf_step;
#pragma unroll
        for (int n = 0; n < D / 32; ++n) {
            v_addr[n][0] += buf_step;
            v_addr[n][1] += buf_step;
        }
        buf_step = -buf_step;
        cur = nxt;
        kc = kn;
        tc = tn;

        have = have_next;
    }

    if (!wave_active) return;
    if constexpr (DUMP) {
        if (hkv == 0 && (my_h % G) == 0 && dump.count != nullptr) {
            const int tot = cnt + __shfl_xor(cnt, 32, 64);
            if (row_ok && h == 0) dump.count[(size_t)b * T + my_q] = tot;
        }
        return;
    }
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    // The output block of the wave (32 rows x D) goes through LDS (the wave's
    // own 64 D bytes of the K buffers, free after the walk) so that it reaches
    // global memory in whole rows: each store instruction then writes
    // 64 x 16 contiguous bytes (1024 / 2D rows) instead of 16 bytes of each of
    // 32 rows.  In LDS, rows are row-major with their 16-byte chunks XOR-swizzled
    // by the row, so both the writes (a lane per row) and the reads (a row per
    // group of D / 8 lanes) spread over the banks.
    {
        constexpr int CPR = D / 8;  // 16-byte chunks per row
        const float inv = (row_ok && l_tot > 0.f) ? 1.f / l_tot : 0.f;
        const uint32_t ob = lds_off(&sm.k[0][0]) + (uint32_t)wave * 32u * D * 2u;
#pragma unroll
        for (int n = 0; n < D / 32; ++n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 4 * n + i;  // chunk of channels 32n + 8i .. +7; this lane has +4h .. +3
                u32x2 w;
                w[0] = cvt_pk_bf16(o[n][4 * i] * inv, o[n][4 * i + 1] * inv);
                w[1] = cvt_pk_bf16(o[n][4 * i + 2] * inv, o[n][4 * i + 3] * inv);
                lds_store64(ob + (uint32_t)(lq * CPR + (c ^ (lq % CPR))) * 16u + 8u * h, w);
            }
        }
        lds_reads_done();  // (also the writes: the LDS wait covers both)
        constexpr int RPI = 64 / CPR;  // rows per store instruction
        uint16_t* ohead = (uint16_t*)a.out + qhead * D;
#pragma unroll
        for (int j = 0; j < 32 / RPI; ++j) {
            const int r = j * RPI + lane / CPR, c = lane % CPR;
            const u32x4 x = lds_load128(ob + (uint32_t)(r * CPR + (c ^ (r % CPR))) * 16u);
            // non-temporal: nothing in this launch reads the output back, and the
            // cache lines it would occupy hold K/V tiles other workgroups reuse
            if (r0 + r < T) __builtin_nontemporal_store(x, (u32x4*)(ohead + (size_t)(r0 + r - q_first) * D + 8 * c));
        }
    }
    if (row_ok) {
        // lse = base / log2 e + ln(l) (base is in log2 units of the scaled scores)
        if (a.lse && h == 0)
            a.lse[qhead + (my_q - q_first)] = l_tot > 0.f ? base * 0.6931471805599453f + __logf(l_tot)
                                                                      : kNegInf;
    }
    SWA_TRACE(5);
}


template <bool DUMP>
hipError_t launch_bf16(const PrefillArgs& args, DumpOut dump, hipStream_t s) {
    PrefillArgs a = args;
    const int G = a.Hq / a.Hkv;
    const int wg_rows = 32 * a.rbs;
    const int nqb = (a.T - a.q_first + wg_rows - 1) / wg_rows;
    const long long nblocks = (long long)nqb * a.Hkv * (G / a.hpw) * a.B;
    if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    a.div_nqb = make_fastdiv((uint32_t)nqb);
    a.div_hg = make_fastdiv((uint32_t)(a.Hkv * (G / a.hpw)));
    a.div_groups = make_fastdiv((uint32_t)(G / a.hpw));
    a.div_hpw = make_fastdiv((uint32_t)a.hpw);
    a.div_block = make_fastdiv((uint32_t)(a.block > 0 ? a.block : 1));
    dim3 grid((unsigned)nblocks);
    dim3 block(64 * kMfmaWaves);
    const bool rope = !DUMP && a.rope_len > 0;
    const bool comp = a.block > 0;
#define SWA_LAUNCH(DD, RR, CC) \
    hipLaunchKernelGGL((prefill_bf16_kernel<DD, RR, CC, DUMP, false>), grid, block, 0, s, a, dump)
    if (!DUMP && a.k2 != nullptr) {  // split sources: plain mode, no rotation
        if (a.D == 64)
            hipLaunchKernelGGL((prefill_bf16_kernel<64, false, false, false, true>), grid, block, 0, s, a, dump);
        else
            hipLaunchKernelGGL((prefill_bf16_kernel<32, false, false, false, true>), grid, block, 0, s, a, dump);
    } else if (a.D == 64) {
        if (comp) {
            if (rope) SWA_LAUNCH(64, !DUMP, true);
            else SWA_LAUNCH(64, false, true);
        } else {
            if (rope) SWA_LAUNCH(64, !DUMP, false);
            else SWA_LAUNCH(64, false, false);
        }
    } else {
        if (comp) {
            if (rope) SWA_LAUNCH(32, !DUMP, true);
            else SWA_LAUNCH(32, false, true);
        } else {
            if (rope) SWA_LAUNCH(32, !DUMP, false);
            else SWA_LAUNCH(32, false, false);
        }
    }
#undef SWA_LAUNCH
    return hipGetLastError();
}

__global__ void fill_zero_kernel(uint8_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) { return launch_bf16<false>(a, DumpOut{}, s); }

hipError_t launch_prefill_bf16_dump(const PrefillArgs& a, uint8_t* mask, int32_t* count, hipStream_t s) {
    if (mask != nullptr) {  // zero the mask first (a fill kernel, not a memset)
        const int Tk = a.block > 0 ? a.nblk + a.T : a.T;
        hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, s, mask, (size_t)a.B * a.T * Tk);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_bf16<true>(a, DumpOut{mask, count}, s);
}

}  // namespace swa
