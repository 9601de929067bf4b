// chunk.hip -- chunked prefill into existing int8 caches.
//
// A chunk of Tc tokens at positions pos0 .. pos0 + Tc - 1 attends, with the
// decode mask of [NS] "256-token滑动窗口+KV sink：Needle 2工具钉住机制源码分析"
// (section "256-token 滑动窗口：源码走读": recent | sink, no packing term), over
// the sink rows, the ring as it holds positions before the chunk, and its own
// keys; then the chunk's last min(W, Tc) tokens are quantized into the ring.
// The pages name chunked prefill (the DwarfStar README runs long prompts in
// chunks of 4096 tokens) without defining the step; this is its plainest
// reading.
//
// The attention itself is the bf16 prefill kernel over a key sequence of
// Tv = C + Tc rows per (batch row, kv head), C = S + W - 1 rounded up to 64:
//   rows [0, S)            sink rows (prefix, segment 1) up to sink_len,
//                          padding (segment 0) after it;
//   rows [S, C - W + 1)    padding (at most 63 rows);
//   rows [C - W + 1, C)    ring positions pos0 - W + 1 .. pos0 - 1, in order,
//                          padding where the ring holds no such position;
//   rows [C, Tv)           the chunk.
// Ring and chunk rows are contiguous in position, so the kernel's window test
// on row indices is the test on positions; the sinks are visible as prefix
// keys; padding rows are in no segment.  Only the C cached rows are staged
// (dequantized: code x scale in fp32, then rounded to bf16); the kernel reads
// the chunk's keys and values, and its queries, where the caller keeps them,
// and writes the output in place (its query rows start at C, its keys switch
// source at C).
#include "swa_common.h"
#include "swa_internal.h"
#include "swa_tiles.h"

namespace swa {
namespace {

// Where cached row j of batch row b comes from: kind 0 padding, 1 sink row
// src of the sink cache, 2 ring slot src; src counts rows of the (batch row,
// kv head) bh's cache.
struct CachedRow {
    int kind;
    long long src;
};
__device__ __forceinline__ CachedRow cached_row(const ChunkArgs& a, int j, int bh) {
    const int b = bh / a.Hkv;
    const int p0 = a.pos0[b] > 0 ? a.pos0[b] : 0;
    int sl = a.sink_len ? a.sink_len[b] : a.S;
    sl = max(0, min(min(sl, a.S), p0));
    const int ring0 = a.C - (a.W - 1);
    CachedRow r{0, 0};
    if (j < a.S) {
        if (j < sl) r = CachedRow{1, (long long)bh * a.S + j};
    } else if (j >= ring0) {
        const int p = p0 - (a.W - 1) + (j - ring0);
        if (p >= sl && p >= 0) r = CachedRow{2, (long long)bh * a.W + (p % a.W)};
    }
    return r;
}

// One launch stages everything.  Blocks below kv_blocks: one thread per
// (batch row, kv head, cached row j, 16 channels) dequantizes K and V (code x
// scale in fp32, rounded to bf16), 16-byte accesses; padding rows are zero.
// The other blocks: one wave per (batch row, 64-key tile) writes the keys'
// segment ids and prefix flags -- sinks up to sink_len and held ring
// positions in segment 1 (sinks flagged), the chunk in segment 1, padding in
// segment 0 -- and the prefill's key metadata of the tile, so that the
// prefill needs no pre-pass.
__global__ __launch_bounds__(256) void chunk_stage_kernel(ChunkArgs a, uint16_t* ks, uint16_t* vs, int32_t* seg,
                                                          uint8_t* prefix, int kv_blocks) {
    if ((int)blockIdx.x < kv_blocks) {
        const int D = a.D, per = D / 16;
        const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
        if (idx >= (long long)a.B * a.Hkv * a.C * per) return;
        const int d0 = 16 * (int)(idx % per);
        const long long rowid = idx / per;  // bh * C + j
        const int j = (int)(rowid % a.C);
        const int bh = (int)(rowid / a.C);
        const CachedRow r = cached_row(a, j, bh);
        uint32_t kw[8] = {0, 0, 0, 0, 0, 0, 0, 0}, vw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r.kind != 0) {
            const int8_t* kc = r.kind == 1 ? a.sink_k : a.ring_k;
            const int8_t* vc = r.kind == 1 ? a.sink_v : a.ring_v;
            const float* kss = r.kind == 1 ? a.sink_ks : a.ring_ks;
            const float* vss = r.kind == 1 ? a.sink_vs : a.ring_vs;
            // (non-temporal: every cached row is read once per call)
            const uint4 kq = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(kc + r.src * D + d0)));
            const uint4 vq = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(vc + r.src * D + d0)));
            const float sk = kss[r.src * (D / 32) + d0 / 32], sv = vss[r.src * (D / 32) + d0 / 32];
            const uint32_t kq4[4] = {kq.x, kq.y, kq.z, kq.w}, vq4[4] = {vq.x, vq.y, vq.z, vq.w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    // codes of channels 4w + 2h and 4w + 2h + 1 (bytes 2h, 2h + 1), sign-extended
                    const int k0 = (int)(kq4[w] << (24 - 16 * h)) >> 24, k1 = (int)(kq4[w] << (16 - 16 * h)) >> 24;
                    const int v0 = (int)(vq4[w] << (24 - 16 * h)) >> 24, v1 = (int)(vq4[w] << (16 - 16 * h)) >> 24;
                    kw[2 * w + h] = f32_to_bf16_bits((float)k0 * sk) | (f32_to_bf16_bits((float)k1 * sk) << 16);
                    vw[2 * w + h] = f32_to_bf16_bits((float)v0 * sv) | (f32_to_bf16_bits((float)v1 * sv) << 16);
                }
            }
        }
        const size_t dst = ((size_t)bh * a.C + j) * D + d0;
        *(uint4*)(ks + dst) = make_uint4(kw[0], kw[1], kw[2], kw[3]);
        *(uint4*)(ks + dst + 8) = make_uint4(kw[4], kw[5], kw[6], kw[7]);
        *(uint4*)(vs + dst) = make_uint4(vw[0], vw[1], vw[2], vw[3]);
        *(uint4*)(vs + dst + 8) = make_uint4(vw[4], vw[5], vw[6], vw[7]);
        return;
    }
    const long long gt = (long long)(blockIdx.x - kv_blocks) * 4 + (threadIdx.x >> 6);
    if (gt >= (long long)a.B * a.ntile) return;
    const int lane = threadIdx.x & 63;
    const int b = (int)(gt / a.ntile), jt = (int)(gt % a.ntile);
    const int j = 64 * jt + lane;
    const bool valid = j < a.Tv;
    int kind = 3;  // the chunk
    if (valid && j < a.C) kind = cached_row(a, j, b * a.Hkv).kind;
    const int sg = kind != 0 ? 1 : 0;
    const bool sk = kind == 1;
    if (valid) {
        seg[(size_t)b * a.Tv + j] = sg;
        prefix[(size_t)b * a.Tv + j] = sk ? 1 : 0;
    }
    write_key_tile_meta(b, jt, lane, a.Tv, a.ntile, valid, sg, sk, a.info, a.ksub, a.tsink);
}

// The ring write: token i of the chunk (one of its last min(W, Tc)) goes to
// slot (pos0 + i) mod W, K and V quantized like swa_kv_quantize.  One 64-lane
// block per (token, batch row, kv head); lane l quantizes channel l % D.
__global__ __launch_bounds__(64) void chunk_ring_write_kernel(ChunkArgs a, int first) {
    const int i = first + blockIdx.x;
    const int bh = blockIdx.y;
    const int b = bh / a.Hkv;
    const int lane = threadIdx.x;
    const int D = a.D;
    const int p0 = a.pos0[b] > 0 ? a.pos0[b] : 0;
    const long long src = ((long long)bh * a.Tc + i) * D;
    const int d = lane % D;
    float sk, sv;
    const int ck = quantize_lane(bf16_bits_to_f32(((const uint16_t*)a.k)[src + d]), sk);
    const int cv = quantize_lane(bf16_bits_to_f32(((const uint16_t*)a.v)[src + d]), sv);
    const size_t slot = (size_t)bh * a.W + (size_t)((p0 + (long long)i) % a.W);
    if (lane < D) {
        a.ring_k[slot * D + d] = (int8_t)ck;
        a.ring_v[slot * D + d] = (int8_t)cv;
        if ((lane & 31) == 0) {
            a.ring_ks[slot * (D / 32) + lane / 32] = sk;
            a.ring_vs[slot * (D / 32) + lane / 32] = sv;
        }
    }
}

}  // namespace

hipError_t launch_chunk_stage(const ChunkArgs& a, void* k_stage, void* v_stage, int32_t* seg, uint8_t* prefix,
                              hipStream_t s) {
    const long long kv = (long long)a.B * a.Hkv * a.C * (a.D / 16);
    const long long meta = (long long)a.B * a.ntile;  // one wave per 64-key tile
    const long long kv_blocks = (kv + 255) / 256, blocks = kv_blocks + (meta + 3) / 4;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(chunk_stage_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, (uint16_t*)k_stage,
                       (uint16_t*)v_stage, seg, prefix, (int)kv_blocks);
    return hipGetLastError();
}

hipError_t launch_chunk_finish(const ChunkArgs& a, hipStream_t s) {
    const int first = a.Tc > a.W ? a.Tc - a.W : 0;
    if (a.Tc - first > 0) {
        hipLaunchKernelGGL(chunk_ring_write_kernel, dim3((unsigned)(a.Tc - first), (unsigned)(a.B * a.Hkv)), dim3(64),
                           0, s, a, first);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace swa
