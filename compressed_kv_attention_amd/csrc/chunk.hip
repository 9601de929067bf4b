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
#include <algorithm>

#include "swa_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

// One (cached row j, batch row b, kv head) per 64-lane block: lane d < D
// moves channel d of K and V.
__global__ __launch_bounds__(64) void chunk_stage_kv_kernel(ChunkArgs a, uint16_t* ks, uint16_t* vs) {
    const int j = blockIdx.x;   // < C
    const int bh = blockIdx.y;  // b * Hkv + hkv
    const int b = bh / a.Hkv;
    const int d = threadIdx.x;
    const int D = a.D, W = a.W, S = a.S;
    const int p0 = a.pos0[b] > 0 ? a.pos0[b] : 0;
    int sl = a.sink_len ? a.sink_len[b] : S;
    sl = max(0, min(min(sl, S), p0));
    const int ring0 = a.C - (W - 1);
    int kind = 0;  // 0 padding, 1 sink, 2 ring
    long long src = 0;
    if (j < S) {
        if (j < sl) {
            kind = 1;
            src = (long long)bh * S + j;
        }
    } else if (j >= ring0) {
        const int p = p0 - (W - 1) + (j - ring0);
        if (p >= sl && p >= 0) {
            kind = 2;
            src = (long long)bh * W + (p % W);
        }
    }
    if (d < D) {
        uint16_t kb = 0, vb = 0;
        if (kind != 0) {
            const int8_t* kc = kind == 1 ? a.sink_k : a.ring_k;
            const int8_t* vc = kind == 1 ? a.sink_v : a.ring_v;
            const float* kss = kind == 1 ? a.sink_ks : a.ring_ks;
            const float* vss = kind == 1 ? a.sink_vs : a.ring_vs;
            const float kf = (float)kc[src * D + d] * kss[src * (D / 32) + d / 32];
            const float vf = (float)vc[src * D + d] * vss[src * (D / 32) + d / 32];
            kb = (uint16_t)f32_to_bf16_bits(kf);
            vb = (uint16_t)f32_to_bf16_bits(vf);
        }
        const size_t dst = ((size_t)bh * a.C + j) * D;
        ks[dst + d] = kb;
        vs[dst + d] = vb;
    }
}

// Segment ids and prefix flags of the key sequence, one thread per (b, row):
// sinks up to sink_len and held ring positions in segment 1 (sinks flagged),
// the chunk in segment 1, padding in segment 0.
__global__ void chunk_stage_meta_kernel(ChunkArgs a, int32_t* seg, uint8_t* prefix) {
    const long long total = (long long)a.B * a.Tv;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const int b = (int)(i / a.Tv);
        const int j = (int)(i - (long long)b * a.Tv);
        const int p0 = a.pos0[b] > 0 ? a.pos0[b] : 0;
        int sl = a.sink_len ? a.sink_len[b] : a.S;
        sl = max(0, min(min(sl, a.S), p0));
        const int ring0 = a.C - (a.W - 1);
        int kind = 0;
        if (j >= a.C) {
            kind = 3;
        } else if (j < a.S) {
            kind = j < sl ? 1 : 0;
        } else if (j >= ring0) {
            const int p = p0 - (a.W - 1) + (j - ring0);
            kind = (p >= sl && p >= 0) ? 2 : 0;
        }
        seg[i] = kind != 0 ? 1 : 0;
        prefix[i] = kind == 1 ? 1 : 0;
    }
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
    if (a.C > 0) {
        hipLaunchKernelGGL(chunk_stage_kv_kernel, dim3((unsigned)a.C, (unsigned)(a.B * a.Hkv)), dim3(64), 0, s, a,
                           (uint16_t*)k_stage, (uint16_t*)v_stage);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long long n = (long long)a.B * a.Tv;
    const unsigned blocks = (unsigned)std::min<long long>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(chunk_stage_meta_kernel, dim3(blocks), dim3(256), 0, s, a, seg, prefix);
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
