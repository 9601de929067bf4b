// oracle.cpp -- plain CPU oracle for windowed+sink GQA attention and its
// compressed-KV variant.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
// its Python binding) may link, load or call this file.  Only the tests, the
// graft entry's smoke check and the benchmark's CPU-baseline leg use it.  It
// shares no code, header, table or constant generator with the GPU path.
//
// Every result is computed the slow, obvious way: fp64 plain loops, scores and
// softmax in two passes (no online rescaling, no blocking, no fusion).  The
// only fp32 arithmetic is the int8 quantizer, whose rounding the method fixes
// in fp32 (see oracle_quantize).
//
// Sources (web pages; cited by title and section):
//   [NW] "How the 256-Token Sliding Window Works with Tools as KV Sinks in
//        Needle" (instagit.com)
//   [NS] "256-token滑动窗口+KV sink：Needle 2工具钉住机制源码分析" (cf-1.com)
//   [CA] "Compressed attention and the copy probe" (octlm.ramaa.tech)
//
// Readings taken where the pages are silent:
//   R-A1 prefill mask = packing & causal & (recent | sink), literally as the
//        make_causal_packing_mask code composes it, so sinks do not cross
//        segments in prefill; the decode mask has no packing term.
//   R-A3 window == 0 disables windowing (the code tests `if window:`).
//   R-A4 a row with no visible key: output 0, lse = -inf.
//   R-A5 GQA: kv head = q head / (Hq / Hkv).
//   R-A6 scale defaults to 1/sqrt(D) (the caller passes it explicitly here).
//   R-A7 RoPE is rotate-half with inv_freq_i = theta^(-2i/D), position = row
//        index.  The pairing convention is parity-unpinned.
//   R-A8 pool_blocks = arithmetic mean of b consecutive rows, T mod b dropped.
//   R-A9 the exact-key mask of the compressed variant is the causal window
//        t <= q && q - t < W with no sinks and no segments.
//   R-A13 int8 scheme: symmetric absmax/127 per 32 channels, round half even,
//        clamp to +-127, zero group -> zero scale and zero codes.
//   R-A14 decode ring: slot = position mod W; sinks live in their own cache.
//   R-A15 compressed decode state: exact ring + pooled blocks (capacity P) +
//        frontier sums of the block in progress (see O8).
//   R-A20 chunked prefill: the chunk attends over the sinks, the ring as it
//        was before the chunk, and its own unquantized keys; then the ring
//        takes its last W tokens (see O9).
//   R-A21 backward: the plain derivative of the forward definition (O10).
//   R-A22 NSA selection branch: top-k pooled blocks among those that cleared
//        the window, by compressed score; attention over their exact tokens.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// O1: prefill visibility.  [NW §"KV Sinks for Tools: Pinning Critical
// Context"]: mask = block & causal, then, if a window is set,
// mask &= (recent | sink) with recent = (q - k) < window and sink = prefix > 0;
// block = (seg_q == seg_k) & (seg_q > 0).  seg == NULL means every position
// is segment 1; prefix == NULL means no sinks.
bool visible_prefill(const int32_t* seg_row, const uint8_t* prefix_row, int q, int k, int window) {
    const int seg_q = seg_row ? seg_row[q] : 1;
    const int seg_k = seg_row ? seg_row[k] : 1;
    const bool block = (seg_q == seg_k) && (seg_q > 0);
    const bool causal = k <= q;
    bool keep = block && causal;
    if (window != 0) {
        const bool recent = (q - k) < window;
        const bool sink = prefix_row ? (prefix_row[k] > 0) : false;
        keep = keep && (recent || sink);
    }
    return keep;
}

// O4 masks.  [CA §"Two kinds of columns, pooled blocks and exact recent
// keys"]: pooled block j is visible to row q once (j + 1) * b <= q - W + 1;
// exact column t follows the plain causal window (reading R-A9).
bool visible_pooled(int q, int j, int window, int block) {
    return static_cast<long long>(j + 1) * block <= static_cast<long long>(q) - window + 1;
}
bool visible_exact_window(int q, int t, int window) {
    return t <= q && (q - t) < window;
}

// O2: RoPE, rotate-half pairing (i, i + D/2), angle = pos * theta^(-2i/D),
// all in fp64 (reading R-A7).  [CA §"Pool before rotating, not after"] applies
// it to q and exact k at their own positions and to each pooled key at its
// block midpoint.
void rope_rotate(const double* x, double* y, int D, double theta, long long pos) {
    const int half = D / 2;
    for (int i = 0; i < half; ++i) {
        const double inv_freq = std::pow(theta, -2.0 * static_cast<double>(i) / static_cast<double>(D));
        const double angle = static_cast<double>(pos) * inv_freq;
        const double c = std::cos(angle);
        const double s = std::sin(angle);
        const double a = x[i];
        const double b = x[i + half];
        y[i] = a * c - b * s;
        y[i + half] = b * c + a * s;
    }
}

// O3: softmax attention of one query row over an explicit list of columns,
// exact two-pass form: s_j = scale * <q, k_j>; m = max s; w_j = exp(s_j - m);
// l = sum w; o = sum w_j v_j / l; lse = m + log(l).  Empty column list gives
// o = 0 and lse = -inf (reading R-A4).
void attend_row(const double* q, const std::vector<const double*>& keys,
                const std::vector<const double*>& vals, int D, double scale,
                double* out, double* lse) {
    const size_t n = keys.size();
    if (n == 0) {
        for (int d = 0; d < D; ++d) out[d] = 0.0;
        if (lse) *lse = -std::numeric_limits<double>::infinity();
        return;
    }
    std::vector<double> s(n);
    double m = -std::numeric_limits<double>::infinity();
    for (size_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += q[d] * keys[j][d];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (size_t j = 0; j < n; ++j) {
        s[j] = std::exp(s[j] - m);
        l += s[j];
    }
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (size_t j = 0; j < n; ++j) acc += s[j] * vals[j][d];
        out[d] = acc / l;
    }
    if (lse) *lse = m + std::log(l);
}

// Rotated copy of a [N, T, D] tensor at positions 0..T-1 (fp64).
std::vector<double> rotate_rows(const double* x, long long N, int T, int D, double theta) {
    std::vector<double> y(static_cast<size_t>(N) * T * D);
    for (long long n = 0; n < N; ++n)
        for (int t = 0; t < T; ++t)
            rope_rotate(x + (n * T + t) * D, y.data() + (n * T + t) * D, D, theta, t);
    return y;
}

}  // namespace

extern "C" {

int oracle_version(void) { return 1; }

// O1 written out: mask[b, q, k] for all b, q, k ([B, T, T] u8, 1 = visible).
void oracle_mask(int B, int T, const int32_t* seg, const uint8_t* prefix, int window, uint8_t* mask) {
    for (int b = 0; b < B; ++b) {
        const int32_t* seg_row = seg ? seg + static_cast<size_t>(b) * T : nullptr;
        const uint8_t* pre_row = prefix ? prefix + static_cast<size_t>(b) * T : nullptr;
        for (int q = 0; q < T; ++q)
            for (int k = 0; k < T; ++k)
                mask[(static_cast<size_t>(b) * T + q) * T + k] =
                    visible_prefill(seg_row, pre_row, q, k, window) ? 1 : 0;
    }
}

// O4 mask written out: [T, T/block + T] u8, columns [pooled blocks, exact].
void oracle_compressed_mask(int T, int window, int block, uint8_t* mask) {
    const int nblk = T / block;
    const int ncol = nblk + T;
    for (int q = 0; q < T; ++q) {
        for (int j = 0; j < nblk; ++j)
            mask[static_cast<size_t>(q) * ncol + j] = visible_pooled(q, j, window, block) ? 1 : 0;
        for (int t = 0; t < T; ++t)
            mask[static_cast<size_t>(q) * ncol + nblk + t] = visible_exact_window(q, t, window) ? 1 : 0;
    }
}

// O2 exposed for the pins: rotate x[N, D] at pos[N].
void oracle_rope(int N, int D, double theta, const int64_t* pos, const double* x, double* y) {
    for (int n = 0; n < N; ++n)
        rope_rotate(x + static_cast<size_t>(n) * D, y + static_cast<size_t>(n) * D, D, theta, pos[n]);
}

// O1 + O2 + O3: windowed+sink GQA prefill.
//   q [B,Hq,T,D], k/v [B,Hkv,T,D] fp64 (values exactly as the GPU receives them)
//   seg [B,T] i32 or NULL, prefix [B,T] u8 or NULL, window >= 0
//   theta > 0 rotates q and k at their row index; theta == 0 means no RoPE
//   rows: nrows flat indices ((b*Hq + h)*T + t), or NULL for all rows in order
//   out [nrows, D], lse [nrows] (lse may be NULL)
void oracle_prefill(int B, int Hq, int Hkv, int T, int D, const double* q, const double* k,
                    const double* v, const int32_t* seg, const uint8_t* prefix, int window,
                    double scale, double theta, long long nrows, const int64_t* rows,
                    double* out, double* lse) {
    const int G = Hq / Hkv;
    std::vector<double> k_rot;
    const double* kk = k;
    if (theta > 0.0) {
        k_rot = rotate_rows(k, static_cast<long long>(B) * Hkv, T, D, theta);
        kk = k_rot.data();
    }
    const long long total = rows ? nrows : static_cast<long long>(B) * Hq * T;
#pragma omp parallel for schedule(dynamic, 16)
    for (long long r = 0; r < total; ++r) {
        const long long flat = rows ? rows[r] : r;
        const int t = static_cast<int>(flat % T);
        const int h = static_cast<int>((flat / T) % Hq);
        const int b = static_cast<int>(flat / (static_cast<long long>(T) * Hq));
        const int hk = h / G;
        std::vector<double> qrow(D);
        const double* qsrc = q + flat * D;
        if (theta > 0.0) rope_rotate(qsrc, qrow.data(), D, theta, t);
        else for (int d = 0; d < D; ++d) qrow[d] = qsrc[d];
        const int32_t* seg_row = seg ? seg + static_cast<size_t>(b) * T : nullptr;
        const uint8_t* pre_row = prefix ? prefix + static_cast<size_t>(b) * T : nullptr;
        const size_t kv_base = (static_cast<size_t>(b) * Hkv + hk) * T;
        std::vector<const double*> keys, vals;
        for (int s = 0; s < T; ++s) {
            if (!visible_prefill(seg_row, pre_row, t, s, window)) continue;
            keys.push_back(kk + (kv_base + s) * D);
            vals.push_back(v + (kv_base + s) * D);
        }
        attend_row(qrow.data(), keys, vals, D, scale, out + r * D, lse ? lse + r : nullptr);
    }
}

// O4, first half: pool_blocks then midpoint RoPE.  [CA §"Pool before
// rotating, not after"]: pooled key/value j = mean of rows j*b .. j*b+b-1 of
// the PRE-RoPE key (and of the value); the pooled key alone is then rotated
// at min(j*b + b/2, rope_len - 1).  theta == 0 skips the rotation.
//   k_pre, v [N, T, D]; pk, pv [N, T/block, D]
void oracle_pool_rope(long long N, int T, int D, int block, double theta, int rope_len,
                      const double* k_pre, const double* v, double* pk, double* pv) {
    const int nblk = T / block;
    std::vector<double> mean_k(D);
    for (long long n = 0; n < N; ++n) {
        for (int j = 0; j < nblk; ++j) {
            double* pk_row = pk + (n * nblk + j) * D;
            double* pv_row = pv + (n * nblk + j) * D;
            for (int d = 0; d < D; ++d) {
                double sk = 0.0, sv = 0.0;
                for (int i = 0; i < block; ++i) {
                    const long long t = static_cast<long long>(j) * block + i;
                    sk += k_pre[(n * T + t) * D + d];
                    sv += v[(n * T + t) * D + d];
                }
                mean_k[d] = sk / block;
                pv_row[d] = sv / block;
            }
            if (theta > 0.0) {
                long long mid = static_cast<long long>(j) * block + block / 2;
                if (mid > rope_len - 1) mid = rope_len - 1;
                rope_rotate(mean_k.data(), pk_row, D, theta, mid);
            } else {
                for (int d = 0; d < D; ++d) pk_row[d] = mean_k[d];
            }
        }
    }
}

// O4, second half: attention of each row over [pooled blocks, exact keys]
// with one softmax.  q/k_pre/v [B,Hq|Hkv,T,D]; the pooled columns are built
// here with oracle_pool_rope; q and exact k are rotated at their row index.
// rows/out/lse as in oracle_prefill.
void oracle_compressed_prefill(int B, int Hq, int Hkv, int T, int D, const double* q,
                               const double* k_pre, const double* v, int window, int block,
                               double scale, double theta, int rope_len, long long nrows,
                               const int64_t* rows, double* out, double* lse) {
    const int G = Hq / Hkv;
    const int nblk = T / block;
    const long long NKV = static_cast<long long>(B) * Hkv;
    std::vector<double> pk(static_cast<size_t>(NKV) * nblk * D), pv(static_cast<size_t>(NKV) * nblk * D);
    oracle_pool_rope(NKV, T, D, block, theta, rope_len, k_pre, v, pk.data(), pv.data());
    std::vector<double> k_rot;
    const double* kk = k_pre;
    if (theta > 0.0) {
        k_rot = rotate_rows(k_pre, NKV, T, D, theta);
        kk = k_rot.data();
    }
    const long long total = rows ? nrows : static_cast<long long>(B) * Hq * T;
#pragma omp parallel for schedule(dynamic, 16)
    for (long long r = 0; r < total; ++r) {
        const long long flat = rows ? rows[r] : r;
        const int t = static_cast<int>(flat % T);
        const int h = static_cast<int>((flat / T) % Hq);
        const int b = static_cast<int>(flat / (static_cast<long long>(T) * Hq));
        const int hk = h / G;
        std::vector<double> qrow(D);
        const double* qsrc = q + flat * D;
        if (theta > 0.0) rope_rotate(qsrc, qrow.data(), D, theta, t);
        else for (int d = 0; d < D; ++d) qrow[d] = qsrc[d];
        const size_t nk = static_cast<size_t>(b) * Hkv + hk;
        std::vector<const double*> keys, vals;
        for (int j = 0; j < nblk; ++j) {           // pooled columns first
            if (!visible_pooled(t, j, window, block)) continue;
            keys.push_back(pk.data() + (nk * nblk + j) * D);
            vals.push_back(pv.data() + (nk * nblk + j) * D);
        }
        for (int s = 0; s < T; ++s) {              // then the exact keys
            if (!visible_exact_window(t, s, window)) continue;
            keys.push_back(kk + (nk * T + s) * D);
            vals.push_back(v + (nk * T + s) * D);
        }
        attend_row(qrow.data(), keys, vals, D, scale, out + r * D, lse ? lse + r : nullptr);
    }
}

// O5: budget window.  [NW §"Effective KV Window: Bounding the Cache Size"]
// and [NS §"256 这个窗口宽度从哪来：内存预算计算器"], restated: the whole KV
// cache gets a fixed budget of 11.5 MiB.  One cached position costs, in every
// layer, one byte per K and per V channel plus one 4-byte scale per group of
// 32 channels of each; every engram site adds d_model bytes plus 128.  The
// channel count is num_kv_heads times the head size, the head size being
// attn_dim (or d_model when attn_dim is unset, 0) divided by num_heads.  The
// budget window is the largest multiple of 32 positions whose cache fits the
// budget, capped at max_seq_len, with a floor of 160 that wins over the cap.
// The effective window is the smaller of that and a set kv_window.
long long oracle_kv_budget_per_pos(long long d_model, long long attn_dim, long long num_heads,
                                   long long num_kv_heads, long long num_layers, long long sites) {
    const long long group = 32;          // channels sharing one fp32 scale
    const long long scale_bytes = 4;     // one fp32 scale
    const long long head_size = (attn_dim != 0 ? attn_dim : d_model) / num_heads;
    const long long channels = num_kv_heads * head_size;
    const long long one_tensor = channels * 1 + (channels / group) * scale_bytes;  // int8 codes + scales
    const long long per_layer = 2 * one_tensor;                                    // K and V
    const long long per_site = d_model + group * scale_bytes;
    return num_layers * per_layer + sites * per_site;
}
long long oracle_kv_budget_window(long long d_model, long long attn_dim, long long num_heads,
                                  long long num_kv_heads, long long num_layers, long long sites,
                                  long long max_seq_len) {
    const long long budget_bytes = 11LL * 1024 * 1024 + 512LL * 1024;
    const long long per_pos =
        oracle_kv_budget_per_pos(d_model, attn_dim, num_heads, num_kv_heads, num_layers, sites);
    // largest multiple of 32 positions that fits: 32 * floor(budget / (32 * per_pos))
    const long long fits = 32 * (budget_bytes / (32 * per_pos));
    if (fits <= 160 || max_seq_len <= 160) return 160;
    return fits < max_seq_len ? fits : max_seq_len;
}
// effective window: the budget window, or kv_window when one is set and smaller
long long oracle_effective_kv_window(long long d_model, long long attn_dim, long long num_heads,
                                     long long num_kv_heads, long long num_layers, long long sites,
                                     long long max_seq_len, long long kv_window) {
    const long long budget = oracle_kv_budget_window(d_model, attn_dim, num_heads, num_kv_heads,
                                                     num_layers, sites, max_seq_len);
    return (kv_window != 0 && kv_window < budget) ? kv_window : budget;
}

// O6: int8 quantizer with one fp32 scale per 32 channels (the cache layout
// the budget formula prices in [NW §"Effective KV Window"]: one byte per K/V
// element plus 4 bytes per 32 channels).  The scheme itself is reading R-A13,
// evaluated in IEEE fp32 exactly as written:
//   amax = max |x| over the group; s = amax / 127.0f;
//   q = clamp(rint(x / s), -127, 127) (round half to even); s == 0 -> q = 0.
//   x [N, D] fp32, xq [N, D] i8, xs [N, D/32] fp32.
void oracle_quantize(long long N, int D, const float* x, int8_t* xq, float* xs) {
    const int groups = D / 32;
    for (long long n = 0; n < N; ++n) {
        for (int g = 0; g < groups; ++g) {
            const float* xg = x + n * D + g * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                const float a = std::fabs(xg[i]);
                if (a > amax) amax = a;
            }
            const float s = amax / 127.0f;
            xs[n * groups + g] = s;
            for (int i = 0; i < 32; ++i) {
                int8_t code = 0;
                if (s != 0.0f) {
                    const float r = std::nearbyint(xg[i] / s);   // default mode: half to even
                    const float c = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
                    code = static_cast<int8_t>(c);
                }
                xq[n * D + g * 32 + i] = code;
            }
        }
    }
}

// O7: one decode step over a sink cache plus a ring-buffer window cache.
// [NS §"256-token 滑动窗口：源码走读"]: keep = recent | sink with
// recent = (q_pos - k_pos) < W, and no packing term.  Reading R-A14: the new
// token (k_new, v_new) is quantized (O6) into ring slot pos % W first; then
// the query at position pos attends to sink rows [0, sink_len) and to ring
// positions [max(sink_len, pos - W + 1), pos], each at slot k_pos % W.  K/V
// are dequantized in fp64 as code * scale.
//   q [B,Hq,D] fp64; k_new/v_new [B,Hkv,D] fp32 (NULL = no append)
//   ring_k/ring_v [B,Hkv,W,D] i8 and ring_ks/ring_vs [B,Hkv,W,D/32] fp32 are
//   UPDATED in place by the append; sink_* [B,Hkv,S,D] / [B,Hkv,S,D/32]
//   pos [B], sink_len [B] (NULL = S); out [B,Hq,D] fp64, lse [B,Hq] or NULL.
void oracle_decode(int B, int Hq, int Hkv, int D, int W, int S, const double* q,
                   const float* k_new, const float* v_new, int8_t* ring_k, int8_t* ring_v,
                   float* ring_ks, float* ring_vs, const int8_t* sink_k, const int8_t* sink_v,
                   const float* sink_ks, const float* sink_vs, const int32_t* pos,
                   const int32_t* sink_len, double scale, double* out, double* lse) {
    const int G = Hq / Hkv;
    const int groups = D / 32;
    if (k_new && v_new) {
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < Hkv; ++h) {
                const size_t slot = (static_cast<size_t>(b) * Hkv + h) * W + (pos[b] % W);
                const size_t src = (static_cast<size_t>(b) * Hkv + h) * D;
                oracle_quantize(1, D, k_new + src, ring_k + slot * D, ring_ks + slot * groups);
                oracle_quantize(1, D, v_new + src, ring_v + slot * D, ring_vs + slot * groups);
            }
    }
#pragma omp parallel for schedule(dynamic, 4)
    for (int bh = 0; bh < B * Hq; ++bh) {
        const int b = bh / Hq;
        const int h = bh % Hq;
        const int hk = h / G;
        const int n_sink = sink_len ? sink_len[b] : S;
        const size_t base = static_cast<size_t>(b) * Hkv + hk;
        // dequantized copies of every visible row, in fp64
        std::vector<double> kd, vd;
        auto add_row = [&](const int8_t* kc, const float* ks, const int8_t* vc, const float* vs) {
            for (int d = 0; d < D; ++d) {
                kd.push_back(static_cast<double>(kc[d]) * static_cast<double>(ks[d / 32]));
                vd.push_back(static_cast<double>(vc[d]) * static_cast<double>(vs[d / 32]));
            }
        };
        for (int s = 0; s < n_sink; ++s) {
            const size_t row = base * S + s;
            add_row(sink_k + row * D, sink_ks + row * groups, sink_v + row * D, sink_vs + row * groups);
        }
        const long long p = pos[b];
        long long first = p - W + 1;
        if (first < n_sink) first = n_sink;
        for (long long kp = first; kp <= p; ++kp) {
            const size_t row = base * W + static_cast<size_t>(kp % W);
            add_row(ring_k + row * D, ring_ks + row * groups, ring_v + row * D, ring_vs + row * groups);
        }
        const size_t n = kd.size() / D;
        std::vector<const double*> keys(n), vals(n);
        for (size_t j = 0; j < n; ++j) {
            keys[j] = kd.data() + j * D;
            vals[j] = vd.data() + j * D;
        }
        attend_row(q + static_cast<size_t>(bh) * D, keys, vals, D, scale,
                   out + static_cast<size_t>(bh) * D, lse ? lse + bh : nullptr);
    }
}

// O8: one decode step of the compressed variant.  [CA §"Two kinds of columns,
// pooled blocks and exact recent keys"]: the columns are the pooled blocks
// that have cleared the window, (j + 1) * b <= pos - W + 1, then the exact
// keys of the window, positions max(0, pos - W + 1) .. pos (no sinks,
// reading R-A9).  [CA §"Pool before rotating, not after"]: a pooled key is
// the mean of its block's keys BEFORE rotation, rotated once at
// min(j * b + b/2, rope_len - 1); the pooled value is the mean of the values.
// [CA §"So what happened ?"]: blocks join one at a time as they clear the
// window.  Reading R-A15 (the decode-side state, which the pages only name,
// as the compressor frontier of [DS §磁盘 KV 缓存]): per (sequence, kv head)
// the cache holds the exact ring (slot = position mod W, post-RoPE keys), the
// pooled blocks in order of j (capacity P; a block with j >= P is dropped and
// at most P blocks are visible), and the frontier: the running sums of the
// pre-RoPE keys and of the values of the block in progress.  A step at
// position pos (steps of one sequence come at consecutive positions) first
// appends: ring slot pos % W takes (k_new, v_new); the frontier restarts at
// pos % b == 0 and adds (k_pre, v_new); at pos % b == b - 1 the block
// j = pos / b is complete and is pooled into slot j.  Then the query attends.
// A block completed at pos is not visible before pos + W, so the order of
// pooling and attending within a step does not matter.
//   q [B,Hq,D] (rotated at pos), k_new [B,Hkv,D] (rotated at pos), k_pre
//   [B,Hkv,D] (the same key before rotation), v_new [B,Hkv,D]: fp64 holding
//   the values the GPU receives.  ring_k/ring_v [B,Hkv,W,D], pool_k/pool_v
//   [B,Hkv,P,D]: row values in fp64; with quantize != 0 every stored row is
//   the O6 quantization of its fp32-rounded value, dequantized as code * scale
//   (the int8 cache), else the exact value.  front_k/front_v [B,Hkv,D] fp64.
//   Every state array is UPDATED in place.  pos < 0 appends nothing and sees
//   no column.  out [B,Hq,D], lse [B,Hq] or NULL.
void oracle_compressed_decode(int B, int Hq, int Hkv, int D, int W, int P, int block,
                              const double* q, const double* k_new, const double* k_pre,
                              const double* v_new, double* ring_k, double* ring_v, double* pool_k,
                              double* pool_v, double* front_k, double* front_v, const int32_t* pos,
                              double theta, int rope_len, double scale, int quantize, double* out,
                              double* lse) {
    const int G = Hq / Hkv;
    auto store = [&](const double* x, double* row) {
        if (!quantize) {
            for (int d = 0; d < D; ++d) row[d] = x[d];
            return;
        }
        std::vector<float> xf(D), xs(D / 32);
        std::vector<int8_t> xq(D);
        for (int d = 0; d < D; ++d) xf[d] = static_cast<float>(x[d]);
        oracle_quantize(1, D, xf.data(), xq.data(), xs.data());
        for (int d = 0; d < D; ++d) row[d] = static_cast<double>(xq[d]) * static_cast<double>(xs[d / 32]);
    };
    for (int b = 0; b < B; ++b) {
        const long long p = pos[b];
        if (p < 0) continue;
        for (int h = 0; h < Hkv; ++h) {
            const size_t nk = static_cast<size_t>(b) * Hkv + h;
            const size_t slot = nk * W + static_cast<size_t>(p % W);
            store(k_new + nk * D, ring_k + slot * D);
            store(v_new + nk * D, ring_v + slot * D);
            double* fk = front_k + nk * D;
            double* fv = front_v + nk * D;
            for (int d = 0; d < D; ++d) {
                fk[d] = (p % block == 0 ? 0.0 : fk[d]) + k_pre[nk * D + d];
                fv[d] = (p % block == 0 ? 0.0 : fv[d]) + v_new[nk * D + d];
            }
            const long long j = p / block;
            if (p % block == block - 1 && j < P) {
                std::vector<double> mk(D), mv(D), rk(D);
                for (int d = 0; d < D; ++d) {
                    mk[d] = fk[d] / block;
                    mv[d] = fv[d] / block;
                }
                long long mid = j * block + block / 2;
                if (mid > rope_len - 1) mid = rope_len - 1;
                if (theta > 0.0) rope_rotate(mk.data(), rk.data(), D, theta, mid);
                else rk = mk;
                store(rk.data(), pool_k + (nk * P + j) * D);
                store(mv.data(), pool_v + (nk * P + j) * D);
            }
        }
    }
#pragma omp parallel for schedule(dynamic, 4)
    for (int bh = 0; bh < B * Hq; ++bh) {
        const int b = bh / Hq;
        const int hk = (bh % Hq) / G;
        const size_t nk = static_cast<size_t>(b) * Hkv + hk;
        const long long p = pos[b];
        std::vector<const double*> keys, vals;
        if (p >= 0) {
            for (long long j = 0; j < P; ++j) {            // pooled columns first
                if (!visible_pooled(static_cast<int>(p), static_cast<int>(j), W, block)) break;
                keys.push_back(pool_k + (nk * P + j) * D);
                vals.push_back(pool_v + (nk * P + j) * D);
            }
            for (long long t = (p - W + 1 > 0 ? p - W + 1 : 0); t <= p; ++t) {   // then the window
                const size_t row = nk * W + static_cast<size_t>(t % W);
                keys.push_back(ring_k + row * D);
                vals.push_back(ring_v + row * D);
            }
        }
        attend_row(q + static_cast<size_t>(bh) * D, keys, vals, D, scale,
                   out + static_cast<size_t>(bh) * D, lse ? lse + bh : nullptr);
    }
}

// O9: chunked prefill into existing caches.  Reading A20 (the pages name
// chunked prefill -- [DS] runs long prompts in chunks of 4096 tokens,
// "工作原理与配置方式" -- and [NW] "End-to-End Execution Flow" keeps in the
// cache only what the mask can still show, but neither defines the step):
// a chunk of Tc tokens at positions pos0 .. pos0 + Tc - 1 attends, with the
// decode mask of [NS §"256-token 滑动窗口：源码走读"] (recent | sink, no
// packing term), over the sink rows [0, sl) with sl = min(sink_len, pos0),
// the ring positions [max(sl, t - W + 1), pos0 - 1] as the ring holds them
// BEFORE the chunk, and the chunk's own keys [max(pos0, t - W + 1), t] as
// given (not quantized); then the chunk's last min(W, Tc) tokens are
// quantized (O6) into ring slots position mod W.  K/V of the caches are
// dequantized in fp64 as code * scale.
//   q [B,Hq,Tc,D] fp64 (rotated), k/v [B,Hkv,Tc,D] fp32 (k rotated); ring/sink
//   caches as in O7 (the ring is UPDATED in place); pos0 [B], sink_len [B] or
//   NULL (= S); out [B,Hq,Tc,D] fp64, lse [B,Hq,Tc] or NULL.
void oracle_chunk_prefill(int B, int Hq, int Hkv, int D, int W, int S, int Tc, const double* q,
                          const float* k, const float* v, int8_t* ring_k, int8_t* ring_v, float* ring_ks,
                          float* ring_vs, const int8_t* sink_k, const int8_t* sink_v, const float* sink_ks,
                          const float* sink_vs, const int32_t* pos0, const int32_t* sink_len, double scale,
                          double* out, double* lse) {
    const int G = Hq / Hkv;
    const int groups = D / 32;
#pragma omp parallel for schedule(dynamic, 4)
    for (int bh = 0; bh < B * Hq; ++bh) {
        const int b = bh / Hq;
        const int hk = (bh % Hq) / G;
        const size_t nk = static_cast<size_t>(b) * Hkv + hk;
        const long long p0 = pos0[b];
        long long sl = sink_len ? sink_len[b] : S;
        if (sl > p0) sl = p0;
        if (sl > S) sl = S;
        if (sl < 0) sl = 0;
        std::vector<double> kd, vd;  // dequantized sink and ring rows
        std::vector<long long> kpos;  // their positions
        auto add_row = [&](const int8_t* kc, const float* ks, const int8_t* vc, const float* vs, long long p) {
            for (int d = 0; d < D; ++d) {
                kd.push_back(static_cast<double>(kc[d]) * static_cast<double>(ks[d / 32]));
                vd.push_back(static_cast<double>(vc[d]) * static_cast<double>(vs[d / 32]));
            }
            kpos.push_back(p);
        };
        for (long long s = 0; s < sl; ++s) {
            const size_t row = nk * S + static_cast<size_t>(s);
            add_row(sink_k + row * D, sink_ks + row * groups, sink_v + row * D, sink_vs + row * groups, -1);
        }
        for (long long p = (p0 - W + 1 > sl ? p0 - W + 1 : sl); p < p0; ++p) {
            const size_t row = nk * W + static_cast<size_t>(p % W);
            add_row(ring_k + row * D, ring_ks + row * groups, ring_v + row * D, ring_vs + row * groups, p);
        }
        std::vector<double> kc(static_cast<size_t>(Tc) * D), vc(static_cast<size_t>(Tc) * D);
        for (size_t x = 0; x < kc.size(); ++x) {
            kc[x] = k[nk * Tc * D + x];
            vc[x] = v[nk * Tc * D + x];
        }
        for (int i = 0; i < Tc; ++i) {
            const long long t = p0 + i;
            std::vector<const double*> keys, vals;
            for (size_t r = 0; r < kpos.size(); ++r) {
                if (kpos[r] >= 0 && t - kpos[r] >= W) continue;   // sinks (-1) always; ring rows in the window
                keys.push_back(kd.data() + r * D);
                vals.push_back(vd.data() + r * D);
            }
            for (int j = 0; j <= i; ++j) {
                if (t - (p0 + j) >= W) continue;
                keys.push_back(kc.data() + static_cast<size_t>(j) * D);
                vals.push_back(vc.data() + static_cast<size_t>(j) * D);
            }
            const size_t o = static_cast<size_t>(bh) * Tc + i;
            attend_row(q + o * D, keys, vals, D, scale, out + o * D, lse ? lse + o : nullptr);
        }
    }
    // the ring write: the chunk's last min(W, Tc) tokens, after every query has read the old ring
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hkv; ++h) {
            const size_t nk = static_cast<size_t>(b) * Hkv + h;
            for (int i = (Tc > W ? Tc - W : 0); i < Tc; ++i) {
                const size_t slot = nk * W + static_cast<size_t>((pos0[b] + static_cast<long long>(i)) % W);
                oracle_quantize(1, D, k + (nk * Tc + i) * D, ring_k + slot * D, ring_ks + slot * groups);
                oracle_quantize(1, D, v + (nk * Tc + i) * D, ring_v + slot * D, ring_vs + slot * groups);
            }
        }
}

// O10: backward of the windowed+sink prefill (O1 + O2 + O3).  [NS §"KV sink
// 如何「钉住」工具"] and [NW §"KV Sinks for Tools"]: the packing mask is the
// training-side mask, so its gradients are part of the method; the pages give
// no backward, and this is the plain derivative of the forward definition
// (reading A21).  Per visible column j of row t (exact two-pass softmax):
//   p_j = softmax_j(scale <q_t, k_j>),  dP_j = <dO_t, v_j>,
//   Delta_t = sum_j p_j dP_j,  dS_j = p_j (dP_j - Delta_t),
//   dq_t = scale sum_j dS_j k_j,  dk_j += scale dS_j q_t,  dv_j += p_j dO_t.
// With theta > 0 q and k are rotated at their row index first (O2), and the
// gradients are taken back through the rotation (rotating by the negative
// angle, the transpose of the rotation).  GQA: a kv head's dk/dv sum over its
// query heads.  q [B,Hq,T,D], k/v [B,Hkv,T,D], dout [B,Hq,T,D]; seg/prefix as
// in O1; dq [B,Hq,T,D], dk/dv [B,Hkv,T,D] fp64 (written, not accumulated into).
void oracle_prefill_backward(int B, int Hq, int Hkv, int T, int D, const double* q, const double* k,
                             const double* v, const double* dout, const int32_t* seg,
                             const uint8_t* prefix, int window, double scale, double theta,
                             double* dq, double* dk, double* dv) {
    const int G = Hq / Hkv;
    const long long NKV = static_cast<long long>(B) * Hkv;
    std::vector<double> kr;
    const double* kk = k;
    if (theta > 0.0) {
        kr = rotate_rows(k, NKV, T, D, theta);
        kk = kr.data();
    }
    const size_t nkv = static_cast<size_t>(NKV) * T * D;
    std::vector<double> dk_rot(nkv, 0.0), dv_acc(nkv, 0.0);
    // rows of one (batch row, kv head) group are handled by one thread so the
    // dk/dv sums need no synchronisation
#pragma omp parallel for schedule(dynamic, 1)
    for (long long nk = 0; nk < NKV; ++nk) {
        const int b = static_cast<int>(nk / Hkv);
        const int hk = static_cast<int>(nk % Hkv);
        const int32_t* seg_row = seg ? seg + static_cast<size_t>(b) * T : nullptr;
        const uint8_t* pre_row = prefix ? prefix + static_cast<size_t>(b) * T : nullptr;
        std::vector<double> qrow(D), dqr(D), s, dp;
        std::vector<int> cols;
        for (int h = hk * G; h < (hk + 1) * G; ++h) {
            for (int t = 0; t < T; ++t) {
                const size_t qo = ((static_cast<size_t>(b) * Hq + h) * T + t) * D;
                if (theta > 0.0) rope_rotate(q + qo, qrow.data(), D, theta, t);
                else for (int d = 0; d < D; ++d) qrow[d] = q[qo + d];
                cols.clear();
                for (int j = 0; j < T; ++j)
                    if (visible_prefill(seg_row, pre_row, t, j, window)) cols.push_back(j);
                for (int d = 0; d < D; ++d) dqr[d] = 0.0;
                if (!cols.empty()) {
                    const size_t n = cols.size();
                    s.assign(n, 0.0);
                    dp.assign(n, 0.0);
                    double m = -std::numeric_limits<double>::infinity();
                    for (size_t c = 0; c < n; ++c) {
                        const double* kj = kk + (static_cast<size_t>(nk) * T + cols[c]) * D;
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d) dot += qrow[d] * kj[d];
                        s[c] = scale * dot;
                        if (s[c] > m) m = s[c];
                    }
                    double l = 0.0;
                    for (size_t c = 0; c < n; ++c) {
                        s[c] = std::exp(s[c] - m);
                        l += s[c];
                    }
                    double delta = 0.0;
                    for (size_t c = 0; c < n; ++c) {
                        s[c] /= l;  // p_j
                        const double* vj = v + (static_cast<size_t>(nk) * T + cols[c]) * D;
                        double x = 0.0;
                        for (int d = 0; d < D; ++d) x += dout[qo + d] * vj[d];
                        dp[c] = x;
                        delta += s[c] * x;
                    }
                    for (size_t c = 0; c < n; ++c) {
                        const double ds = s[c] * (dp[c] - delta);
                        const size_t ko = (static_cast<size_t>(nk) * T + cols[c]) * D;
                        for (int d = 0; d < D; ++d) {
                            dqr[d] += scale * ds * kk[ko + d];
                            dk_rot[ko + d] += scale * ds * qrow[d];
                            dv_acc[ko + d] += s[c] * dout[qo + d];
                        }
                    }
                }
                if (theta > 0.0) rope_rotate(dqr.data(), dq + qo, D, theta, -static_cast<long long>(t));
                else for (int d = 0; d < D; ++d) dq[qo + d] = dqr[d];
            }
        }
        for (int j = 0; j < T; ++j) {
            const size_t ko = (static_cast<size_t>(nk) * T + j) * D;
            if (theta > 0.0) rope_rotate(dk_rot.data() + ko, dk + ko, D, theta, -static_cast<long long>(j));
            else for (int d = 0; d < D; ++d) dk[ko + d] = dk_rot[ko + d];
            for (int d = 0; d < D; ++d) dv[ko + d] = dv_acc[ko + d];
        }
    }
}

// O11: the selection branch of NSA without its gate.  [CA §"Two kinds of
// columns, pooled blocks and exact recent keys"] names NSA's three branches
// -- compressed, selected (the top-k blocks by their compressed scores) and
// the window -- mixed by a learned gate; [CA §"What we didn't build, and
// why"] left selection and the gate out.  Reading A22: for row t the
// candidates are the pooled blocks the compressed variant shows,
// (j + 1) * b <= t - W + 1 (so no selected token is in the window); block
// j's score is scale <q_t, pk_j> with q rotated at t and pk_j the O4 pooled
// key (mean before RoPE, rotated at the block midpoint); the branch takes the
// n_select best blocks (higher score first, the lower j on ties; all when
// fewer) and attends with one softmax over the exact keys, rotated at their
// positions, of every token in them.  No candidate: output 0, lse -inf.
// sel_in (optional, [B,Hq,T,n_select], -1 = none) replaces the selection;
// sel_out (optional) receives it, in score order.
//   q/k/v [B,Hq|Hkv,T,D] (pre-RoPE), out [B,Hq,T,D], lse [B,Hq,T] or NULL.
void oracle_nsa_select(int B, int Hq, int Hkv, int T, int D, const double* q, const double* k_pre,
                       const double* v, int window, int block, int n_select, double scale, double theta,
                       int rope_len, const int32_t* sel_in, int32_t* sel_out, double* out, double* lse) {
    const int G = Hq / Hkv;
    const int nblk = T / block;
    const long long NKV = static_cast<long long>(B) * Hkv;
    std::vector<double> pk(static_cast<size_t>(NKV) * nblk * D), pv(static_cast<size_t>(NKV) * nblk * D);
    oracle_pool_rope(NKV, T, D, block, theta, rope_len, k_pre, v, pk.data(), pv.data());
    std::vector<double> k_rot;
    const double* kk = k_pre;
    if (theta > 0.0) {
        k_rot = rotate_rows(k_pre, NKV, T, D, theta);
        kk = k_rot.data();
    }
    const long long rows = static_cast<long long>(B) * Hq * T;
#pragma omp parallel for schedule(dynamic, 16)
    for (long long r = 0; r < rows; ++r) {
        const int t = static_cast<int>(r % T);
        const int h = static_cast<int>((r / T) % Hq);
        const int b = static_cast<int>(r / (static_cast<long long>(T) * Hq));
        const size_t nk = static_cast<size_t>(b) * Hkv + h / G;
        std::vector<double> qrow(D);
        if (theta > 0.0) rope_rotate(q + r * D, qrow.data(), D, theta, t);
        else for (int d = 0; d < D; ++d) qrow[d] = q[r * D + d];
        std::vector<int> chosen;
        if (sel_in) {
            for (int i = 0; i < n_select; ++i)
                if (sel_in[r * n_select + i] >= 0) chosen.push_back(sel_in[r * n_select + i]);
        } else {
            std::vector<std::pair<double, int>> cand;  // (-score, j): ascending = best first, lower j on ties
            for (int j = 0; j < nblk; ++j) {
                if (!visible_pooled(t, j, window, block)) continue;
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += qrow[d] * pk[(nk * nblk + j) * D + d];
                cand.push_back({-scale * dot, j});
            }
            std::sort(cand.begin(), cand.end());
            for (size_t i = 0; i < cand.size() && static_cast<int>(i) < n_select; ++i) chosen.push_back(cand[i].second);
        }
        if (sel_out)
            for (int i = 0; i < n_select; ++i)
                sel_out[r * n_select + i] = i < static_cast<int>(chosen.size()) ? chosen[i] : -1;
        std::vector<const double*> keys, vals;
        for (int j : chosen)
            for (int u = 0; u < block; ++u) {
                const size_t row = nk * T + static_cast<size_t>(j) * block + u;
                keys.push_back(kk + row * D);
                vals.push_back(v + row * D);
            }
        attend_row(qrow.data(), keys, vals, D, scale, out + r * D, lse ? lse + r : nullptr);
    }
}

}  // extern "C"
