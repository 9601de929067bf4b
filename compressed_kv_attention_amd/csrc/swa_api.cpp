// swa_api.cpp -- the C ABI of libswa.so (declared in include/swa.h).
//
// Every entry point validates its arguments on the host before any HIP call,
// then enqueues kernels on the caller's stream.  Nothing here allocates,
// frees or synchronises, and no state survives a call except the
// thread-local text of the last error.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/swa.h"
#include "swa_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return SWA_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SWA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, ...)                                  \
    do {                                                    \
        if (!(cond)) return fail(SWA_ERR_INVALID, __VA_ARGS__); \
    } while (0)

#define REQUIRE_PTR(p)                                                          \
    do {                                                                        \
        if ((p) == nullptr) return fail(SWA_ERR_INVALID, "%s must not be NULL", #p); \
        if (!aligned16(p)) return fail(SWA_ERR_INVALID, "%s is not 16-byte aligned", #p); \
    } while (0)

#define OPTIONAL_PTR(p)                                                            \
    do {                                                                           \
        if ((p) != nullptr && !aligned16(p))                                       \
            return fail(SWA_ERR_INVALID, "%s is not 16-byte aligned", #p);         \
    } while (0)

// Shared validation of prefill parameters; fills the kernel argument block.
int check_prefill(const swa_prefill_params* p, const int32_t* seg_ids, const uint8_t* prefix, swa::PrefillArgs& a) {
    REQUIRE(p != nullptr, "params must not be NULL");
    REQUIRE(p->B >= 0 && p->T >= 0, "B and T must be >= 0 (B=%d, T=%d)", p->B, p->T);
    REQUIRE(p->Hq > 0 && p->Hkv > 0, "Hq and Hkv must be > 0 (Hq=%d, Hkv=%d)", p->Hq, p->Hkv);
    REQUIRE(p->Hq % p->Hkv == 0, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
    REQUIRE(p->window >= 0, "window must be >= 0 (got %d)", p->window);
    REQUIRE(p->compress_block >= 0, "compress_block must be >= 0 (got %d)", p->compress_block);
    REQUIRE(p->rope_len >= 0, "rope_len must be >= 0 (got %d)", p->rope_len);
    REQUIRE(p->scale >= 0.f && std::isfinite(p->scale), "scale must be finite and >= 0");
    REQUIRE(p->dtype == SWA_F32 || p->dtype == SWA_BF16, "dtype must be SWA_F32 or SWA_BF16 (got %d)", p->dtype);
    if (p->D != 32 && p->D != 64) return fail(SWA_ERR_UNSUPPORTED, "head dim D=%d is not built (32 or 64)", p->D);
    if (p->T > swa::kMaxT) return fail(SWA_ERR_UNSUPPORTED, "T=%d exceeds the supported %d", p->T, swa::kMaxT);
    if (p->compress_block > 0) {
        REQUIRE(p->window >= 1, "compressed mode needs window >= 1 (got %d)", p->window);
        if (seg_ids != nullptr || prefix != nullptr)
            return fail(SWA_ERR_UNSUPPORTED, "compressed mode takes no seg_ids or prefix");
    }
    if (p->rope_len > 0) REQUIRE(p->rope_len >= p->T, "rope_len (%d) must be >= T (%d)", p->rope_len, p->T);
    OPTIONAL_PTR(seg_ids);
    OPTIONAL_PTR(prefix);
    a = swa::PrefillArgs{};
    a.B = p->B;
    a.Hq = p->Hq;
    a.Hkv = p->Hkv;
    a.T = p->T;
    a.D = p->D;
    a.window = p->window;
    a.block = p->compress_block;
    a.nblk = p->compress_block > 0 ? p->T / p->compress_block : 0;
    a.rope_len = p->rope_len;
    a.scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->D);
    a.seg = seg_ids;
    a.prefix = prefix;
    a.kinfo = nullptr;
    a.ksub = nullptr;
    a.tsink = nullptr;
    a.ntile = (p->T + 63) / 64;
    const swa::MfmaGeom g = swa::mfma_geometry(p->Hq / p->Hkv);
    a.hpw = g.hpw;
    a.rbs = g.rbs;
    return SWA_OK;
}

// Workspace layout of a prefill: [key metadata, bf16 plain mode only:
// packed key info, sub-tile summaries, tile sink ranges] [rotated keys, with
// RoPE only]; each part starts 256-byte aligned.
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
struct MetaLayout {
    size_t info, ksub, tsink, total;  // byte offsets and size
};
MetaLayout key_meta_layout(const swa_prefill_params* p) {
    MetaLayout m{0, 0, 0, 0};
    if (p->dtype != SWA_BF16 || p->compress_block != 0) return m;
    const size_t ntile = ((size_t)p->T + 63) / 64;
    m.info = 0;
    m.ksub = round256((size_t)p->B * p->T * sizeof(int32_t));
    m.tsink = m.ksub + round256((size_t)p->B * 2 * ntile * 4 * sizeof(int32_t));
    m.total = m.tsink + round256((size_t)p->B * ntile * 2 * sizeof(int32_t));
    return m;
}
size_t rotated_key_bytes(const swa_prefill_params* p) {
    if (p->rope_len <= 0) return 0;
    const size_t elem = p->dtype == SWA_BF16 ? 2 : 4;
    return round256((size_t)p->B * p->Hkv * p->T * p->D * elem);
}
// Compressed mode: room for one pooled tensor (keys or values), used when the
// caller passes no pooled_k / pooled_v and the call pools them itself.
size_t pooled_bytes(const swa_prefill_params* p) {
    if (p->compress_block <= 0) return 0;
    const size_t elem = p->dtype == SWA_BF16 ? 2 : 4;
    return round256((size_t)p->B * p->Hkv * (size_t)(p->T / p->compress_block) * p->D * elem);
}

}  // namespace

extern "C" {

const char* swa_last_error(void) { return g_last_error.c_str(); }

int swa_version(void) { return 100; }

size_t swa_prefill_workspace_size(const swa_prefill_params* p) {
    if (p == nullptr || p->B <= 0 || p->T <= 0 || p->Hkv <= 0 || p->D <= 0) return 0;
    return key_meta_layout(p).total + rotated_key_bytes(p) + 2 * pooled_bytes(p);
}

}  // extern "C"

namespace {
// Sources of a prefill whose queries and keys are not one [T] sequence each:
// the queries (and outputs) hold rows q_first .. T - 1; keys before kv_split
// come from the call's k / v (kv_split rows per head), the rest from k2 / v2.
struct SplitSources {
    int q_first, kv_split;
    const void* k2;
    const void* v2;
    bool meta_ready;  // the key metadata is already in the workspace (no pre-pass)
};

int prefill_run(const swa_prefill_params* p, const void* q, const void* k, const void* v, const void* pooled_k,
                const void* pooled_v, const int32_t* seg_ids, const uint8_t* prefix, const float* rope_cos,
                const float* rope_sin, void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream,
                const SplitSources* split) {
    swa::PrefillArgs a;
    int rc = check_prefill(p, seg_ids, prefix, a);
    if (rc != SWA_OK) return rc;
    if (split != nullptr) {
        REQUIRE(p->dtype == SWA_BF16 && p->rope_len == 0 && p->compress_block == 0 && split->q_first % 64 == 0 &&
                    split->kv_split % 64 == 0 && split->q_first <= p->T && split->kv_split <= p->T &&
                    split->k2 != nullptr && split->v2 != nullptr,
                "split prefill sources out of range");
        a.q_first = split->q_first;
        a.kv_split = split->kv_split;
        a.k2 = split->k2;
        a.v2 = split->v2;
    }
    if (p->B == 0 || p->T == 0) return ok();
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(lse);
    // compressed mode without pooled inputs: the call pools k and v itself
    const bool pool_here = p->compress_block > 0 && a.nblk > 0 && pooled_k == nullptr && pooled_v == nullptr;
    if (p->compress_block > 0 && a.nblk > 0 && !pool_here) {
        REQUIRE_PTR(pooled_k);
        REQUIRE_PTR(pooled_v);
    }
    if (p->rope_len > 0) {
        REQUIRE_PTR(rope_cos);
        REQUIRE_PTR(rope_sin);
    }
    const size_t ws_need = swa_prefill_workspace_size(p);
    if (ws_need > 0) {
        REQUIRE(workspace != nullptr && ((uintptr_t)workspace & 255u) == 0,
                "workspace must be a 256-byte aligned buffer of swa_prefill_workspace_size() bytes");
        REQUIRE(workspace_bytes >= ws_need, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, ws_need);
    }
    a.q = q;
    a.k = k;
    a.v = v;
    a.pk = pooled_k;
    a.pv = pooled_v;
    a.rope_cos = p->rope_len > 0 ? rope_cos : nullptr;
    a.rope_sin = p->rope_len > 0 ? rope_sin : nullptr;
    a.out = out;
    a.lse = lse;
    const hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    const MetaLayout meta = key_meta_layout(p);
    void* kr = p->rope_len > 0 ? ws + meta.total : nullptr;  // rotated keys
    bool rotated = false;  // the exact keys are already in kr
    if (pool_here) {
        char* pk = ws + meta.total + rotated_key_bytes(p);
        char* pv = pk + pooled_bytes(p);
        a.pk = pk;
        a.pv = pv;
        hipError_t e;
        if (p->dtype == SWA_BF16 && kr != nullptr && swa::pool_rotate_fits(p->D, p->compress_block) &&
            (long long)p->B * p->Hkv <= 65535) {
            // one pass: rotated exact keys and the pooled keys and values
            swa::PoolRotArgs pr{};
            pr.N = p->B * p->Hkv;
            pr.T = p->T;
            pr.D = p->D;
            pr.block = p->compress_block;
            pr.nblk = a.nblk;
            pr.rope_len = p->rope_len;
            pr.k = (const uint16_t*)k;
            pr.v = (const uint16_t*)v;
            pr.cs = rope_cos;
            pr.sn = rope_sin;
            pr.kr = (uint16_t*)kr;
            pr.pk = (uint16_t*)pk;
            pr.pv = (uint16_t*)pv;
            e = swa::launch_pool_rotate_bf16(pr, s);
            rotated = true;
        } else {
            e = swa::launch_pool_rope(p->B, p->Hkv, p->T, p->D, p->compress_block, p->dtype, k, v,
                                      p->rope_len > 0 ? rope_cos : nullptr, p->rope_len > 0 ? rope_sin : nullptr,
                                      p->rope_len, pk, pv, s);
        }
        if (e != hipSuccess) return hip_status(e, "swa_attn_prefill pooling launch");
    }
    if (p->dtype == SWA_BF16) {
        swa::PrepArgs pa{};
        pa.B = p->B;
        pa.T = p->T;
        pa.D = p->D;
        pa.ntile = a.ntile;
        pa.div_T = swa::make_fastdiv((uint32_t)p->T);
        if (kr && !rotated) {  // rotate the exact keys once, into the workspace
            pa.rope_rows = (long long)p->B * p->Hkv * p->T;
            pa.rope_blocks = (pa.rope_rows * (p->D / 16) + 255) / 256;
            pa.x = (const uint16_t*)k;
            pa.cs = rope_cos;
            pa.sn = rope_sin;
            pa.y = (uint16_t*)kr;
        }
        if (meta.total > 0 && (a.seg || a.prefix) && split != nullptr && split->meta_ready) {
            a.kinfo = (const int32_t*)(ws + meta.info);
            a.ksub = (const int32_t*)(ws + meta.ksub);
            a.tsink = (const int32_t*)(ws + meta.tsink);
        } else if (meta.total > 0 && (a.seg || a.prefix)) {  // key metadata once per prefill
            pa.seg = a.seg;
            pa.prefix = a.prefix;
            pa.info = (int32_t*)(ws + meta.info);
            pa.ksub = (int32_t*)(ws + meta.ksub);
            pa.tsink = (int32_t*)(ws + meta.tsink);
            a.kinfo = pa.info;
            a.ksub = pa.ksub;
            a.tsink = pa.tsink;
        }
        if (pa.rope_blocks > 0 || pa.info != nullptr) {
            const hipError_t e = swa::launch_prefill_prep(pa, s);
            if (e != hipSuccess) return hip_status(e, "swa_attn_prefill prep launch");
        }
    } else if (kr) {
        const hipError_t e = swa::launch_rope_rows_f32((long long)p->B * p->Hkv * p->T, p->T, p->D, (const float*)k,
                                                       rope_cos, rope_sin, (float*)kr, s);
        if (e != hipSuccess) return hip_status(e, "swa_attn_prefill key rotation launch");
    }
    if (kr) a.k = kr;
    const hipError_t e = p->dtype == SWA_BF16 ? swa::launch_prefill_bf16(a, s) : swa::launch_prefill_f32(a, s);
    return hip_status(e, "swa_attn_prefill launch");
}
}  // namespace

extern "C" {

int swa_attn_prefill(const swa_prefill_params* p, const void* q, const void* k, const void* v, const void* pooled_k,
                     const void* pooled_v, const int32_t* seg_ids, const uint8_t* prefix, const float* rope_cos,
                     const float* rope_sin, void* out, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream) {
    return prefill_run(p, q, k, v, pooled_k, pooled_v, seg_ids, prefix, rope_cos, rope_sin, out, lse, workspace,
                       workspace_bytes, stream, nullptr);
}

int swa_debug_visibility(const swa_prefill_params* p, const int32_t* seg_ids, const uint8_t* prefix,
                         uint8_t* mask_out, int32_t* count_out, void* workspace, size_t workspace_bytes,
                         void* stream) {
    swa::PrefillArgs a;
    int rc = check_prefill(p, seg_ids, prefix, a);
    if (rc != SWA_OK) return rc;
    if (mask_out != nullptr && p->T > swa::kDebugMaxT)
        return fail(SWA_ERR_UNSUPPORTED, "swa_debug_visibility writes masks for T <= %d (got %d)", swa::kDebugMaxT,
                    p->T);
    if (p->B == 0 || p->T == 0) return ok();
    REQUIRE_PTR(count_out);
    OPTIONAL_PTR(mask_out);
    const hipStream_t s = (hipStream_t)stream;
    if (p->dtype != SWA_BF16) {
        if (p->T > swa::kDebugMaxT)
            return fail(SWA_ERR_UNSUPPORTED, "swa_debug_visibility (fp32) supports T <= %d (got %d)", swa::kDebugMaxT,
                        p->T);
        return hip_status(swa::launch_debug_visibility(a, false, mask_out, count_out, s), "swa_debug_visibility launch");
    }
    // bf16: the MFMA kernel's own walk and masks, fed by the same key-metadata
    // pre-pass as a prefill call (rope_len is irrelevant to visibility)
    swa_prefill_params pm = *p;
    pm.rope_len = 0;
    const MetaLayout meta = key_meta_layout(&pm);
    if (meta.total > 0 && (seg_ids || prefix)) {
        REQUIRE(workspace != nullptr && ((uintptr_t)workspace & 255u) == 0,
                "workspace must be a 256-byte aligned buffer of swa_prefill_workspace_size() bytes");
        REQUIRE(workspace_bytes >= meta.total, "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
                meta.total);
        char* ws = (char*)workspace;
        swa::PrepArgs pa{};
        pa.B = p->B;
        pa.T = p->T;
        pa.D = p->D;
        pa.ntile = a.ntile;
        pa.div_T = swa::make_fastdiv((uint32_t)p->T);
        pa.seg = seg_ids;
        pa.prefix = prefix;
        pa.info = (int32_t*)(ws + meta.info);
        pa.ksub = (int32_t*)(ws + meta.ksub);
        pa.tsink = (int32_t*)(ws + meta.tsink);
        a.kinfo = pa.info;
        a.ksub = pa.ksub;
        a.tsink = pa.tsink;
        const hipError_t e = swa::launch_prefill_prep(pa, s);
        if (e != hipSuccess) return hip_status(e, "swa_debug_visibility prep launch");
    }
    a.rope_len = 0;
    return hip_status(swa::launch_prefill_bf16_dump(a, mask_out, count_out, s), "swa_debug_visibility launch");
}

int swa_rope_table(double theta, int rope_len, int D, float* cos_out, float* sin_out, void* stream) {
    REQUIRE(theta > 0.0 && std::isfinite(theta), "theta must be finite and > 0");
    REQUIRE(rope_len >= 0, "rope_len must be >= 0 (got %d)", rope_len);
    REQUIRE(D > 0 && D % 2 == 0, "D must be positive and even (got %d)", D);
    if (rope_len == 0) return ok();
    REQUIRE_PTR(cos_out);
    REQUIRE_PTR(sin_out);
    return hip_status(swa::launch_rope_table(theta, rope_len, D, cos_out, sin_out, (hipStream_t)stream),
                      "swa_rope_table launch");
}

int swa_rope_table_host(double theta, int rope_len, int D, float* cos_out, float* sin_out) {
    REQUIRE(theta > 0.0 && std::isfinite(theta), "theta must be finite and > 0");
    REQUIRE(rope_len >= 0, "rope_len must be >= 0 (got %d)", rope_len);
    REQUIRE(D > 0 && D % 2 == 0, "D must be positive and even (got %d)", D);
    if (rope_len == 0) return ok();
    REQUIRE(cos_out != nullptr && sin_out != nullptr, "cos_out and sin_out must not be NULL");
    const int half = D / 2;
    for (int i = 0; i < half; ++i) {
        const double inv_freq = std::pow(theta, -2.0 * (double)i / (double)D);
        for (int pos = 0; pos < rope_len; ++pos) {
            const double ang = (double)pos * inv_freq;
            cos_out[(size_t)pos * half + i] = (float)std::cos(ang);
            sin_out[(size_t)pos * half + i] = (float)std::sin(ang);
        }
    }
    return ok();
}

int kv_pool_compress_rope(int B, int H, int T, int D, int block, int dtype, const void* k_pre, const void* v,
                          const float* rope_cos, const float* rope_sin, int rope_len, void* pooled_k, void* pooled_v,
                          void* stream) {
    REQUIRE(B >= 0 && H > 0 && T >= 0, "bad shape (B=%d, H=%d, T=%d)", B, H, T);
    REQUIRE(block >= 1, "block must be >= 1 (got %d)", block);
    REQUIRE(dtype == SWA_F32 || dtype == SWA_BF16, "dtype must be SWA_F32 or SWA_BF16 (got %d)", dtype);
    REQUIRE(D > 0 && D % 2 == 0, "D must be positive and even (got %d)", D);
    REQUIRE(rope_len >= 0, "rope_len must be >= 0 (got %d)", rope_len);
    if (B == 0 || T / block == 0) return ok();
    REQUIRE_PTR(k_pre);
    REQUIRE_PTR(v);
    REQUIRE_PTR(pooled_k);
    REQUIRE_PTR(pooled_v);
    const bool rope = rope_cos != nullptr || rope_sin != nullptr || rope_len > 0;
    if (rope) {
        REQUIRE_PTR(rope_cos);
        REQUIRE_PTR(rope_sin);
        REQUIRE(rope_len >= 1, "rope_len must be >= 1 with RoPE tables");
    }
    return hip_status(swa::launch_pool_rope(B, H, T, D, block, dtype, k_pre, v, rope ? rope_cos : nullptr,
                                            rope ? rope_sin : nullptr, rope_len, pooled_k, pooled_v,
                                            (hipStream_t)stream),
                      "kv_pool_compress_rope launch");
}

int swa_kv_quantize(long long N, int D, const void* x_bf16, int8_t* xq, float* xs, void* stream) {
    REQUIRE(N >= 0, "N must be >= 0");
    REQUIRE(D > 0 && D % 32 == 0, "D must be a positive multiple of 32 (got %d)", D);
    if (N == 0) return ok();
    REQUIRE_PTR(x_bf16);
    REQUIRE_PTR(xq);
    REQUIRE_PTR(xs);
    return hip_status(swa::launch_kv_quantize(N, D, x_bf16, xq, xs, (hipStream_t)stream), "swa_kv_quantize launch");
}

namespace {
// Split count a decode call runs with (0 = automatic), or -1 if invalid.
int resolve_splits(const swa_decode_params* p) {
    if (p->num_splits < 0 || p->num_splits > swa::kMaxDecodeSplits) return -1;
    if (p->num_splits > 0) return p->num_splits;
    return swa::decode_auto_splits(p->B, p->Hq, p->Hkv, p->W, p->S);
}
}  // namespace

size_t swa_decode_workspace_size(const swa_decode_params* p) {
    if (p == nullptr || p->B <= 0 || p->Hkv <= 0 || p->Hq <= 0 || p->Hq % p->Hkv != 0 || p->D <= 0 || p->W < 1 ||
        p->S < 0)
        return 0;
    const int splits = resolve_splits(p);
    if (splits < 0) return 0;
    return swa::decode_workspace_layout(p->B, p->Hq, p->Hkv, p->D, splits).total;
}

}  // extern "C"

namespace {
// Validation shared by both decode entry points; fills the argument block and
// the split-K workspace layout (the caller decides where that memory is).
int check_decode(const swa_decode_params* p, const void* q, const void* k_new, const void* v_new, int8_t* ring_k,
                 int8_t* ring_v, float* ring_ks, float* ring_vs, const int8_t* sink_k, const int8_t* sink_v,
                 const float* sink_ks, const float* sink_vs, const int32_t* pos, const int32_t* sink_len, void* out,
                 swa::DecodeArgs& a, swa::DecodeWorkspace& wl, bool& empty) {
    empty = false;
    REQUIRE(p != nullptr, "params must not be NULL");
    REQUIRE(p->B >= 0, "B must be >= 0");
    REQUIRE(p->Hq > 0 && p->Hkv > 0 && p->Hq % p->Hkv == 0, "Hq (%d) must be a positive multiple of Hkv (%d)", p->Hq,
            p->Hkv);
    REQUIRE(p->W >= 1, "W must be >= 1 (got %d)", p->W);
    REQUIRE(p->S >= 0, "S must be >= 0 (got %d)", p->S);
    REQUIRE(p->scale >= 0.f && std::isfinite(p->scale), "scale must be finite and >= 0");
    REQUIRE(p->num_splits >= 0 && p->num_splits <= swa::kMaxDecodeSplits, "num_splits must be in [0, %d] (got %d)",
            swa::kMaxDecodeSplits, p->num_splits);
    if (p->D != 32 && p->D != 64) return fail(SWA_ERR_UNSUPPORTED, "head dim D=%d is not built (32 or 64)", p->D);
    REQUIRE((k_new == nullptr) == (v_new == nullptr), "k_new and v_new must both be given or both be NULL");
    if (p->B == 0) {
        empty = true;
        return SWA_OK;
    }
    const int splits = resolve_splits(p);
    wl = swa::decode_workspace_layout(p->B, p->Hq, p->Hkv, p->D, splits);
    REQUIRE_PTR(q);
    REQUIRE_PTR(ring_k);
    REQUIRE_PTR(ring_v);
    REQUIRE_PTR(ring_ks);
    REQUIRE_PTR(ring_vs);
    REQUIRE_PTR(pos);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(k_new);
    OPTIONAL_PTR(v_new);
    OPTIONAL_PTR(sink_len);
    if (p->S > 0) {
        REQUIRE_PTR(sink_k);
        REQUIRE_PTR(sink_v);
        REQUIRE_PTR(sink_ks);
        REQUIRE_PTR(sink_vs);
    }
    a = swa::DecodeArgs{};
    a.q = q;
    a.k_new = k_new;
    a.v_new = v_new;
    a.ring_k = ring_k;
    a.ring_v = ring_v;
    a.ring_ks = ring_ks;
    a.ring_vs = ring_vs;
    a.sink_k = p->S > 0 ? sink_k : nullptr;
    a.sink_v = p->S > 0 ? sink_v : nullptr;
    a.sink_ks = p->S > 0 ? sink_ks : nullptr;
    a.sink_vs = p->S > 0 ? sink_vs : nullptr;
    a.pos = pos;
    a.sink_len = sink_len;
    a.out = out;
    a.B = p->B;
    a.Hq = p->Hq;
    a.Hkv = p->Hkv;
    a.D = p->D;
    a.W = p->W;
    a.S = p->S;
    a.num_splits = splits;
    a.scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->D);
    return SWA_OK;
}
}  // namespace

extern "C" {

int swa_attn_decode(const swa_decode_params* p, const void* q, const void* k_new, const void* v_new, int8_t* ring_k,
                    int8_t* ring_v, float* ring_ks, float* ring_vs, const int8_t* sink_k, const int8_t* sink_v,
                    const float* sink_ks, const float* sink_vs, const int32_t* pos, const int32_t* sink_len,
                    void* out, void* workspace, size_t workspace_bytes, void* stream) {
    swa::DecodeArgs a;
    swa::DecodeWorkspace wl;
    bool empty;
    const int rc = check_decode(p, q, k_new, v_new, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks,
                                sink_vs, pos, sink_len, out, a, wl, empty);
    if (rc != SWA_OK) return rc;
    if (empty) return ok();
    if (wl.total > 0) {
        REQUIRE(workspace != nullptr && ((uintptr_t)workspace & 255u) == 0,
                "workspace must be a 256-byte aligned buffer of swa_decode_workspace_size() bytes (%d splits)",
                a.num_splits);
        REQUIRE(workspace_bytes >= wl.total, "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
                wl.total);
        char* ws = (char*)workspace;
        a.counters = (int*)(ws + wl.counters);
        a.part_ml = (float*)(ws + wl.part_ml);
        a.part_o = (float*)(ws + wl.part_o);
    }
    return hip_status(swa::launch_decode(a, (hipStream_t)stream), "swa_attn_decode launch");
}

int swa_attn_decode_noalloc(const swa_decode_params* p, const void* q, const void* k_new, const void* v_new,
                            int8_t* ring_k, int8_t* ring_v, float* ring_ks, float* ring_vs, const int8_t* sink_k,
                            const int8_t* sink_v, const float* sink_ks, const float* sink_vs, const int32_t* pos,
                            const int32_t* sink_len, void* out, void* stream) {
    swa::DecodeArgs a;
    swa::DecodeWorkspace wl;
    bool empty;
    const int rc = check_decode(p, q, k_new, v_new, ring_k, ring_v, ring_ks, ring_vs, sink_k, sink_v, sink_ks,
                                sink_vs, pos, sink_len, out, a, wl, empty);
    if (rc != SWA_OK) return rc;
    if (empty) return ok();
    if (wl.total > swa::kNoAllocScratchBytes)
        return fail(SWA_ERR_UNSUPPORTED,
                    "split-K state of %zu bytes (%d splits) exceeds the %zu bytes swa_attn_decode_noalloc holds; "
                    "use fewer splits or swa_attn_decode with a workspace",
                    wl.total, a.num_splits, swa::kNoAllocScratchBytes);
    return hip_status(swa::launch_decode_noalloc(a, wl, (hipStream_t)stream), "swa_attn_decode_noalloc launch");
}

int swa_attn_decode_compressed(const swa_decode_params* p, int block, const float* rope_cos, const float* rope_sin,
                               int rope_len, const void* q, const void* k_new, const void* k_new_pre,
                               const void* v_new, int8_t* ring_k, int8_t* ring_v, float* ring_ks, float* ring_vs,
                               int8_t* pool_k, int8_t* pool_v, float* pool_ks, float* pool_vs, float* front_k,
                               float* front_v, const int32_t* pos, void* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
    REQUIRE(block >= 1, "block must be >= 1 (got %d)", block);
    REQUIRE((rope_cos == nullptr) == (rope_sin == nullptr), "rope_cos and rope_sin must both be given or both be NULL");
    REQUIRE(rope_cos == nullptr || rope_len >= 1, "rope_len must be >= 1 with a table (got %d)", rope_len);
    swa::DecodeArgs a;
    swa::DecodeWorkspace wl;
    bool empty;
    const int rc = check_decode(p, q, k_new, v_new, ring_k, ring_v, ring_ks, ring_vs, pool_k, pool_v, pool_ks,
                                pool_vs, pos, nullptr, out, a, wl, empty);
    if (rc != SWA_OK) return rc;
    if (empty) return ok();
    REQUIRE_PTR(k_new);
    REQUIRE_PTR(v_new);
    REQUIRE_PTR(k_new_pre);
    REQUIRE_PTR(front_k);
    REQUIRE_PTR(front_v);
    OPTIONAL_PTR(rope_cos);
    OPTIONAL_PTR(rope_sin);
    a.block = block;
    a.k_pre = k_new_pre;
    a.front_k = front_k;
    a.front_v = front_v;
    a.pool_k = p->S > 0 ? pool_k : nullptr;
    a.pool_v = p->S > 0 ? pool_v : nullptr;
    a.pool_ks = p->S > 0 ? pool_ks : nullptr;
    a.pool_vs = p->S > 0 ? pool_vs : nullptr;
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    a.rope_len = rope_cos ? rope_len : 0;
    if (wl.total > 0) {
        REQUIRE(workspace != nullptr && ((uintptr_t)workspace & 255u) == 0,
                "workspace must be a 256-byte aligned buffer of swa_decode_workspace_size() bytes (%d splits)",
                a.num_splits);
        REQUIRE(workspace_bytes >= wl.total, "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
                wl.total);
        char* ws = (char*)workspace;
        a.counters = (int*)(ws + wl.counters);
        a.part_ml = (float*)(ws + wl.part_ml);
        a.part_o = (float*)(ws + wl.part_o);
    }
    return hip_status(swa::launch_decode(a, (hipStream_t)stream), "swa_attn_decode_compressed launch");
}

size_t swa_nsa_select_workspace_size(const swa_prefill_params* p) {
    if (p == nullptr || p->B <= 0 || p->T <= 0 || p->Hkv <= 0 || p->D <= 0 || p->compress_block <= 0) return 0;
    const size_t elem = p->dtype == SWA_BF16 ? 2 : 4;
    const size_t nk = p->rope_len > 0 ? (size_t)p->B * p->Hkv * p->T * p->D * elem : 0;  // rotated keys
    const size_t np = (size_t)p->B * p->Hkv * (p->T / p->compress_block) * p->D * 4;    // fp32 pooled keys
    return round256(nk) + round256(np);
}

int swa_nsa_select_attn(const swa_prefill_params* p, int n_select, const void* q, const void* k, const void* v,
                        const float* rope_cos, const float* rope_sin, void* out, float* lse, int32_t* sel,
                        void* workspace, size_t workspace_bytes, void* stream) {
    swa::PrefillArgs pa;
    int rc = check_prefill(p, nullptr, nullptr, pa);
    if (rc != SWA_OK) return rc;
    REQUIRE(p->compress_block >= 1, "compress_block (the block size) must be >= 1 (got %d)", p->compress_block);
    REQUIRE(n_select >= 1 && n_select <= 32, "n_select must be in [1, 32] (got %d)", n_select);
    if (p->B > 65535 || p->Hq > 65535) return fail(SWA_ERR_UNSUPPORTED, "B and Hq must be <= 65535");
    if (p->B == 0 || p->T == 0) return ok();
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(lse);
    OPTIONAL_PTR(sel);
    if (p->rope_len > 0) {
        REQUIRE_PTR(rope_cos);
        REQUIRE_PTR(rope_sin);
    }
    const size_t need = swa_nsa_select_workspace_size(p);
    REQUIRE(workspace != nullptr && ((uintptr_t)workspace & 255u) == 0,
            "workspace must be a 256-byte aligned buffer of swa_nsa_select_workspace_size() bytes");
    REQUIRE(workspace_bytes >= need, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
    swa::NsaArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.rope_cos = p->rope_len > 0 ? rope_cos : nullptr;
    a.rope_sin = p->rope_len > 0 ? rope_sin : nullptr;
    a.out = out;
    a.lse = lse;
    a.sel = sel;
    a.B = p->B;
    a.Hq = p->Hq;
    a.Hkv = p->Hkv;
    a.T = p->T;
    a.D = p->D;
    a.window = p->window;
    a.block = p->compress_block;
    a.nblk = p->T / p->compress_block;
    a.n_select = n_select;
    a.rope_len = p->rope_len;
    a.dtype = p->dtype == SWA_BF16 ? 1 : 0;
    a.scale = pa.scale;
    const size_t elem = p->dtype == SWA_BF16 ? 2 : 4;
    const size_t nk = p->rope_len > 0 ? round256((size_t)p->B * p->Hkv * p->T * p->D * elem) : 0;
    char* ws = (char*)workspace;
    return hip_status(swa::launch_nsa_select(a, ws, (float*)(ws + nk), (hipStream_t)stream),
                      "swa_nsa_select_attn launch");
}

}  // extern "C"

namespace {
// Workspace of a backward call: fp32 q, dO, k, v and Delta, 256-byte aligned parts.
struct BwdLayout {
    size_t q32, do32, k32, v32, delta, pk, pv, total;
};
BwdLayout bwd_layout(const swa_prefill_params* p) {
    BwdLayout L{0, 0, 0, 0, 0, 0, 0, 0};
    const size_t nq = (size_t)p->B * p->Hq * p->T * p->D * 4, nk = (size_t)p->B * p->Hkv * p->T * p->D * 4;
    L.do32 = round256(nq);
    L.k32 = L.do32 + round256(nq);
    L.v32 = L.k32 + round256(nk);
    L.delta = L.v32 + round256(nk);
    L.pk = L.delta + round256((size_t)p->B * p->Hq * p->T * 4);
    const size_t part = p->Hq != p->Hkv ? round256(nq) : 0;  // per-head dk/dv shares
    L.pv = L.pk + part;
    L.total = L.pv + part;
    return L;
}
}  // namespace

extern "C" {

size_t swa_prefill_backward_workspace_size(const swa_prefill_params* p) {
    if (p == nullptr || p->B <= 0 || p->T <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->D <= 0) return 0;
    return bwd_layout(p).total;
}

int swa_attn_prefill_backward(const swa_prefill_params* p, const void* q, const void* k, const void* v,
                              const void* out, const float* lse, const void* dout, const int32_t* seg_ids,
                              const uint8_t* prefix, const float* rope_cos, const float* rope_sin, float* dq,
                              float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream) {
    swa::PrefillArgs pa;
    int rc = check_prefill(p, seg_ids, prefix, pa);
    if (rc != SWA_OK) return rc;
    if (p->compress_block != 0)
        return fail(SWA_ERR_UNSUPPORTED, "the backward is built for plain mode (compress_block 0)");
    if (p->T > 65535 * 32) return fail(SWA_ERR_UNSUPPORTED, "T=%d too long for the backward grid", p->T);
    if (p->B > 65535 || p->Hq > 65535) return fail(SWA_ERR_UNSUPPORTED, "B and Hq must be <= 65535");
    if (p->B == 0 || p->T == 0) return ok();
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(out);
    REQUIRE_PTR(lse);
    REQUIRE_PTR(dout);
    REQUIRE_PTR(dq);
    REQUIRE_PTR(dk);
    REQUIRE_PTR(dv);
    if (p->rope_len > 0) {
        REQUIRE_PTR(rope_cos);
        REQUIRE_PTR(rope_sin);
    }
    const BwdLayout L = bwd_layout(p);
    REQUIRE(workspace != nullptr && ((uintptr_t)workspace & 255u) == 0,
            "workspace must be a 256-byte aligned buffer of swa_prefill_backward_workspace_size() bytes");
    REQUIRE(workspace_bytes >= L.total, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, L.total);
    swa::BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.dout = dout;
    a.lse = lse;
    a.seg = seg_ids;
    a.prefix = prefix;
    a.rope_cos = p->rope_len > 0 ? rope_cos : nullptr;
    a.rope_sin = p->rope_len > 0 ? rope_sin : nullptr;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.B = p->B;
    a.Hq = p->Hq;
    a.Hkv = p->Hkv;
    a.T = p->T;
    a.D = p->D;
    a.window = p->window;
    a.dtype = p->dtype == SWA_BF16 ? 1 : 0;
    a.scale = pa.scale;
    char* ws = (char*)workspace;
    const swa::BwdWorkspace w{(float*)(ws + L.q32), (float*)(ws + L.k32), (float*)(ws + L.v32),
                              (float*)(ws + L.do32), (float*)(ws + L.delta), (float*)(ws + L.pk),
                              (float*)(ws + L.pv)};
    return hip_status(swa::launch_prefill_backward(a, w, (hipStream_t)stream), "swa_attn_prefill_backward launch");
}

}  // extern "C"

namespace {
// Workspace layout of a chunked prefill: the staged cached rows of k and v
// (C = S + W - 1 rounded up to 64 per kv head), segment ids and prefix flags
// of the C + Tc keys, then the prefill workspace of that key sequence.
struct ChunkLayout {
    size_t k, v, seg, prefix, pf, pf_bytes, total;
    int C;
    swa_prefill_params pp;
};
bool chunk_layout(const swa_chunk_params* p, ChunkLayout& L) {
    if (p == nullptr || p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->D <= 0 || p->W < 1 || p->S < 0 || p->Tc <= 0)
        return false;
    const long long C = ((long long)p->S + p->W - 1 + 63) / 64 * 64;
    const long long Tv = C + p->Tc;
    if (Tv > swa::kMaxT) return false;
    L.C = (int)C;
    L.pp = swa_prefill_params{p->B, p->Hq, p->Hkv, (int)Tv, p->D, p->W, 0, 0, p->scale, SWA_BF16};
    const size_t kb = (size_t)p->B * p->Hkv * C * p->D * 2;
    L.k = 0;
    L.v = L.k + round256(kb);
    L.seg = L.v + round256(kb);
    L.prefix = L.seg + round256((size_t)p->B * Tv * 4);
    L.pf = L.prefix + round256((size_t)p->B * Tv);
    L.pf_bytes = swa_prefill_workspace_size(&L.pp);
    L.total = L.pf + round256(L.pf_bytes);
    return true;
}
}  // namespace

extern "C" {

size_t swa_chunk_prefill_workspace_size(const swa_chunk_params* p) {
    ChunkLayout L;
    return chunk_layout(p, L) ? L.total : 0;
}

int swa_attn_chunk_prefill(const swa_chunk_params* p, const void* q, const void* k, const void* v, int8_t* ring_k,
                           int8_t* ring_v, float* ring_ks, float* ring_vs, const int8_t* sink_k, const int8_t* sink_v,
                           const float* sink_ks, const float* sink_vs, const int32_t* pos0, const int32_t* sink_len,
                           void* out, void* workspace, size_t workspace_bytes, void* stream) {
    REQUIRE(p != nullptr, "params must not be NULL");
    REQUIRE(p->B >= 0 && p->Tc >= 0, "B and Tc must be >= 0 (B=%d, Tc=%d)", p->B, p->Tc);
    REQUIRE(p->Hq > 0 && p->Hkv > 0 && p->Hq % p->Hkv == 0, "Hq (%d) must be a positive multiple of Hkv (%d)", p->Hq,
            p->Hkv);
    REQUIRE(p->W >= 1, "W must be >= 1 (got %d)", p->W);
    REQUIRE(p->S >= 0, "S must be >= 0 (got %d)", p->S);
    REQUIRE(p->scale >= 0.f && std::isfinite(p->scale), "scale must be finite and >= 0");
    if (p->D != 32 && p->D != 64) return fail(SWA_ERR_UNSUPPORTED, "head dim D=%d is not built (32 or 64)", p->D);
    const long long cached = ((long long)p->S + p->W - 1 + 63) / 64 * 64;
    if (cached + p->Tc > swa::kMaxT)
        return fail(SWA_ERR_UNSUPPORTED, "S + W - 1 (rounded up to 64) + Tc = %lld exceeds the supported %d",
                    cached + p->Tc, swa::kMaxT);
    if ((long long)p->B * p->Hkv > 65535)
        return fail(SWA_ERR_UNSUPPORTED, "B * Hkv = %lld exceeds 65535", (long long)p->B * p->Hkv);
    if (p->B == 0 || p->Tc == 0) return ok();
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(ring_k);
    REQUIRE_PTR(ring_v);
    REQUIRE_PTR(ring_ks);
    REQUIRE_PTR(ring_vs);
    REQUIRE_PTR(pos0);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(sink_len);
    if (p->S > 0) {
        REQUIRE_PTR(sink_k);
        REQUIRE_PTR(sink_v);
        REQUIRE_PTR(sink_ks);
        REQUIRE_PTR(sink_vs);
    }
    ChunkLayout L;
    if (!chunk_layout(p, L)) return fail(SWA_ERR_INVALID, "chunk parameters out of range");
    REQUIRE(workspace != nullptr && ((uintptr_t)workspace & 255u) == 0,
            "workspace must be a 256-byte aligned buffer of swa_chunk_prefill_workspace_size() bytes");
    REQUIRE(workspace_bytes >= L.total, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, L.total);
    swa::ChunkArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.ring_k = ring_k;
    a.ring_v = ring_v;
    a.ring_ks = ring_ks;
    a.ring_vs = ring_vs;
    a.sink_k = p->S > 0 ? sink_k : nullptr;
    a.sink_v = p->S > 0 ? sink_v : nullptr;
    a.sink_ks = p->S > 0 ? sink_ks : nullptr;
    a.sink_vs = p->S > 0 ? sink_vs : nullptr;
    a.pos0 = pos0;
    a.sink_len = sink_len;
    a.out = out;
    a.B = p->B;
    a.Hq = p->Hq;
    a.Hkv = p->Hkv;
    a.D = p->D;
    a.W = p->W;
    a.S = p->S;
    a.Tc = p->Tc;
    a.C = L.C;
    a.Tv = L.pp.T;
    char* ws = (char*)workspace;
    // the prefill's key metadata, written by the staging into the prefill's
    // workspace where its pre-pass would have put it
    const MetaLayout meta = key_meta_layout(&L.pp);
    a.info = (int32_t*)(ws + L.pf + meta.info);
    a.ksub = (int32_t*)(ws + L.pf + meta.ksub);
    a.tsink = (int32_t*)(ws + L.pf + meta.tsink);
    a.ntile = (L.pp.T + 63) / 64;
    const hipStream_t s = (hipStream_t)stream;
    hipError_t e = swa::launch_chunk_stage(a, ws + L.k, ws + L.v, (int32_t*)(ws + L.seg), (uint8_t*)(ws + L.prefix), s);
    if (e != hipSuccess) return hip_status(e, "swa_attn_chunk_prefill staging launch");
    // queries and outputs in place (rows C .. Tv - 1 of the key sequence); keys
    // switch from the staged cached rows to the caller's chunk at row C
    const SplitSources split{L.C, L.C, k, v, true};
    const int rc = prefill_run(&L.pp, q, ws + L.k, ws + L.v, nullptr, nullptr, (const int32_t*)(ws + L.seg),
                               (const uint8_t*)(ws + L.prefix), nullptr, nullptr, out, nullptr,
                               L.pf_bytes ? ws + L.pf : nullptr, L.pf_bytes, stream, &split);
    if (rc != SWA_OK) return rc;
    e = swa::launch_chunk_finish(a, s);
    return hip_status(e, "swa_attn_chunk_prefill ring write launch");
}

long long swa_kv_budget_window(long long d_model, long long attn_dim, long long num_heads, long long num_kv_heads,
                               long long num_layers, long long sites, long long max_seq_len) {
    if (d_model <= 0 || num_heads <= 0 || num_kv_heads <= 0 || num_layers <= 0 || sites < 0 || max_seq_len <= 0 ||
        attn_dim < 0)
        return -1;
    // Bytes one cached position costs: per layer, K and V each hold one int8
    // code per channel and one fp32 scale per 32 channels; per engram site,
    // d_model bytes and one 128-byte record.
    constexpr long long kBudget = (23LL << 20) / 2;  // 11.5 MiB for the whole cache
    constexpr long long kScaleGroup = 32, kScaleBytes = sizeof(float), kFloor = 160;
    const long long channels = num_kv_heads * ((attn_dim > 0 ? attn_dim : d_model) / num_heads);
    const long long codes_and_scales = channels + kScaleBytes * (channels / kScaleGroup);
    const long long bytes_per_pos = num_layers * 2 * codes_and_scales + sites * (d_model + kScaleGroup * kScaleBytes);
    if (bytes_per_pos <= 0) return -1;
    const long long positions = kBudget / bytes_per_pos;
    const long long window = positions - positions % kScaleGroup;  // whole groups of 32 positions
    return std::max(kFloor, std::min(window, max_seq_len));          // the floor wins over the cap
}

long long swa_effective_kv_window(long long d_model, long long attn_dim, long long num_heads, long long num_kv_heads,
                                  long long num_layers, long long sites, long long max_seq_len, long long kv_window) {
    const long long w = swa_kv_budget_window(d_model, attn_dim, num_heads, num_kv_heads, num_layers, sites, max_seq_len);
    if (w < 0 || kv_window < 0) return -1;
    return kv_window != 0 && kv_window < w ? kv_window : w;
}

}  // extern "C"
