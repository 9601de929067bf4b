/* swa.h -- C ABI of libswa.so: windowed+sink GQA attention and compressed-KV
 * attention on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; cited by title and section):
 *   [NW] "How the 256-Token Sliding Window Works with Tools as KV Sinks in
 *        Needle" (instagit.com)
 *   [NS] "256-token滑动窗口+KV sink：Needle 2工具钉住机制源码分析" (cf-1.com)
 *   [CA] "Compressed attention and the copy probe" (octlm.ramaa.tech)
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers to contiguous row-major arrays owned
 *     by the caller, unless the comment says HOST.  The library never
 *     allocates, frees or synchronises; it keeps no state between calls and is
 *     safe to call from several threads.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns at once.
 *   - The return value is a status code.  Arguments are validated on the host
 *     before any HIP call; a non-OK status leaves outputs untouched and sets a
 *     thread-local message readable with swa_last_error().
 *   - Device pointers must be 16-byte aligned.
 *   - Empty problems (B == 0, T == 0, N == 0) return SWA_OK and launch nothing.
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWA_OK 0
#define SWA_ERR_INVALID 1     /* bad shape, argument, NULL or misaligned pointer */
#define SWA_ERR_UNSUPPORTED 2 /* valid request this library does not implement  */
#define SWA_ERR_HIP 3         /* a HIP launch or runtime error (message has the HIP text) */

typedef enum { SWA_F32 = 0, SWA_BF16 = 1 } swa_dtype;

/* Text of the last non-OK status on the calling thread ("" if none). */
const char* swa_last_error(void);
/* Library version, major*100 + minor. */
int swa_version(void);

/* ------------------------------------------------------------------------ */
/* Prefill attention.                                                        */
/*                                                                           */
/* Plain mode (compress_block == 0) computes, for every (b, query head h,     */
/* row t), softmax attention over the keys s that the packing mask of         */
/* [NW §"KV Sinks for Tools: Pinning Critical Context"] keeps:                */
/*   vis(t, s) = seg[t] > 0 && seg[s] == seg[t] && s <= t                     */
/*               && (window == 0 || t - s < window || prefix[s] != 0)         */
/* i.e. packing & causal & (recent | sink).  Sinks never leave the window but */
/* stay inside their own segment (the code composes the terms that way).      */
/* GQA: query head h reads kv head h / (Hq / Hkv).                            */
/*                                                                           */
/* Compressed mode (compress_block = b >= 1) follows [CA §"Two kinds of       */
/* columns, pooled blocks and exact recent keys"]: the columns are            */
/* [pooled blocks j < T/b, exact keys s < T]; pooled block j is visible to    */
/* row t iff (j + 1) * b <= t - window + 1 and exact key s iff s <= t and     */
/* t - s < window.  One softmax runs over both column sets.  pooled_k must   */
/* already be rotated (kv_pool_compress_rope does that); seg_ids and prefix   */
/* must be NULL and window >= 1.  With pooled_k and pooled_v both NULL the    */
/* call pools k and v itself (the arithmetic of kv_pool_compress_rope, into   */
/* the workspace): for bf16 with RoPE and b <= 256 / (D / 16), in the same    */
/* pass over k that rotates the exact keys.                                  */
/*                                                                           */
/* RoPE: with rope_len > 0, q and the exact k are rotated at their row index */
/* t with the tables from swa_rope_table (rotate-half pairing (i, i + D/2)):  */
/* q inside the attention kernel, k by a pre-pass into the workspace.         */
/* rope_len must be >= T.  rope_len == 0 means q and k are used as given.     */
/*                                                                           */
/* Rows with no visible key (segment 0 padding) get out = 0 and lse = -inf.  */
/* Accumulation is fp32 for both dtypes; bf16 runs the MFMA kernel, f32 runs */
/* an fp32 vector kernel.                                                    */
/*                                                                           */
/* Workspace (swa_prefill_workspace_size bytes, 256-byte aligned; required */
/* whenever that size is > 0): pre-passes write into it (a) for bf16 plain   */
/* mode, the key metadata: seg_ids and prefix packed to one int32 per key     */
/* (B*T*4 bytes) and summaries of every 32-key sub-tile and 64-key tile       */
/* (B*ceil(T/64)*40 bytes); (b) with RoPE, the rotated keys,                  */
/* B*Hkv*T*D*sizeof(dtype) bytes; (c) in compressed mode, room for pooled     */
/* keys and values, 2*B*Hkv*(T/b)*D*sizeof(dtype) bytes (used when the call   */
/* pools); each part is rounded up to 256 bytes.  Its contents are scratch   */
/* between calls; two calls that overlap in time need two workspaces.        */
/* ------------------------------------------------------------------------ */
typedef struct {
    int B, Hq, Hkv, T, D; /* q, out: [B,Hq,T,D]; k, v: [B,Hkv,T,D]; Hq % Hkv == 0; D in {32, 64} */
    int window;           /* >= 0; 0 = no window                                         */
    int compress_block;   /* 0 = plain; b >= 1 = compressed columns (pooled_k/v [B,Hkv,T/b,D]) */
    int rope_len;         /* rows of rope_cos/rope_sin; 0 = no in-kernel RoPE              */
    float scale;          /* softmax scale; 0 selects 1/sqrt(D)                           */
    int dtype;            /* swa_dtype of q, k, v, pooled_k, pooled_v and out             */
} swa_prefill_params;

/* Bytes of workspace swa_attn_prefill needs for these parameters.          */
size_t swa_prefill_workspace_size(const swa_prefill_params* p);

int swa_attn_prefill(const swa_prefill_params* p,
                     const void* q, const void* k, const void* v,
                     const void* pooled_k, const void* pooled_v, /* compressed mode; both NULL: pooled here */
                     const int32_t* seg_ids,                     /* [B,T] or NULL (all segment 1)  */
                     const uint8_t* prefix,                      /* [B,T] sink flags or NULL       */
                     const float* rope_cos, const float* rope_sin, /* [rope_len, D/2] or NULL      */
                     void* out,                                  /* [B,Hq,T,D], dtype of q         */
                     float* lse,                                 /* [B,Hq,T] natural-log LSE or NULL */
                     void* workspace, size_t workspace_bytes,    /* see swa_prefill_workspace_size */
                     void* stream);

/* Visibility as the prefill kernels apply it (a test hook): for bf16, the   */
/* MFMA kernel itself runs its walk, sub-tile classification and masks and   */
/* writes the pairs it would let through instead of computing attention; for */
/* fp32, a kernel with the fp32 kernel's tile enumeration and predicate does. */
/* mask_out [B,T,Tk] u8 (Tk = T, or T/b + T in compressed mode, pooled        */
/* columns first) may be NULL (then any T is accepted, else T <= 16384);      */
/* count_out [B,T] i32 receives the number of visible columns per row.  bf16  */
/* calls with seg_ids or prefix need the workspace swa_prefill_workspace_size */
/* reports (the key-metadata pre-pass writes into it).                       */
int swa_debug_visibility(const swa_prefill_params* p, const int32_t* seg_ids, const uint8_t* prefix,
                         uint8_t* mask_out, int32_t* count_out, void* workspace, size_t workspace_bytes,
                         void* stream);

/* ------------------------------------------------------------------------ */
/* RoPE tables and block pooling.                                            */
/* ------------------------------------------------------------------------ */
/* [CA §"Pool before rotating, not after"]: RoPE rotates q and the exact keys */
/* at their own position and each pooled key once, at its block midpoint;    */
/* these are the tables every rotation here reads.  Pairing is rotate-half   */
/* over channels (i, i + D/2) with angle = pos * theta^(-2i/D) (the pages    */
/* do not print the pairing; this is the common convention).                 */
/* cos_out/sin_out [rope_len, D/2] fp32, row pos, column i.  D even.          */
/* Device variant: DEVICE pointers, angles in fp64 on the device, each value  */
/* rounded once to fp32, enqueued on `stream`.                                */
int swa_rope_table(double theta, int rope_len, int D, float* cos_out, float* sin_out, void* stream);
/* Host variant: HOST pointers, angles in fp64 on the host, rounded once to   */
/* fp32, computed before the call returns (no device work).  The two agree to */
/* within one fp32 ulp (the two fp64 libraries may round differently).        */
int swa_rope_table_host(double theta, int rope_len, int D, float* cos_out, float* sin_out);

/* [CA §"Pool before rotating, not after"]: pooled_k[j] and pooled_v[j] are   */
/* the means of rows j*b .. j*b+b-1 of k_pre (the key BEFORE RoPE) and v;     */
/* rows past (T/b)*b are dropped.  With rope tables given, pooled_k[j] alone  */
/* is then rotated once at position min(j*b + b/2, rope_len - 1).  Sums are   */
/* fp32; the result is rounded once to dtype.                                */
/*   k_pre, v [B,H,T,D]; pooled_k, pooled_v [B,H,T/block,D]; block >= 1.     */
int kv_pool_compress_rope(int B, int H, int T, int D, int block, int dtype,
                          const void* k_pre, const void* v,
                          const float* rope_cos, const float* rope_sin, int rope_len, /* NULL/0 = no RoPE */
                          void* pooled_k, void* pooled_v, void* stream);

/* ------------------------------------------------------------------------ */
/* Int8 KV cache and decode.                                                 */
/*                                                                           */
/* The cache stores one int8 per K/V element plus one fp32 scale per 32       */
/* channels, the layout the budget formula of [NW §"Effective KV Window:      */
/* Bounding the Cache Size"] prices.  Quantization is symmetric:              */
/* s = max|x| / 127 over the 32-channel group (IEEE fp32 division), code =    */
/* clamp(rint(x / s), -127, 127) with round-half-even; an all-zero group gets */
/* s = 0 and zero codes.  Dequantized value = code * s.                      */
/* ------------------------------------------------------------------------ */
/* x [N,D] bf16 -> xq [N,D] i8, xs [N,D/32] f32.  D % 32 == 0.               */
int swa_kv_quantize(long long N, int D, const void* x_bf16, int8_t* xq, float* xs, void* stream);

typedef struct {
    int B, Hq, Hkv, D; /* D in {32, 64}; Hq % Hkv == 0 (any group size)        */
    int W;             /* ring capacity = window length, >= 1                   */
    int S;             /* sink cache capacity, >= 0                             */
    float scale;       /* 0 selects 1/sqrt(D)                                   */
    int num_splits;    /* split-K parts per (b, kv head) walk, 0..256.  0 lets  */
                       /* the library choose: one part, unless the batch has    */
                       /* fewer than 512 (b, kv head, group of 4 query heads)   */
                       /* units and S + W exceeds 1024 rows; then one part per  */
                       /* 1024 rows, within 1024 workgroups.  Parts are whole   */
                       /* 16-row pieces; extra parts are empty.                 */
} swa_decode_params;

/* Workspace bytes swa_attn_decode needs for these parameters: 0 with one    */
/* split; else one int32 arrival counter per (b, kv head, group of 4 query    */
/* heads), then per split and query head the softmax partial (m, l) and o[D] */
/* as fp32, each part 256-byte aligned.  The workspace must be zero-filled   */
/* before its first use; every completed call leaves the counters zero       */
/* again, so it can be reused by later calls on the same stream.  Two calls  */
/* that overlap in time need two workspaces.                                 */
size_t swa_decode_workspace_size(const swa_decode_params* p);

/* One decode step with the mask of [NS §"256-token 滑动窗口：源码走读"]:     */
/* the new token at position pos[b] sees the sink rows [0, sink_len[b]) and  */
/* the ring positions [max(sink_len[b], pos[b] - W + 1), pos[b]], stored at   */
/* slot position % W.  There is no packing term in decode.  When k_new and   */
/* v_new are given they are first quantized into slot pos[b] % W of the ring. */
/* Preconditions the device cannot check cheaply: sink_len[b] <= pos[b] (else */
/* the ring counts as empty) and sink_len[b] <= S.                           */
/* Numerics: the dot products run on f16 matrix instructions with fp32       */
/* accumulation.  q enters as f16 after an exact power-of-two scaling per    */
/* head (its largest magnitude lands in [2^13, 2^14)), so any finite q is    */
/* taken; components below 2^-27 of the head's largest lose bits.  Each P.V  */
/* weight enters as the f16 number p * s_v / 2^e, with s_v the row's V scale */
/* of a 32-channel group and 2^e a power of two at least as large as every   */
/* V scale of that group seen so far in the walk (p <= 2^8): rows whose      */
/* p * s_v is below 2^(e-14) keep fewer bits, below 2^(e-25) they add 0 --   */
/* a V group whose scale is 2^25 times smaller than the largest one of the   */
/* window is counted as zero.                                                */
int swa_attn_decode(const swa_decode_params* p,
                    const void* q,                        /* [B,Hq,D] bf16, already rotated   */
                    const void* k_new, const void* v_new, /* [B,Hkv,D] bf16, or both NULL      */
                    int8_t* ring_k, int8_t* ring_v,       /* [B,Hkv,W,D]                       */
                    float* ring_ks, float* ring_vs,       /* [B,Hkv,W,D/32]                    */
                    const int8_t* sink_k, const int8_t* sink_v, /* [B,Hkv,S,D] (NULL if S==0)  */
                    const float* sink_ks, const float* sink_vs, /* [B,Hkv,S,D/32]              */
                    const int32_t* pos,                   /* [B]                               */
                    const int32_t* sink_len,              /* [B] or NULL (= S)                 */
                    void* out,                            /* [B,Hq,D] bf16                     */
                    void* workspace, size_t workspace_bytes, void* stream);

/* One decode step of the compressed variant ([CA §"Two kinds of columns,   */
/* pooled blocks and exact recent keys", §"Pool before rotating, not after"]).*/
/* Per (b, kv head) the cache is an exact ring (as in swa_attn_decode), a    */
/* pooled-block cache of capacity P = p->S rows, and the frontier: fp32      */
/* running sums of the pre-RoPE keys and of the values of the block in       */
/* progress (the compressor frontier of [DS §磁盘 KV 缓存]).  The step at     */
/* position pos[b] (steps of one sequence come at consecutive positions):    */
/*  1. quantizes k_new (rotated at pos) and v_new into ring slot pos % W;    */
/*  2. sets the frontier to (k_new_pre, v_new) when pos % block == 0, else   */
/*     adds them;                                                            */
/*  3. when pos % block == block - 1 the block j = pos / block is complete:  */
/*     if j < P, its mean key, rotated at min(j*block + block/2, rope_len-1) */
/*     with the tables of swa_rope_table (no rotation when they are NULL),   */
/*     and its mean value are quantized into pooled row j;                   */
/*  4. the query attends over the pooled rows j < min(P, floor((pos - W + 1) */
/*     / block)) -- the blocks that have cleared the window -- and the ring  */
/*     positions [max(0, pos - W + 1), pos], one softmax.                    */
/* A block completed at pos is first read at pos + W, so no step reads a row */
/* it writes.  pos[b] < 0 appends nothing and gives out = 0.  Blocks with   */
/* j >= P are dropped.  Quantization is that of swa_kv_quantize.  num_splits */
/* and the workspace are those of swa_attn_decode for the same params.       */
int swa_attn_decode_compressed(const swa_decode_params* p,   /* S = P, the pooled capacity     */
                               int block,                    /* b >= 1                          */
                               const float* rope_cos, const float* rope_sin, /* [rope_len,D/2] or NULL */
                               int rope_len,
                               const void* q,                /* [B,Hq,D] bf16, rotated at pos   */
                               const void* k_new,            /* [B,Hkv,D] bf16, rotated at pos  */
                               const void* k_new_pre,        /* [B,Hkv,D] bf16, before rotation */
                               const void* v_new,            /* [B,Hkv,D] bf16                  */
                               int8_t* ring_k, int8_t* ring_v,   /* [B,Hkv,W,D]                 */
                               float* ring_ks, float* ring_vs,   /* [B,Hkv,W,D/32]              */
                               int8_t* pool_k, int8_t* pool_v,   /* [B,Hkv,P,D] (NULL if P==0)  */
                               float* pool_ks, float* pool_vs,   /* [B,Hkv,P,D/32]              */
                               float* front_k, float* front_v,   /* [B,Hkv,D] fp32              */
                               const int32_t* pos,           /* [B]                             */
                               void* out,                    /* [B,Hq,D] bf16                   */
                               void* workspace, size_t workspace_bytes, void* stream);

/* Gradients of swa_attn_prefill in plain mode (compress_block == 0): the    */
/* training-side use of the packing & causal & (recent | sink) mask ([NS]    */
/* "KV sink 如何「钉住」工具"; [NW] "KV Sinks for Tools").  The pages give no  */
/* backward; this is the derivative of the forward: with P = exp(scale q k^T */
/* - lse) over the visible pairs, dP = dO v^T, Delta = rowsum(dO * out),     */
/* dS = P (dP - Delta): dq = scale dS k, dk = scale dS^T q, dv = P^T dO,     */
/* summed over each kv head's query heads.  out and lse are the forward's    */
/* (lse: [B,Hq,T] fp32, natural log).  With rope_len > 0, q and k are the    */
/* unrotated inputs (as for the forward) and so are dq and dk.  All         */
/* arithmetic is fp32; dq/dk/dv are fp32, written (not accumulated into).   */
/* Rows that see nothing (segment 0, lse = -inf) get dq = 0 and give nothing.*/
size_t swa_prefill_backward_workspace_size(const swa_prefill_params* p);
int swa_attn_prefill_backward(const swa_prefill_params* p,
                              const void* q, const void* k, const void* v, /* as for swa_attn_prefill   */
                              const void* out, const float* lse,           /* the forward's out and lse  */
                              const void* dout,                            /* [B,Hq,T,D], p->dtype       */
                              const int32_t* seg_ids, const uint8_t* prefix,
                              const float* rope_cos, const float* rope_sin,
                              float* dq, float* dk, float* dv,             /* [B,Hq|Hkv,T,D] fp32        */
                              void* workspace, size_t workspace_bytes, void* stream);

/* The selection branch of NSA, without its learned gate ([CA] "Two kinds of */
/* columns, pooled blocks and exact recent keys": the top-k blocks by their  */
/* compressed scores; "What we didn't build, and why").  For row t the        */
/* candidates are the pooled blocks that have cleared the window,            */
/* (j + 1) * b <= t - W + 1 with b = p->compress_block and W = p->window;    */
/* block j's score is scale <q_t, pk_j>, pk_j the mean of the block's keys   */
/* before RoPE rotated at min(j b + b/2, rope_len - 1) ([CA] "Pool before    */
/* rotating, not after"); the n_select best blocks (the lower j on ties; all */
/* when fewer) are chosen, and one softmax runs over the exact keys, rotated */
/* at their positions, of all their tokens.  out [B,Hq,T,D] (p->dtype), lse  */
/* [B,Hq,T] fp32 or NULL, sel [B,Hq,T,n_select] int32 (the chosen blocks in  */
/* score order, -1 after the last) or NULL.  A row with no candidate gets    */
/* out = 0, lse = -inf.  Arithmetic is fp32 (with bf16 inputs the rotated   */
/* exact keys are rounded to bf16 once, as in swa_attn_prefill).             */
/* 1 <= n_select <= 32; W >= 1; q, k, v as for swa_attn_prefill (rope_len 0: */
/* no rotation).  Workspace: the rotated exact keys (B*Hkv*T*D elements of   */
/* the dtype, with RoPE only) and the fp32 pooled keys (B*Hkv*(T/b)*D*4      */
/* bytes), each rounded up to 256 bytes.                                     */
size_t swa_nsa_select_workspace_size(const swa_prefill_params* p);
int swa_nsa_select_attn(const swa_prefill_params* p, int n_select,
                        const void* q, const void* k, const void* v, /* [B,Hq|Hkv,T,D], before RoPE */
                        const float* rope_cos, const float* rope_sin,
                        void* out, float* lse, int32_t* sel,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Chunked prefill into existing caches (the long-prompt path of [DS]       */
/* "工作原理与配置方式", which prefills in chunks of 4096 tokens; mask of [NS] */
/* "256-token 滑动窗口：源码走读").  A chunk of Tc tokens at positions         */
/* pos0[b] .. pos0[b] + Tc - 1 attends, for token t, over the sink rows      */
/* [0, sl) with sl = min(sink_len[b], pos0[b], S), the ring positions        */
/* [max(sl, t - W + 1), pos0[b] - 1] as the ring holds them before the call, */
/* and the chunk's own keys [max(pos0[b], t - W + 1), t] (unquantized); one  */
/* softmax.  Then the chunk's last min(W, Tc) tokens are quantized (as by    */
/* swa_kv_quantize) into ring slots position % W.  Precondition: the ring    */
/* holds positions pos0[b] - W .. pos0[b] - 1 (those >= sl), as after a      */
/* decode or a chunk that ended at pos0[b] - 1.  Negative pos0 counts as 0.  */
/* Cached rows are dequantized and rounded to bf16 for the MFMA attention;   */
/* q, k, v are read and out written in place.                              */
typedef struct {
    int B, Hq, Hkv, D; /* D in {32, 64}; Hq % Hkv == 0; B * Hkv <= 65535      */
    int W;             /* ring capacity = window length, >= 1                   */
    int S;             /* sink cache capacity, >= 0                             */
    int Tc;            /* chunk length, >= 0; C + Tc <= 131072 with C =        */
                       /* S + W - 1 rounded up to a multiple of 64             */
    float scale;       /* 0 selects 1/sqrt(D)                                   */
} swa_chunk_params;

/* Bytes of workspace swa_attn_chunk_prefill needs (the C cached rows of   */
/* keys and values per kv head, dequantized to bf16; segment ids and prefix */
/* flags of the C + Tc keys; the prefill workspace of that key sequence).   */
size_t swa_chunk_prefill_workspace_size(const swa_chunk_params* p);

int swa_attn_chunk_prefill(const swa_chunk_params* p,
                           const void* q,                       /* [B,Hq,Tc,D] bf16, rotated     */
                           const void* k, const void* v,        /* [B,Hkv,Tc,D] bf16, k rotated  */
                           int8_t* ring_k, int8_t* ring_v,      /* [B,Hkv,W,D], updated          */
                           float* ring_ks, float* ring_vs,      /* [B,Hkv,W,D/32], updated       */
                           const int8_t* sink_k, const int8_t* sink_v, /* [B,Hkv,S,D] (NULL if S==0) */
                           const float* sink_ks, const float* sink_vs, /* [B,Hkv,S,D/32]         */
                           const int32_t* pos0,                 /* [B] first position of the chunk */
                           const int32_t* sink_len,             /* [B] or NULL (= S)             */
                           void* out,                           /* [B,Hq,Tc,D] bf16              */
                           void* workspace, size_t workspace_bytes, void* stream);

/* swa_attn_decode for callers that cannot allocate memory (code under HIP   */
/* graph capture, tight serving loops, harnesses that forbid allocation):    */
/* the same computation, kernels and results, with the split-K state kept in */
/* a device array inside the library (4 MiB per GPU, held until the process  */
/* ends) instead of a caller workspace.  Calls needing more state than that  */
/* return SWA_ERR_UNSUPPORTED (use fewer splits).  It allocates nothing.  All */
/* calls on one GPU share the array: calls that overlap in time on one GPU   */
/* race.  The device current at the call must be the stream's device.       */
int swa_attn_decode_noalloc(const swa_decode_params* p, const void* q, const void* k_new, const void* v_new,
                            int8_t* ring_k, int8_t* ring_v, float* ring_ks, float* ring_vs, const int8_t* sink_k,
                            const int8_t* sink_v, const float* sink_ks, const float* sink_vs, const int32_t* pos,
                            const int32_t* sink_len, void* out, void* stream);

/* ------------------------------------------------------------------------ */
/* Window sizing (HOST functions, no device work).                           */
/* [NW §"Effective KV Window: Bounding the Cache Size"], [NS §"256 这个窗口宽  */
/* 度从哪来：内存预算计算器"]: per_pos = L*(2*kv + 2*(kv/32)*4)               */
/* + sites*(d_model + 32*4) bytes with kv = num_kv_heads * head_dim and       */
/* head_dim = (attn_dim ? attn_dim : d_model) / num_heads; the budget window  */
/* is (11.5 MiB / per_pos) rounded down to a multiple of 32, clamped to       */
/* [160, max_seq_len] (the lower bound wins).  The effective window is        */
/* min(budget window, kv_window) when kv_window != 0.  Returns -1 on invalid  */
/* arguments (non-positive sizes).                                           */
/* ------------------------------------------------------------------------ */
long long swa_kv_budget_window(long long d_model, long long attn_dim, long long num_heads,
                               long long num_kv_heads, long long num_layers, long long sites,
                               long long max_seq_len);
long long swa_effective_kv_window(long long d_model, long long attn_dim, long long num_heads,
                                  long long num_kv_heads, long long num_layers, long long sites,
                                  long long max_seq_len, long long kv_window);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
