/*
 * qknorm_rope_attn -- QK-RMSNorm + RoPE + causal grouped-query attention for
 * one decoder layer, prefill and decode, on AMD Instinct MI355X (gfx950).
 *
 * What the calls compute (zero-to-sglang, "Chapter 3 Forward Pass and
 * Generation (Code Walkthrough)", section 3.3 "QKV, RoPE, and causal
 * attention"; jq-wei, "transformer basics", "Attention calculation: part 1"):
 *
 *   for every token row n of the packed projection qkv[N, (Hq + 2*Hkv) * D]
 *     q_h  = columns [h*D, (h+1)*D)                     (h < Hq)
 *     k_g  = columns [(Hq+g)*D, (Hq+g+1)*D)             (g < Hkv)
 *     v_g  = columns [(Hq+Hkv+g)*D, (Hq+Hkv+g+1)*D)
 *     q~_h = RoPE(RMSNorm(q_h) * w_q, pos[n]);  k~_g = RoPE(RMSNorm(k_g) * w_k, pos[n])
 *       RMSNorm(x) = x / sqrt(mean(x^2) + eps)
 *       RoPE pairs element i with i + D/2 and turns it by pos * base^(-2i/D)
 *     out[n, h*D:(h+1)*D] = sum_t softmax_t(q~_h . k~_{h/G}(t) / sqrt(D)) v_{h/G}(t)
 *       over the request's keys t = 0..i (i = the token's index in its request),
 *       G = Hq / Hkv (query head h reads KV head floor(h / G)).
 *
 * Prefill processes whole requests packed back to back and writes every
 * token's K~ and V to the request's cache (concept chapter "Chapter 3 Forward
 * Pass and Generation", section 4.1).  Decode takes one new token per request,
 * appends its K~ and V at slot L_b, then attends over slots 0..L_b (section 4.2;
 * "transformer basics", "Prefill vs Decode": the cache grows from 12 to 13
 * entries before attention runs).
 *
 * Conventions for every call
 *   - Every pointer argument except `cfg` and `workspace_bytes`-style scalars is
 *     a DEVICE pointer; all device buffers are owned by the caller, must stay
 *     alive until the enqueued work completes, and are never freed or kept by
 *     the library.
 *   - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the default
 *     stream).  Calls return without synchronising.  They allocate no device
 *     memory and are reentrant.
 *   - Element type of qkv, both norm weights, both caches, out and the Q~ part
 *     of the workspace is `cfg->dtype` (bf16 or fp32).  Accumulation is fp32.
 *   - Cache layout (exact): element (b, g, s, d) of a cache lives at
 *       ((b * Hkv + g) * cache_capacity + s) * D + d
 *     K holds post-norm post-RoPE values rounded to the dtype, V holds the
 *     input bits unchanged.  Slots a call does not write keep their contents.
 *   - Errors: the return value is QKRA_OK or one of the QKRA_ERR_* codes below;
 *     argument checks happen on the host before anything is enqueued, so an
 *     error return means nothing was launched (except QKRA_ERR_HIP, where a
 *     launch failed; qknorm_rope_attn_last_hip_error() then gives the hipError_t).
 *     No C++ exception crosses this interface.
 *   - Contents of device arrays (monotone cu_seqlens, positions >= 0,
 *     cache_lens[b] + 1 <= cache_capacity) are the caller's contract; they are
 *     not checked, and violating them is undefined behaviour.
 */
#ifndef QKNORM_ROPE_ATTN_H
#define QKNORM_ROPE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKRA_API __attribute__((visibility("default")))

/* Element types. */
#define QKRA_BF16 0
#define QKRA_FP32 1

/* Status codes. */
#define QKRA_OK 0
#define QKRA_ERR_INVALID_ARGUMENT 1   /* Hq % Hkv != 0, negative size, null pointer with work to do, bad eps/base */
#define QKRA_ERR_UNSUPPORTED 2        /* head_dim not 64 or 128, unknown dtype */
#define QKRA_ERR_CAPACITY 3           /* cache_capacity too small for the longest request / new token */
#define QKRA_ERR_WORKSPACE_TOO_SMALL 4
#define QKRA_ERR_ALIASING 5           /* out overlaps an input, a cache or the workspace, or buffers overlap each other */
#define QKRA_ERR_HIP 6                /* a HIP launch or runtime call failed */
#define QKRA_ERR_SCRATCH_LIMIT 7      /* qknorm_rope_attn_decode_noalloc: the call needs more than its fixed scratch */

/* Workspace query modes. */
#define QKRA_MODE_PREFILL 0
#define QKRA_MODE_DECODE 1

/* Layer configuration, passed by pointer (host memory) to every call. */
typedef struct qkra_config {
  int32_t num_q_heads;   /* Hq > 0 */
  int32_t num_kv_heads;  /* Hkv > 0, Hq % Hkv == 0 (whole groups of query heads share a KV head) */
  int32_t head_dim;      /* D: 64 or 128; independent of the hidden size */
  int32_t dtype;         /* QKRA_BF16 or QKRA_FP32 */
  float rms_eps;         /* >= 0, added to mean(x^2) inside the square root */
  /* 0, or the caller's upper bound on max|q_norm_weight| * max|k_norm_weight|
   * (static for a layer).  A bf16 prefill bounds every score by this product
   * (times sqrt(D) log2(e)) and then takes the softmax with no shift when it is
   * small enough (qknorm_rope_attn_unshifted_weight_limit(D)); the choice is
   * made on the device from the weights, so by default both softmax kernels
   * are launched and one of them returns at once.  With a bound here the host
   * launches only the one it selects.  The device check stays: if the weights
   * break a bound that selected the unshifted softmax, the rows it cannot
   * compute are written as NaN, never as wrong numbers.  Must be finite and
   * >= 0.  Appends (calls with cache_lens) and fp32 ignore it. */
  float qk_weight_bound;
  double rope_base;      /* > 0, e.g. 1e4 or 1e6 */
} qkra_config;

/*
 * Finite-input ranges.  With finite inputs every call returns finite results
 * (each within the stated tolerance of the exact layer) when, additionally:
 *  - every qkv element of a Q or K head has |x| < 2^60, so that the fp32 sum of
 *    squares over a head row stays finite;
 *  - with the running-max softmax (decode, appends, fp32 mode, and a bf16
 *    prefill whose weights exceed qknorm_rope_attn_unshifted_weight_limit(D)),
 *    (keys a row attends to) * max|v| < 2^119: the max is raised lazily, only
 *    when a score passes it by more than 8 in log2 units, so a probability
 *    stays at most 2^8 inside the fp32 accumulators' 2^128; and
 *    max|q_norm_weight| * max|k_norm_weight| * D < 2^120, so that a score is
 *    finite;
 *  - with the softmax without a shift (a bf16 prefill with no history and
 *    weights within that limit), every probability is at most 2^48, so
 *    (keys a row attends to) * max|v| < 2^79 (for example |v| < 2^64 for rows of
 *    up to 32768 keys).
 * V enters only the products with the probabilities, so outputs are linear in
 * V: inside these ranges a power-of-two scale of V scales every output by
 * exactly that power.
 */

/* Largest max|q_norm_weight| * max|k_norm_weight| for which a bf16 prefill of
 * head dimension D takes the softmax without a shift (0 for an unsupported D).
 * Pure host computation. */
QKRA_API float qknorm_rope_attn_unshifted_weight_limit(int32_t head_dim);

/*
 * Prefill of `num_seqs` requests packed into `num_tokens` rows.
 *
 *   qkv            [num_tokens, (Hq+2Hkv)*D], row-major, read-only.
 *   q_norm_weight  [D], k_norm_weight [D], read-only.
 *   positions      int32 [num_tokens]: RoPE position of each row (only the angle
 *                  depends on it; the cache slot is the in-request index).
 *   cu_seqlens     int32 [num_seqs+1]: cu[0] = 0, non-decreasing, cu[num_seqs] =
 *                  num_tokens; request r owns rows cu[r] .. cu[r+1]-1.  Zero-length
 *                  requests are allowed and produce nothing.
 *   max_seqlen     host copy of max_r (cu[r+1]-cu[r]); used to size the launch.
 *   k_cache, v_cache [num_seqs, Hkv, cache_capacity, D]; token j of request r
 *                  is written to slot j; slots >= the request's length are not
 *                  touched.  cache_capacity >= max_seqlen.
 *   out            [num_tokens, Hq*D], write-only; must not overlap any other buffer.
 *   workspace      device scratch of at least
 *                  qknorm_rope_attn_workspace_bytes(cfg, QKRA_MODE_PREFILL,
 *                  num_tokens, max_seqlen) bytes.  On return (after the stream
 *                  work completes) it holds, for fp32, q~ as [num_tokens, Hq,
 *                  D]; for bf16, each token's RoPE pairs as fp32 [num_tokens]
 *                  [D]: cos in the first half, sin in the second, pair i of
 *                  each half at (D/4)*((i/4)%2) + 4*(i/8) + i%4 (the attention
 *                  kernel normalises and rotates Q as it loads it, so q~ is
 *                  never stored).
 * num_tokens == 0 is a no-op returning QKRA_OK.
 */
QKRA_API int32_t qknorm_rope_attn_prefill(const qkra_config* cfg, const void* qkv,
                                          const void* q_norm_weight, const void* k_norm_weight,
                                          const int32_t* positions, const int32_t* cu_seqlens,
                                          int32_t num_tokens, int32_t num_seqs, int32_t max_seqlen,
                                          void* k_cache, void* v_cache, int32_t cache_capacity,
                                          void* out, void* workspace, size_t workspace_bytes,
                                          void* hip_stream);

/*
 * Prefill of a chunk of new tokens per request onto caches that already hold
 * entries (chunked prefill, prompt continuation).  It extends the cached
 * history of each request the way decode extends it by one token (concept
 * chapter, section 4: later tokens attend to the cached history; "Prefill vs
 * Decode": the cache grows before attention runs): request r's new token j is
 * written to slot P_r + j and its query attends over slots 0 .. P_r + j.
 * With every P_r = 0 this is qknorm_rope_attn_prefill; with one token per
 * request it is qknorm_rope_attn_decode.
 *
 *   qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, max_seqlen, out
 *                  as for qknorm_rope_attn_prefill (positions are usually
 *                  P_r + j, but only the RoPE angle depends on them).
 *   cache_lens     int32 [num_seqs]: P_r, the number of valid cache entries
 *                  before this call (slots 0 .. P_r-1 are read, never
 *                  written).  Not updated by the library.
 *   max_cache_len  host copy of max_r P_r; cache_capacity >= max_cache_len +
 *                  max_seqlen.
 *   k_cache, v_cache [num_seqs, Hkv, cache_capacity, D]; slots P_r .. P_r+T_r-1
 *                  are written, all others keep their contents.
 *   workspace      as for qknorm_rope_attn_prefill (same size and contents).
 * num_tokens == 0 is a no-op returning QKRA_OK; otherwise a null cache_lens
 * is QKRA_ERR_INVALID_ARGUMENT.
 */
QKRA_API int32_t qknorm_rope_attn_prefill_append(const qkra_config* cfg, const void* qkv,
                                                 const void* q_norm_weight, const void* k_norm_weight,
                                                 const int32_t* positions, const int32_t* cu_seqlens,
                                                 const int32_t* cache_lens, int32_t num_tokens,
                                                 int32_t num_seqs, int32_t max_seqlen,
                                                 int32_t max_cache_len, void* k_cache, void* v_cache,
                                                 int32_t cache_capacity, void* out, void* workspace,
                                                 size_t workspace_bytes, void* hip_stream);

/*
 * Decode step: one new token per request.
 *
 *   qkv            [num_seqs, (Hq+2Hkv)*D]: the new token's projection row.
 *   positions      int32 [num_seqs]: RoPE position of the new token.
 *   cache_lens     int32 [num_seqs]: L_b, the number of valid cache entries
 *                  before this step.  The new token's k~ and v are written to
 *                  slot L_b, then its query attends over slots 0..L_b.  The
 *                  library does not update cache_lens.
 *   max_cache_len  host copy of max_b L_b; cache_capacity >= max_cache_len + 1.
 *   k_cache, v_cache [num_seqs, Hkv, cache_capacity, D], read and written.
 *   out            [num_seqs, Hq*D], write-only.
 *   workspace      at least qknorm_rope_attn_workspace_bytes(cfg,
 *                  QKRA_MODE_DECODE, num_seqs, max_cache_len) bytes: q~ as
 *                  [num_seqs, Hq, D] in the dtype, then (bf16) an int32 step
 *                  plan and fp32 partial records of an even split of all
 *                  requests' keys over a fixed set of wavefronts, or (fp32)
 *                  fp32 partials per 1024-key split.
 * num_seqs == 0 is a no-op returning QKRA_OK.  bf16 calls whose step count
 * num_seqs * Hkv * (G / GW) * ceil(cache_capacity / 32) reaches 2^31 (GW: the
 * query heads per matrix tile, the largest divisor of G up to 16) return
 * QKRA_ERR_UNSUPPORTED.
 */
QKRA_API int32_t qknorm_rope_attn_decode(const qkra_config* cfg, const void* qkv,
                                         const void* q_norm_weight, const void* k_norm_weight,
                                         const int32_t* positions, const int32_t* cache_lens,
                                         int32_t num_seqs, int32_t max_cache_len,
                                         void* k_cache, void* v_cache, int32_t cache_capacity,
                                         void* out, void* workspace, size_t workspace_bytes,
                                         void* hip_stream);

/*
 * Decode without allocation or workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, checks, layouts and
 * kernels as qknorm_rope_attn_decode, with the workspace in a fixed device
 * array inside the library, QKRA_NOALLOC_SCRATCH_BYTES per GPU, held from the
 * first call on a GPU until the process ends.  It calls no hipMalloc or
 * hipFree and creates no HIP objects; its first call on a device looks up that
 * device's copy of the array (the calling thread's current device, which
 * must be the stream's).
 *
 * Calls whose decode workspace (qknorm_rope_attn_workspace_bytes(cfg,
 * QKRA_MODE_DECODE, num_seqs, max_cache_len)) exceeds the scratch return
 * QKRA_ERR_SCRATCH_LIMIT before anything is enqueued.  With Qwen3 heads (32
 * query, 8 KV, D = 128) in bf16 that is about 1000 requests; fp32 partials
 * grow with max_cache_len.
 *
 * Every call on a GPU shares that GPU's scratch, which keeps the last call's
 * contents (nothing in it needs to start at zero).  Calls that overlap on one
 * GPU, on different streams or from different threads, race on it: the caller
 * must order them (one stream, or events).
 */
#define QKRA_NOALLOC_SCRATCH_BYTES (16u << 20)
QKRA_API int32_t qknorm_rope_attn_decode_noalloc(const qkra_config* cfg, const void* qkv,
                                                 const void* q_norm_weight, const void* k_norm_weight,
                                                 const int32_t* positions, const int32_t* cache_lens,
                                                 int32_t num_seqs, int32_t max_cache_len,
                                                 void* k_cache, void* v_cache, int32_t cache_capacity,
                                                 void* out, void* hip_stream);

/*
 * One serving step with both kinds of request: exactly what
 * qknorm_rope_attn_prefill(prefill arguments) followed by
 * qknorm_rope_attn_decode(decode arguments) on the same stream computes
 * (the pages' prefill and decode stages, "Chapter 3 Forward Pass and
 * Generation", sections 4.1-4.2, run as one packed step), with the same
 * arguments, layouts, checks and status codes.  Both halves share cfg and
 * the norm weights.  In bf16, with D = 64 or 128 and Hq / Hkv in
 * {1, 2, 4, 8, 16}, the prefill attention and the decode split run in one
 * launch: some workgroups stream the decode requests' caches while the rest
 * run the prefill on the matrix cores.  Otherwise the two calls run in turn.
 * Because the halves run at the same time, what one half writes (its out,
 * caches and workspace) must not overlap anything the other half reads or
 * writes: QKRA_ERR_ALIASING otherwise.  All arguments of both halves are
 * checked before anything is enqueued.
 */
QKRA_API int32_t qknorm_rope_attn_mixed_step(
    const qkra_config* cfg, const void* q_norm_weight, const void* k_norm_weight,
    const void* prefill_qkv, const int32_t* prefill_positions, const int32_t* cu_seqlens, int32_t num_tokens,
    int32_t num_prefill_seqs, int32_t max_seqlen, void* prefill_k_cache, void* prefill_v_cache,
    int32_t prefill_cache_capacity, void* prefill_out, void* prefill_workspace, size_t prefill_workspace_bytes,
    const void* decode_qkv, const int32_t* decode_positions, const int32_t* cache_lens, int32_t num_decode_seqs,
    int32_t max_cache_len, void* decode_k_cache, void* decode_v_cache, int32_t decode_cache_capacity,
    void* decode_out, void* decode_workspace, size_t decode_workspace_bytes, void* hip_stream);

/*
 * ---- Paged K/V cache -------------------------------------------------------
 * The pages defer the optimised cache to a chapter they only name (zero-to-
 * sglang, "Chapter 3 Forward Pass and Generation (Code Walkthrough)", opening
 * paragraph and references: "Chapter 4: KV Cache Optimization"; concept
 * chapter, section 4).  The reading here: a paged cache is the same
 * per-request cache with its slots stored in fixed-size pages of a shared
 * pool, found through a block table, so every result equals the contiguous
 * calls' on the logical cache the table describes.
 *
 *   k_pool, v_pool [num_pages, Hkv, page_size, D] in the dtype, 16-byte
 *                  aligned: element (p, g, r, d) at ((p * Hkv + g) * page_size
 *                  + r) * D + d.  A page holds page_size consecutive slots of
 *                  one request for every KV head.
 *   block_table    int32 [num_seqs, pages_per_seq] (device): slot s of
 *                  request b is row s % page_size of page
 *                  block_table[b * pages_per_seq + s / page_size].  Each
 *                  request can hold pages_per_seq * page_size slots (the
 *                  capacity checked as cache_capacity is for the contiguous
 *                  calls).  Entries the call does not reach may hold anything.
 *   page_size      64, 128, 256, 512 or 1024 (QKRA_ERR_UNSUPPORTED otherwise):
 *                  a page then holds whole 64-key prefill tiles and 32-key
 *                  decode steps.
 * Pages a call writes (the slots of its new tokens) must belong to one request
 * each; pages may be shared between requests for reading (a common prefix).
 * Table entries the call reaches must lie in [0, num_pages) (the caller's
 * contract, like cu_seqlens; the kernels clamp them to the pool, so a bad
 * entry gives wrong values, never an access outside the pool).  The pools and
 * the table may not overlap out, the workspace or each other's written
 * ranges (QKRA_ERR_ALIASING).
 */
typedef struct qkra_paged_cache {
  void* k_pool;
  void* v_pool;
  const int32_t* block_table;
  int32_t num_pages;       /* > 0 */
  int32_t page_size;       /* 64, 128, 256, 512 or 1024 */
  int32_t pages_per_seq;   /* > 0: row length of block_table */
  int32_t reserved;        /* must be 0 */
} qkra_paged_cache;

/*
 * qknorm_rope_attn_decode on a paged cache: the new token's k~ and v go to
 * slot L_b of request b through the table, then its query attends over slots
 * 0..L_b.  Requires max_cache_len + 1 <= pages_per_seq * page_size
 * (QKRA_ERR_CAPACITY).  Workspace as for qknorm_rope_attn_decode (the same
 * size query, QKRA_MODE_DECODE).
 */
QKRA_API int32_t qknorm_rope_attn_decode_paged(const qkra_config* cfg, const void* qkv,
                                               const void* q_norm_weight, const void* k_norm_weight,
                                               const int32_t* positions, const int32_t* cache_lens,
                                               int32_t num_seqs, int32_t max_cache_len,
                                               const qkra_paged_cache* cache, void* out, void* workspace,
                                               size_t workspace_bytes, void* hip_stream);

/*
 * qknorm_rope_attn_prefill_append on a paged cache: request r's new token j is
 * written to slot P_r + j through the table and attends over slots
 * 0..P_r + j.  cache_lens may be NULL (with max_cache_len 0): every P_r = 0,
 * a prefill into the paged cache.  Requires max_cache_len + max_seqlen <=
 * pages_per_seq * page_size.  Workspace as for qknorm_rope_attn_prefill
 * (QKRA_MODE_PREFILL).
 */
QKRA_API int32_t qknorm_rope_attn_prefill_append_paged(const qkra_config* cfg, const void* qkv,
                                                       const void* q_norm_weight, const void* k_norm_weight,
                                                       const int32_t* positions, const int32_t* cu_seqlens,
                                                       const int32_t* cache_lens, int32_t num_tokens,
                                                       int32_t num_seqs, int32_t max_seqlen,
                                                       int32_t max_cache_len, const qkra_paged_cache* cache,
                                                       void* out, void* workspace, size_t workspace_bytes,
                                                       void* hip_stream);

/*
 * Workspace size in bytes for a call (0 when the configuration is invalid).
 * mode QKRA_MODE_PREFILL: n = num_tokens, max_len = max_seqlen.
 * mode QKRA_MODE_DECODE:  n = num_seqs,   max_len = max_cache_len.
 * Pure host computation; needs no GPU.
 */
QKRA_API size_t qknorm_rope_attn_workspace_bytes(const qkra_config* cfg, int32_t mode, int32_t n,
                                                 int32_t max_len);

/* Static string naming a status code (never NULL). */
QKRA_API const char* qknorm_rope_attn_status_string(int32_t status);

/* hipError_t of the most recent QKRA_ERR_HIP on the calling thread (0 if none). */
QKRA_API int32_t qknorm_rope_attn_last_hip_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
QKRA_API int32_t qknorm_rope_attn_version(void);

/*
 * ---- Steps next to the attention layer -------------------------------------
 * The three calls below share the conventions above (device pointers, the
 * caller's stream, host-side checks, QKRA_* status) but take no qkra_config:
 * they work on hidden-size rows, not on heads.
 */

/*
 * Fused residual add + RMSNorm, the step before every attention and MLP
 * sublayer (zero-to-sglang, "Chapter 3 Forward Pass and Generation (Code
 * Walkthrough)", section 3.2 "Computation inside a decoder layer"): the first
 * call of a forward pass keeps x as the residual stream; every later call adds
 * the sublayer output to it.  Row by row, over the hidden_size entries:
 *
 *   has_residual == 0:  residual := x;             out := RMSNorm(x) * weight
 *   has_residual != 0:  residual := x + residual;  out := RMSNorm(x + residual) * weight
 *   RMSNorm(r) = r / sqrt(mean(r^2) + rms_eps)
 *
 *   dtype          QKRA_BF16 or QKRA_FP32: element type of x, residual, weight, out.
 *   x              [num_tokens, hidden_size].
 *   residual       [num_tokens, hidden_size], read (has_residual) and written.
 *                  With has_residual == 0 it may be x itself, and then nothing
 *                  is copied; otherwise it must not overlap x.
 *   weight         [hidden_size].
 *   out            [num_tokens, hidden_size]; may be exactly x (in place);
 *                  must not overlap residual or weight.
 *   hidden_size    a multiple of 8, at most 32768 (QKRA_ERR_UNSUPPORTED above).
 * The sum is formed in fp32; residual keeps it rounded to the dtype and out
 * normalises the fp32 sum.  All pointers 16-byte aligned.  num_tokens == 0 is a
 * no-op returning QKRA_OK.
 */
QKRA_API int32_t qknorm_rope_attn_fused_add_rmsnorm(int32_t dtype, float rms_eps, const void* x, void* residual,
                                                    int32_t has_residual, const void* weight, void* out,
                                                    int32_t num_tokens, int32_t hidden_size, void* hip_stream);

/*
 * Each request's last row of the packed hidden states, the only row the LM
 * head reads (same page, section 4.1 "Keep the last position of each
 * request": the logits at a request's last position predict its next token).
 *
 *   hidden         [num_tokens, hidden_size] in the dtype.
 *   cu_seqlens     int32 [num_seqs+1] (device), as for the prefill calls.
 *   out            [num_seqs, hidden_size]: row r := hidden[cu[r+1]-1] for every
 *                  request with tokens; rows of requests without tokens are
 *                  not written.  Must not overlap hidden or cu_seqlens.
 *   hidden_size    hidden_size * element size a multiple of 16 bytes.
 * hidden and out 16-byte aligned.  num_seqs == 0 is a no-op.
 */
QKRA_API int32_t qknorm_rope_attn_gather_last(int32_t dtype, const void* hidden, const int32_t* cu_seqlens,
                                              int32_t num_tokens, int32_t num_seqs, int32_t hidden_size, void* out,
                                              void* hip_stream);

/*
 * Greedy choice of the next token: per logits row, the index of the largest
 * value (same page, section 4.3 "Find sampling in the engine": a fully greedy
 * batch takes the argmax of each row).  Ties go to the lowest index; a NaN
 * counts as larger than every number, so the first NaN of a row wins.
 *
 *   logits         row b at logits + b * row_stride elements, vocab entries,
 *                  in the dtype; row_stride >= vocab and a multiple of 8;
 *                  16-byte aligned.
 *   out_index      int32 [num_rows].
 *   workspace      at least qknorm_rope_attn_argmax_workspace_bytes(num_rows,
 *                  vocab) bytes, 16-byte aligned: per-segment (value, index)
 *                  records.
 * num_rows == 0 is a no-op.
 */
QKRA_API size_t qknorm_rope_attn_argmax_workspace_bytes(int32_t num_rows, int32_t vocab);
QKRA_API int32_t qknorm_rope_attn_argmax(int32_t dtype, const void* logits, int32_t num_rows, int32_t vocab,
                                         int64_t row_stride, int32_t* out_index, void* workspace,
                                         size_t workspace_bytes, void* hip_stream);

/*
 * Per-kernel timing, for benchmarks.  `enable` is a mask over kernel ids (bit k
 * times kernel id k; -1 times every kernel, 0 switches timing off).  A timed
 * launch records two hipEvents on its own dispatch, at the start and the end
 * of the kernel's execution.  The events come from a pool created by the first
 * call that enables timing (QKRA_ERR_HIP if that fails), never by the
 * attention calls; a launch that finds the pool empty runs untimed.  This is
 * process-wide benchmark instrumentation.
 * qknorm_rope_attn_read_kernel_timing() waits for those events, writes for each
 * kernel id k < max_kernels the summed duration in milliseconds (ms_total[k])
 * and the number of launches (launches[k]), clears the record and returns the
 * number of kernel ids (or a negative QKRA_ERR_* on failure).  Kernel ids are
 * named by qknorm_rope_attn_kernel_name().  Enabling/disabling is process-wide.
 */
QKRA_API int32_t qknorm_rope_attn_set_kernel_timing(int32_t enable);
QKRA_API int32_t qknorm_rope_attn_read_kernel_timing(double* ms_total, int64_t* launches,
                                                     int32_t max_kernels);
QKRA_API const char* qknorm_rope_attn_kernel_name(int32_t kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* QKNORM_ROPE_ATTN_H */
