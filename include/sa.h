/*
 * sa.h -- C ABI of the MI355X (gfx950) RoPE-aware sparse-attention library.
 *
 * The method (from the web summaries "Prism: Spectral-Aware Block-Sparse
 * Attention" and "FASA: Frequency-aware Sparse Attention"): a cheap proxy
 * scores key blocks (prefill) or cached tokens (decode), a per-query top-k
 * keeps the best ones, and exact full-dimension softmax attention runs only
 * over the kept keys, at their original positions.
 *
 * Conventions shared by every entry point
 *  - Tensors are device memory owned by the caller, contiguous, layout BHSD
 *    ([batch, head, sequence, head_dim]) unless stated.  The library never
 *    allocates or frees memory; scratch space is passed in as a workspace
 *    whose size comes from sa_workspace_bytes().
 *  - Work is enqueued on `stream` (a hipStream_t, NULL = the null stream);
 *    no call synchronises the host.  Calls that share a workspace must be
 *    ordered on one stream.
 *  - All argument checks run on the host before any launch; a failing check
 *    returns its status and launches nothing.  A launch error returns
 *    SA_ERR_HIP.  Nothing is thrown across the ABI.
 *  - Floating-point tensors are SA_F32 or SA_BF16 (bf16 = upper half of an
 *    IEEE fp32, round-to-nearest-even on every store).  Scores, pooled
 *    vectors and log-sum-exp outputs are always fp32.  Index outputs int32.
 *  - Supported head_dim: 64 or 128.  Rotary pairs are half-split: pair i is
 *    channels (i, i + d/2), rotated by p * theta^(-2i/d) at position p.
 *  - Query head h reads KV head h / (Hq / Hkv) (grouped-query attention).
 *  - The library keeps no mutable global state; distinct streams may call it
 *    concurrently with distinct buffers.
 *  - Host placement (FASA sec. 2.C, the memory-optimised variant FASA-M):
 *    where an entry point says so, a buffer may instead be pinned host memory
 *    allocated with hipHostMalloc (or a framework's pinned allocator built on
 *    it).  The library looks up its device mapping with
 *    hipPointerGetAttributes and the kernels reach it over the host link;
 *    host memory the device cannot reach (pageable) returns SA_ERR_ACCESS.
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_NULL = 1,        /* a required pointer is NULL                         */
  SA_ERR_SHAPE = 2,       /* sizes inconsistent (S % block, Hq % Hkv, ...)      */
  SA_ERR_DTYPE = 3,       /* unknown dtype                                      */
  SA_ERR_RANGE = 4,       /* a parameter outside its documented range           */
  SA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required         */
  SA_ERR_UNSUPPORTED = 6, /* valid request the library does not implement       */
  SA_ERR_HIP = 7,         /* a HIP launch or runtime call failed                */
  SA_ERR_ACCESS = 8       /* a buffer the device cannot read or write (pageable
                             host memory where pinned memory is allowed)        */
} sa_status;

typedef enum { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;

/* operation ids for sa_workspace_bytes */
enum { SA_OP_BLOCK_SCORE = 1, SA_OP_TOPK = 2, SA_OP_DECODE = 3, SA_OP_TOKEN_TOPK = 4 };

/*
 * sa_rope_apply -- rotary position encoding at absolute positions.
 * FASA sec. 2.A (RoPE frequency chunks) and sec. 2.B (attention keeps the
 * tokens' original absolute positions).
 *   x, out : [B, H, S, d] dtype; out may equal x (in place).
 *   pos    : device int32 [B * S] (position of token s of batch b at
 *            pos[b * S + s]), or NULL for position pos0 + s.
 *   theta  : RoPE base (> 1).
 * The angle p * omega_i is formed and reduced modulo 2*pi in fp64, the
 * rotation is applied in fp32, then stored in dtype.
 * Errors: SA_ERR_NULL (x/out), SA_ERR_SHAPE (B, H, S < 1 or d not 64/128),
 *         SA_ERR_RANGE (theta <= 1, pos0 < 0), SA_ERR_DTYPE.
 */
sa_status sa_rope_apply(const void* x, void* out, sa_dtype dtype, int B, int H, int S, int d,
                        const int32_t* pos, int pos0, double theta, void* stream);

/*
 * sa_kv_cache_append -- write S new tokens into a decode KV cache: keys
 * rotated at their absolute positions, values as they are.  FASA sec. 2.B
 * item 2 (attention over the selected tokens keeps their original absolute
 * positions, so the cache holds keys rotated at those positions) and
 * sec. 2.C (the computation-optimised variant scores from the dominant
 * channels, kept together in a slab).  Used to hand a prefilled prompt to
 * decode (S = prompt length, start = 0) and to append each decoded token
 * (S = 1, start = current cache length).
 *   k_new, v_new : [B, Hkv, S, d] dtype, raw (not rotated) keys and values.
 *   start : device int32 [B]: token s of batch b goes to cache row (and
 *           position) start[b] + s; rows outside [0, Lmax) are skipped.
 *   slab == 0: k_cache [B, Hkv, Lmax, d].
 *   slab == 1: k_cache = k_dom [B, Hkv, Lmax, 2*n_dom] and k_rest
 *           [B, Hkv, Lmax, d - 2*n_dom], laid out as in sa_token_score
 *           (dom_pairs [Hkv, n_dom], distinct pairs < d/2).
 *   slab == 2 (slab + full rows): k_cache = k_dom as for slab == 1, and
 *           k_rest = the full rotated rows [B, Hkv, Lmax, d] in the standard
 *           layout.  Scoring reads the slab; the attention gathers whole
 *           rows of k_rest (sa_sparse_attn_decode with slab == 0), each
 *           256-byte row two whole cache lines instead of a 64-byte slab
 *           piece plus a 192-byte rest piece straddling three, for 2*n_dom
 *           channels of extra memory per token.
 *   v_cache [B, Hkv, Lmax, d].  k_rest and v_cache may be pinned host memory
 *           (host placement, FASA-M).
 * The angle p * omega_i is formed and reduced modulo 2*pi in fp64, the
 * rotation is applied in fp32, then stored in dtype (as sa_rope_apply).
 * Only the written rows change.  Entries of start / dom_pairs are not checked
 * on the host; out-of-range values give undefined cache contents, never a
 * write outside the cache.
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE (B, Hkv, S, Lmax < 1 or d not 64/128),
 *         SA_ERR_RANGE (theta <= 1, slab not 0/1/2, n_dom outside [1, d/2]),
 *         SA_ERR_DTYPE, SA_ERR_ACCESS (k_rest or v_cache in pageable host
 *         memory).
 */
sa_status sa_kv_cache_append(const void* k_new, const void* v_new, sa_dtype dtype, int B,
                             int Hkv, int S, int d, int Lmax, const int32_t* start, double theta,
                             int slab, const int32_t* dom_pairs, int n_dom, void* k_cache,
                             void* k_rest, void* v_cache, void* stream);

/*
 * sa_block_score -- Prism block importance estimation for prefill.
 * Prism sec. 1 (block importance from mean-pooled block vectors), sec. 3
 * item 1 (dual-band pooling), sec. 3 item 2 (energy-based temperature
 * calibration), sec. 5 (block-level matrix products only).
 *   q : [B, Hq, S, d], k : [B, Hkv, S, d], raw (not yet rotated), dtype.
 *   Tokens sit at positions 0 .. S-1.  S % block == 0, N = S / block,
 *   block in {16, 32, 64, 128, 256}.
 *   band_split_pair: pairs [0, split) form the high-frequency band, pairs
 *   [split, d/2) the low band; 0 or d/2 gives a single band.
 *   calibrate: 1 -> per (block, band) the mean m is rescaled by
 *   e_tok / e_pool (token RMS energy over pooled RMS energy; 0 if e_pool is
 *   0); 0 -> plain means.
 *   causal: 1 -> scores[.., I, J] = -inf for J > I.
 *   q_rope_out / k_rope_out (nullable): rotated Q / K written in dtype, as
 *   the sparse attention reads them (one pass over Q and K for both).
 *   q_rope_scale: every stored Q element is the fp32 rotated value times
 *   this factor, then rounded to dtype (1 -> plain rotated Q).  Passing
 *   sm_scale * log2(e) here and sm_scale = ln 2 (the float nearest) to
 *   sa_sparse_attn_prefill gives the same attention with the base-2
 *   exponent folded into Q.  The pooled vectors and scores never see it.
 *   pooled_q_out [B, Hq, N, d] / pooled_k_out [B, Hkv, N, d] (nullable):
 *   calibrated pooled vectors, fp32.
 *   scores [B, Hq, N, N] fp32:  sm_scale * <pooled_q(h, I), pooled_k(g(h), J)>.
 *   ws / ws_bytes: workspace for the pooled vectors whose output pointer is
 *   NULL; sa_workspace_bytes(SA_OP_BLOCK_SCORE, B*(Hq+Hkv)*N, d, 0, 0, 0)
 *   bytes always suffice (ws may be NULL when both pooled outputs are given).
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_RANGE (split outside [0, d/2],
 *         theta <= 1, q_rope_scale not finite), SA_ERR_WORKSPACE,
 *         SA_ERR_DTYPE.
 */
sa_status sa_block_score(const void* q, const void* k, sa_dtype dtype, int B, int Hq, int Hkv,
                         int S, int d, double theta, int block, int band_split_pair,
                         int calibrate, float sm_scale, int causal, void* q_rope_out,
                         float q_rope_scale, void* k_rope_out, float* pooled_q_out,
                         float* pooled_k_out, float* scores, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * sa_token_score -- FASA Token Importance Predictor (sec. 2.B item 1): the
 * score of each cached token uses only the dominant frequency chunks.
 *   q_rope : [B, Hq, d] rotated decode queries, dtype.
 *   slab == 0: k = [B, Hkv, Lmax, d] rotated K cache, k_rest ignored.
 *   slab == 1: k = k_dom [B, Hkv, Lmax, 2*n_dom] (channel j < n_dom holds
 *     channel D[j], channel n_dom + j holds D[j] + d/2), k_rest =
 *     [B, Hkv, Lmax, d - 2*n_dom] (all other channels ascending).  Only
 *     k_dom is read here (FASA sec. 2.C, computation-optimised variant).
 *   cache_len : device int32 [B], 1 <= cache_len[b] <= Lmax.
 *   dom_pairs : device int32 [Hkv, n_dom], ascending distinct pairs < d/2.
 *   Hq / Hkv must be 1, 2, 4 or 8; with slab == 1, 2*n_dom must be 8, 16,
 *   32, 64 or 128 (else SA_ERR_UNSUPPORTED).
 *   scores [B, Hq, Lmax] fp32: sm_scale * sum over i in D of
 *     (q_i k_i + q_{i+d/2} k_{i+d/2}) for t < cache_len[b]; -inf beyond.
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_RANGE (n_dom outside [1, d/2]),
 *         SA_ERR_DTYPE.  Entries of cache_len / dom_pairs are not checked on
 *         the host (device data); out-of-range values give undefined output.
 */
sa_status sa_token_score(const void* q_rope, const void* k, const void* k_rest, sa_dtype dtype,
                         int B, int Hq, int Hkv, int Lmax, int d, const int32_t* cache_len,
                         const int32_t* dom_pairs, int n_dom, int slab, float sm_scale,
                         float* scores, void* stream);

/*
 * sa_token_topk -- FASA Token Importance Predictor and the critical token
 * subset in one call (sec. 2.B items 1 and 2), without writing the score
 * array; standard or dominant-slab cache layout (sec. 2.C).
 *   The result equals, bit for bit, sa_token_score(q_rope, k, NULL, dtype,
 *   B, Hq, Hkv, Lmax, d, cache_len, dom_pairs, n_dom, slab, sm_scale,
 *   scores) followed by sa_topk_select(scores, B*Hq, Lmax, valid_len = row
 *   b*Hq + h -> cache_len[b], k_per_row = NULL, k_const = k_top, n_sink = 0,
 *   n_local = 0, idx_out, max_out, count_out).
 *   q_rope [B, Hq, d]; k: the standard cache [B, Hkv, Lmax, d] (slab = 0) or
 *   the slab [B, Hkv, Lmax, 2*n_dom] (slab = 1); cache_len, dom_pairs as in
 *   sa_token_score.  With the slab, 2*n_dom must be 8, 16, 32 or 64 channels
 *   and a slab row at most 128 bytes (bf16: n_dom 4-32; fp32: n_dom 4-16);
 *   SA_ERR_UNSUPPORTED otherwise.
 *   idx_out [B*Hq, max_out] int32 (max_out >= k_top), count_out [B*Hq].
 *   ws: sa_workspace_bytes(SA_OP_TOKEN_TOPK, B*Hq, Lmax, 0, 0, 0) bytes: per
 *   row a sampled threshold and the keys of its (up to 4096) samples
 *   (16 KiB), and per row, tile of 4096 tokens and scoring wave (4 a tile) a
 *   candidate count and up to 256 candidates of 8 bytes (about 8 KiB per row
 *   and 4096 tokens).
 *   A row's candidates are the tokens whose scores reach its sampled
 *   threshold; when their number falls outside [k_top, 2*k_top + 1024] (at
 *   most 8192) or a list overflows, the row's selection reads all its tokens
 *   again, with their scores recomputed by the same arithmetic, so the
 *   result never depends on the sample.
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE (Lmax outside [1, 262144], d, Hq % Hkv),
 *         SA_ERR_RANGE (n_dom, k_top < 0, max_out < k_top), SA_ERR_WORKSPACE,
 *         SA_ERR_UNSUPPORTED (Hq / Hkv not 1, 2, 4, 8; slab width), SA_ERR_DTYPE.
 */
sa_status sa_token_topk(const void* q_rope, const void* k, sa_dtype dtype, int B, int Hq, int Hkv,
                        int Lmax, int d, const int32_t* cache_len, const int32_t* dom_pairs,
                        int n_dom, int slab, float sm_scale, int k_top, int32_t* idx_out,
                        int max_out, int32_t* count_out, void* ws, size_t ws_bytes, void* stream);

/*
 * sa_topk_select -- per-row selection (Prism sec. 1: keep a subset of
 * relevant blocks; FASA sec. 2.B: the critical token subset T_t).
 *   scores : [rows, cols] fp32.
 *   valid_len : device int32 [rows] (0 <= valid_len <= cols), or NULL = cols.
 *   k_per_row : device int32 [rows], or NULL = k_const for every row.  When
 *     given, entries are clamped to [0, k_const]; k_const bounds them.
 *   Per row with n = valid_len: forced = columns [0, n_sink) and the last
 *   n_local valid columns; from the other valid columns the min(k, count)
 *   best by (score descending, column ascending) are kept.  NaN ranks as
 *   -inf, -0 equals +0.  idx_out [rows, max_out] receives forced + kept,
 *   ascending, padded with -1; count_out [rows] their number.
 *   max_out >= n_sink + n_local + k_const.
 *   ws : workspace of sa_workspace_bytes(SA_OP_TOPK, rows, cols, ...) bytes
 *   (0 today; reserved).
 * Results are bit-exact and deterministic.
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE (rows < 0, cols < 1, cols > 262144),
 *         SA_ERR_RANGE (k_const, n_sink, n_local < 0; max_out too small).
 */
sa_status sa_topk_select(const float* scores, int64_t rows, int cols, const int32_t* valid_len,
                         const int32_t* k_per_row, int k_const, int n_sink, int n_local,
                         int32_t* idx_out, int max_out, int32_t* count_out, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * sa_prefill_row_params -- per-row arguments of sa_topk_select for the
 * B*Hq*N block rows of a prefill layer (host helper: integer arithmetic on
 * host memory, no device work, no stream).  Prism sec. 1 keeps a subset of
 * the key blocks of each query block; the budget reading: query block I sees
 * I + 1 blocks when causal (all N otherwise) and keeps keep_const blocks if
 * keep_const > 0, else ceil(keep_percent * visible / 100) in exact integer
 * arithmetic; forced sink and local blocks come on top of it.
 *   N: query blocks per head (S / block); heads: B * Hq; row r = head * N + I.
 *   valid_len_out, k_per_row_out: caller-owned host int32 arrays of heads*N
 *   entries, each nullable (then not written).
 * Returns the largest per-row budget (>= 0), or -SA_ERR_SHAPE (N < 1, heads
 * < 1, heads * N above 2^31 - 1) / -SA_ERR_RANGE (keep_const < 0,
 * keep_percent outside [0, 100], both zero).
 */
int sa_prefill_row_params(int N, int64_t heads, int causal, int keep_const, int keep_percent,
                          int32_t* valid_len_out, int32_t* k_per_row_out);

/*
 * sa_sparse_attn_prefill -- block-sparse softmax attention (Prism sec. 1).
 *   q_rope [B, Hq, S, d], k_rope [B, Hkv, S, d], v [B, Hkv, S, d], dtype.
 *   blk_idx [B, Hq, N, max_sel] int32: the key blocks each query block
 *   attends to (ascending, distinct, < N; entries past blk_cnt ignored;
 *   an entry outside [0, N), or with causal above the diagonal, is skipped
 *   wherever it sits in the list);
 *   blk_cnt [B, Hq, N] int32 in [0, max_sel] (a count outside that range
 *   is clamped to it on the device, so no read leaves the row).
 *   causal: 1 -> a query at position t sees keys s <= t only (a token mask
 *   inside the diagonal block; blocks J > I contribute nothing).
 *   out [B, Hq, S, d] dtype = softmax(sm_scale q k^T) v over the selected
 *   keys; lse [B, Hq, S] fp32 (nullable) = natural log-sum-exp of the
 *   scaled logits.  A query with no visible key gets out = 0, lse = -inf.
 *   bf16 uses bf16 matrix cores with fp32 accumulation and fp32 softmax;
 *   fp32 computes in fp32 throughout.  With bf16 and sm_scale equal to the
 *   float nearest ln 2, the logits are taken as base-2 exponents directly
 *   (softmax(ln 2 x) = 2^x / sum 2^x), which saves one multiply-add per
 *   score: Q pre-multiplied by sm_scale * log2(e) (sa_block_score's
 *   q_rope_scale) then attends exactly as Q with sm_scale would.
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE (S % block, block not 64/128 for bf16 or
 *         not in {16..256}, d), SA_ERR_RANGE (max_sel < 1), SA_ERR_DTYPE.
 */
sa_status sa_sparse_attn_prefill(const void* q_rope, const void* k_rope, const void* v,
                                 sa_dtype dtype, int B, int Hq, int Hkv, int S, int d, int block,
                                 const int32_t* blk_idx, const int32_t* blk_cnt, int max_sel,
                                 int causal, float sm_scale, void* out, float* lse, void* stream);

/*
 * sa_sparse_attn_decode -- FASA Focused Attention Computation (sec. 2.B
 * item 2): full-dimension attention of one decode query per (b, h) over its
 * selected tokens, at their original positions (the cache holds rotated keys).
 *   q_rope [B, Hq, d]; slab == 0: k [B, Hkv, Lmax, d]; slab == 1: k = k_dom
 *   and k_rest as in sa_token_score (both read; the full key is their
 *   channel union).  v [B, Hkv, Lmax, d].  k_rest and v may be pinned host
 *   memory (host placement, FASA-M: only the dominant slab stays in device
 *   memory and the selected rows of the rest are read over the host link
 *   when they are needed).
 *   tok_idx [B, Hq, max_k] int32 token positions (< cache_len[b]), tok_cnt
 *   [B, Hq] in [0, max_k] (clamped to that range on the device).
 *   cache_len is accepted for symmetry with sa_token_score and may be NULL:
 *   the selection already lies inside each cache.  Entries of tok_idx
 *   outside [0, Lmax) are skipped.  With slab == 1, n_dom must be a
 *   multiple of 4 (SA_ERR_UNSUPPORTED) and dom_pairs is required.
 *   out [B, Hq, d] dtype; lse [B, Hq] fp32 (nullable).  Zero tokens ->
 *   out = 0, lse = -inf.  Split-K partial results (running max, sum, fp32
 *   accumulators) live in ws and are merged by the log-sum-exp rule.
 *   ws_bytes >= sa_workspace_bytes(SA_OP_DECODE, 0, 0, B, Hq, max_k).
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_RANGE, SA_ERR_WORKSPACE,
 *         SA_ERR_DTYPE, SA_ERR_ACCESS (k_rest or v in pageable host memory).
 */
sa_status sa_sparse_attn_decode(const void* q_rope, const void* k, const void* k_rest,
                                const void* v, sa_dtype dtype, int B, int Hq, int Hkv, int Lmax,
                                int d, const int32_t* cache_len, const int32_t* dom_pairs,
                                int n_dom, int slab, const int32_t* tok_idx,
                                const int32_t* tok_cnt, int max_k, float sm_scale, void* out,
                                float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * sa_sparse_attn_decode_static -- sa_sparse_attn_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same kernels and results,
 * with the split-K partials kept in a fixed array of 16 MiB per GPU inside
 * the library (held until the process ends) instead of a workspace argument.
 * Makes no hipMalloc / hipFree or other allocating call.
 *   Arguments as in sa_sparse_attn_decode without ws / ws_bytes.
 *   The partials needed (0 when B * Hq >= 512, the one-pass form; else
 *   B * Hq * ceil(max_k / 256) * 520 bytes) must fit the array:
 *   SA_ERR_WORKSPACE otherwise.  Every call on a GPU shares that GPU's
 *   array, so calls that overlap on one GPU (several streams or threads)
 *   race; serialise them.
 * Errors: as sa_sparse_attn_decode; SA_ERR_HIP if the array's device address
 *         cannot be obtained.
 */
sa_status sa_sparse_attn_decode_static(const void* q_rope, const void* k, const void* k_rest,
                                       const void* v, sa_dtype dtype, int B, int Hq, int Hkv,
                                       int Lmax, int d, const int32_t* cache_len,
                                       const int32_t* dom_pairs, int n_dom, int slab,
                                       const int32_t* tok_idx, const int32_t* tok_cnt, int max_k,
                                       float sm_scale, void* out, float* lse, void* stream);

/*
 * sa_calibrate_dominant -- one-time offline calibration of the dominant
 * rotary pairs of every KV head.  FASA sec. 2.A (a small fixed set of
 * dominant frequency chunks reproduces a head's context selection) and sec.
 * 2.B item 1 (the set comes from a one-time offline calibration).  The pages
 * give no criterion; the one computed here:
 *   for each query head h and calibration query m, the full score of key t
 *   is sum_c q_c k_{t,c} and pair i's partial score is
 *   q_i k_{t,i} + q_{i+P} k_{t,i+P} (P = d/2); pair i's overlap is the number
 *   of keys its partial-score top-k_cal shares with the full-score
 *   top-k_cal (top-k by score descending, then key ascending);
 *   counts_out[g][i] = sum of the overlaps of pair i over the query heads of
 *   KV head g and all calibration queries;
 *   dom_out[g] = the n_dom pairs with the largest counts (ties to the lower
 *   pair), ascending -- the dom_pairs argument of sa_token_score.
 * Scores are decided in fp32: the full score adds the channel products in
 * ascending channel order, a pair score is one rounding of its two products
 * (with bf16 inputs every product is exact, so the result does not depend
 * on the launch).
 *   q_rope : [Hq, M, d] bf16, M rotated calibration queries per query head.
 *   k_rope : [Hkv, L, d] bf16, the rotated keys of the calibration window
 *            (every key is visible to every calibration query).
 *   dom_out [Hkv, n_dom] int32, counts_out [Hkv, d/2] int32 (device).
 *   ws_bytes >= sa_calibrate_workspace_bytes(Hq, Hkv, M, L, d, k_cal): the
 *   full and pair scores, their selections and the counts.
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE (sizes < 1, Hq % Hkv, d not 64/128,
 *         L > 262144), SA_ERR_RANGE (k_cal outside [1, L], n_dom outside
 *         [1, d/2]), SA_ERR_UNSUPPORTED (dtype other than SA_BF16),
 *         SA_ERR_WORKSPACE, SA_ERR_DTYPE.
 */
sa_status sa_calibrate_dominant(const void* q_rope, const void* k_rope, sa_dtype dtype, int Hq,
                                int Hkv, int M, int L, int d, int k_cal, int n_dom,
                                int32_t* dom_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * sa_sfa_sparsify -- k-sparse feature codes for Sparse Feature Attention
 * ("Scaling Attention via Feature Sparsity", sec. 2): every row of x keeps
 * its k_feat channels of largest magnitude (ties to the lower channel, NaN
 * below every number) and zeroes the others.  Attention over the codes is
 * sa_sparse_attn_prefill with every causal block listed: the dot product of
 * two zero-filled codes is the sum over the channels active in both.
 *   x, out : [rows, d] dtype (out may equal x); values are copied bit for bit.
 *   k_feat >= d keeps every channel; k_feat == 0 zeroes the row.
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE (rows < 0, d not 64/128),
 *         SA_ERR_RANGE (k_feat < 0), SA_ERR_DTYPE.
 */
sa_status sa_sfa_sparsify(const void* x, void* out, sa_dtype dtype, int64_t rows, int d,
                          int k_feat, void* stream);

/* Workspace bytes of sa_calibrate_dominant (0 for sizes it rejects). */
size_t sa_calibrate_workspace_bytes(int Hq, int Hkv, int M, int L, int d, int k_cal);

/*
 * sa_workspace_bytes -- bytes of workspace an operation needs.
 *   SA_OP_BLOCK_SCORE: rows = number of pooled vectors B*(Hq+Hkv)*N,
 *       cols = d -> scratch for the pooled Q and K vectors.
 *   SA_OP_TOPK: rows, cols -> 0 (reserved).
 *   SA_OP_DECODE: B, Hq, max_k -> split-K partials (sized for d <= 128).
 *   SA_OP_TOKEN_TOPK: rows = B*Hq, cols = Lmax -> thresholds, counts and
 *   candidate lists of sa_token_topk.
 * Returns 0 for an unknown op.
 */
size_t sa_workspace_bytes(int op, int64_t rows, int cols, int B, int Hq, int max_k);

/* Human-readable name of a status code (static storage). */
const char* sa_status_string(sa_status s);

/* Library version: major * 10000 + minor * 100 + patch. */
int sa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
