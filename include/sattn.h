/*
 * sattn.h -- exact streaming (tiled) attention forward for AMD gfx950.
 *
 * C ABI of libsattn.so. Every entry point takes plain device pointers and
 * sizes; no framework types cross this boundary.
 *
 * What is computed (one query row i, eligible keys j):
 *   S_ij = scale * <q_i, k_j>,  m_i = max_j S_ij,  l_i = sum_j exp(S_ij - m_i)
 *   O_i  = sum_j exp(S_ij - m_i) v_j / l_i,        lse_i = m_i + ln(l_i)
 * computed tile by tile over K/V with a mergeable (running max, rescaled
 * exp-sum, rescaled numerator) state, never forming the full score matrix.
 * Sources: "Intermediate and advanced extension" (workshop table, streaming
 * attention and split softmax rows; "Logic review before implementation":
 * the output sum is rescaled with the exponential sum, a causal row sees the
 * key at its own position, dependent launches are ordered by the stream);
 * "Attention algorithms and data movement", lessons 01 (merge partial states
 * by rescaled denominators, a stated result for a row with no key), 03 (saved per-row
 * normalization state = lse), 04 (packed causal eligibility by logical
 * position), 05 (GQA query-head to KV-head mapping).
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * - dtype: SATTN_F16 (IEEE binary16) or SATTN_BF16 (bfloat16) for q, k, v, o.
 *   Products use fp16/bf16 inputs with fp32 accumulation; the softmax state
 *   is fp32; P is rounded to the input dtype for the P*V product while the
 *   exp-sum l accumulates the fp32 values; O is rounded once (nearest-even).
 * - lse is float32, natural log, of the scaled scores.
 * - Head dimension D must be 32, 64 or 128.
 * - scale must be finite and > 0 (the caller passes e.g. 1/sqrt(D)).
 * - Pointers are device pointers on the current HIP device. q, k, v, o must
 *   be 16-byte aligned, float buffers 4-byte aligned. Inputs are read-only;
 *   outputs must not overlap any input or each other (byte ranges).
 * - stream: a hipStream_t (NULL = the default stream). All work is enqueued
 *   on it asynchronously; nothing synchronizes the host.
 * - Ownership: the caller allocates and owns every buffer, including the
 *   split-KV partial buffers. The library allocates no device memory and
 *   keeps no mutable global state; calls are thread-safe.
 * - Errors: every argument check happens before any launch. On error nothing
 *   is enqueued and outputs are untouched; the return value says why and
 *   sattn_last_error() gives a message (thread-local). A zero-size problem
 *   (for example B, H or N equal to 0) returns SATTN_OK and enqueues nothing;
 *   its pointers may then be NULL.
 * - Every output element is written; outputs need no initialization.
 */
#ifndef SATTN_H
#define SATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SATTN_F16 = 0,
  SATTN_BF16 = 1
} sattn_dtype_t;

typedef enum {
  SATTN_OK = 0,
  SATTN_ERR_NULL = 1,        /* a required pointer is NULL                     */
  SATTN_ERR_SHAPE = 2,       /* negative, inconsistent or overflowing sizes    */
  SATTN_ERR_DTYPE = 3,       /* dtype is not SATTN_F16 / SATTN_BF16            */
  SATTN_ERR_UNSUPPORTED = 4, /* valid but not implemented (e.g. D = 96)        */
  SATTN_ERR_ALIGN = 5,       /* pointer misaligned                             */
  SATTN_ERR_ALIAS = 6,       /* an output overlaps an input or another output  */
  SATTN_ERR_HIP = 7,         /* the HIP runtime reported an error at launch    */
  SATTN_ERR_VALUE = 8        /* bad scalar argument (scale not finite or <= 0) */
} sattn_status_t;

/* Static, human-readable name of a status code. Never NULL. */
const char* sattn_status_string(int status);

/* Message describing the last failed call on this thread ("" if none). */
const char* sattn_last_error(void);

/*
 * Batched multi-head attention forward ("Intermediate and advanced
 * extension", workshop table, streaming-attention row: the score and value
 * products taken tile by tile under a running rescale, with or without the
 * causal mask).
 *
 *   q, k, v, o : [B, H, N, D] contiguous, D innermost, dtype `dtype`.
 *   lse        : [B, H, N] float32.
 *   causal     : nonzero -> key j is eligible for query i iff j <= i
 *                (diagonal included; equal query and key lengths).
 * Key tiles wholly above the diagonal are skipped, not masked.
 */
int sattn_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
              int64_t B, int64_t H, int64_t N, int64_t D, int causal, float scale,
              void* stream);

/*
 * Split-KV partial states, non-causal ("Intermediate and advanced
 * extension", workshop table, split-softmax row: partial statistics as a
 * launch of their own; here applied to attention with K/V split into chunks).
 *
 *   q          : [B, Hq, Nq, D];  k, v : [B, Hkv, Nk, D]  (dtype `dtype`).
 *   Query head h reads KV head h / (Hq / Hkv); Hq % Hkv must be 0.
 *   chunk      : keys per chunk (> 0); C = ceil(Nk / chunk) chunks, chunk c
 *                covering keys [c*chunk, min(Nk, (c+1)*chunk)).
 *   part_m     : [B, Hq, Nq, C] float32, max scaled score of the chunk.
 *   part_l     : [B, Hq, Nq, C] float32, sum over the chunk of exp(S - m).
 *   part_acc   : [B, Hq, Nq, C, D] float32, sum of exp(S - m) * v,
 *                NOT divided by l.
 * The three buffers are private to this call and its following
 * sattn_merge (enqueue the merge on the same stream, or after an event).
 * Nk must be > 0 when B*Hq*Nq > 0. This entry point is non-causal; the
 * causal split over a key/value cache is sattn_fwd_split_cache.
 */
int sattn_fwd_split(int dtype, const void* q, const void* k, const void* v,
                    float* part_m, float* part_l, float* part_acc,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                    int64_t chunk, float scale, void* stream);

/*
 * Merge of partial states ("Attention algorithms and data movement",
 * lesson 01: combine by rescaled denominators, never average).
 *
 *   part_m, part_l : [rows, C] float32;  part_acc : [rows, C, D] float32.
 *   o              : [rows, D] dtype `dtype`;  lse : [rows] float32.
 * With M = max_c m_c and w_c = exp(m_c - M): L = sum_c w_c l_c,
 * O = sum_c w_c acc_c / L, lse = M + ln L, summed in ascending c.
 * An empty partial (m = -inf, l = 0) is the identity; a row whose partials
 * are all empty gives O = 0 and lse = -inf.
 */
int sattn_merge(int dtype, const float* part_m, const float* part_l, const float* part_acc,
                int64_t rows, int64_t C, int64_t D, void* o, float* lse, void* stream);

/*
 * Packed variable-length grouped-query attention ("Attention algorithms and
 * data movement", lessons 04 and 05).
 *
 *   q, o       : [T, Hq, D];  k, v : [T, Hkv, D]  (dtype `dtype`).
 *   lse        : [Hq, T] float32.
 *   cu_seqlens : device int32 [S + 1]; sequence s owns tokens
 *                [cu[s], cu[s+1]). The caller guarantees cu[0] = 0,
 *                non-decreasing, cu[S] = T and every length <= max_seqlen
 *                (checked by the Python binding on its host copy; the kernel
 *                clamps every index into [0, T) so a bad table cannot read
 *                or write out of bounds).
 *   Query head h reads KV head h / (Hq / Hkv); Hq % Hkv must be 0.
 *   Tokens attend only to keys of their own sequence; causal eligibility uses
 *   positions within the sequence (key r' is eligible for query r iff
 *   r' <= r, diagonal included).
 */
int sattn_fwd_varlen(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                     const int32_t* cu_seqlens, int64_t S, int64_t T, int64_t max_seqlen,
                     int64_t Hq, int64_t Hkv, int64_t D, int causal, float scale, void* stream);

/*
 * Queries against a key/value cache of another length, with grouped KV
 * heads ("Attention algorithms and data movement", lesson 04: unequal-length
 * alignment and empty rows from logical positions; lesson 05: GQA head
 * mapping and the cache payload shared by a group of query heads).
 *
 *   q, o       : [B, Hq, Nq, D];  k, v : [B, Hkv, Nk, D]  (dtype `dtype`).
 *   lse        : [B, Hq, Nq] float32.
 *   Query head h reads KV head h / (Hq / Hkv); Hq % Hkv must be 0.
 *   The queries are the last Nq tokens of a sequence whose cache holds Nk
 *   positions: query i sits at logical position i + (Nk - Nq)
 *   (bottom-right alignment; Nq = Nk is ordinary self-attention, Nq = 1 a
 *   decode step, 1 < Nq < Nk a chunk of a chunked prefill).
 *   causal     : nonzero -> key j is eligible for query i iff
 *                j <= i + (Nk - Nq); zero -> all Nk keys are eligible.
 *   A query with no eligible key (i + Nk - Nq < 0 when Nq > Nk, or Nk = 0)
 *   is an empty row: O = 0 and lse = -inf. k and v may be NULL when Nk = 0.
 * Key tiles after a query tile's last position are skipped, not masked.
 */
int sattn_fwd_cache(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                    int causal, float scale, void* stream);

/*
 * Backward pass: gradients of the loss sum(dO * O) with respect to q, k, v
 * ("Attention algorithms and data movement", lesson 03: differentiate the
 * normalized row with probabilities recomputed from the saved lse; lesson
 * 05: the query heads sharing a KV head add their gradients into it;
 * "Intermediate and advanced extension", softmax-backward row: the
 * gradient is formed row by row from P and dP, never as an N x N Jacobian).
 *
 *   q, o, dout, dq : [B, Hq, N, D];  k, v, dk, dv : [B, Hkv, N, D]  (dtype).
 *   lse            : [B, Hq, N] float32, as written by sattn_fwd /
 *                    sattn_fwd_cache for the same q, k, v, causal and scale.
 *   delta          : [B, Hq, N] float32 workspace (caller-owned, overwritten
 *                    with rowsum(dout * o); its contents are not a result).
 *   causal         : nonzero -> key j eligible for query i iff j <= i
 *                    (equal lengths, as in sattn_fwd).
 * With P = exp(scale q k^T - lse): dV = P^T dO, dS = P (dO V^T - delta),
 * dQ = scale dS K, dK = scale dS^T Q, accumulated in fp32 and rounded once;
 * P and dS enter the matrix products rounded to the input dtype. Two launches
 * on `stream` (dQ, which also writes delta, then dK/dV); no atomics, so
 * results are bitwise reproducible. dk, dv of a KV head sum its query heads
 * in ascending order.
 */
int sattn_bwd(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, float* delta, void* dq, void* dk, void* dv,
              int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int causal, float scale,
              void* stream);

/*
 * sattn_bwd without the delta workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The [B, Hq, N] float32 rows of
 * delta live in a fixed device array inside the library (8 MiB per GPU,
 * held until the process ends), so B*Hq*N must be <= 2^21 query rows;
 * larger problems return SATTN_ERR_UNSUPPORTED and enqueue nothing (use
 * sattn_bwd). The call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); on its first use on a device it looks up the
 * array's address there (hipGetSymbolAddress, with that device current).
 * Arguments, results and the other errors are those of sattn_bwd, which
 * runs the same kernels: the gradients are bit-identical to sattn_bwd's.
 * Every call on one GPU shares that GPU's array, and the dQ launch rewrites
 * every row it needs before the dK/dV launch reads it, so nothing has to be
 * cleared; calls that overlap on one GPU (different streams, or threads
 * without ordering) race on the array and must not be issued.
 */
int sattn_bwd_noalloc(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                      int64_t N, int64_t D, int causal, float scale, void* stream);

/*
 * Backward pass of sattn_fwd_cache (contiguous layouts): the same gradients
 * as sattn_bwd for Nq queries against an Nk-key cache, query i at position
 * i + (Nk - Nq) ("Attention algorithms and data movement", lessons 04 and
 * 05: unequal-length alignment, cache payload).
 *
 *   q, o, dout, dq : [B, Hq, Nq, D];  k, v, dk, dv : [B, Hkv, Nk, D]  (dtype).
 *   lse, delta     : [B, Hq, Nq] float32 (lse as written by sattn_fwd_cache
 *                    for the same inputs, causal and scale; delta a
 *                    caller-owned workspace).
 *   causal         : nonzero -> key j eligible for query i iff
 *                    j <= i + (Nk - Nq).
 * Queries with no eligible key (i + Nk - Nq < 0, or Nk = 0) get dq = 0. With
 * Nk = 0 only dq and delta are written and k, v, dk, dv may be NULL.
 * Errors as sattn_bwd. sattn_bwd is this call with Nq = Nk.
 */
int sattn_bwd_cache(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, float* delta, void* dq, void* dk, void* dv, int64_t B, int64_t Hq,
                    int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale, void* stream);

/*
 * Backward pass of sattn_fwd_varlen: the same gradients as sattn_bwd for
 * packed variable-length sequences with grouped KV heads ("Attention
 * algorithms and data movement", lesson 04: per-sequence boundaries and
 * positions; lesson 05: shared KV-head gradients).
 *
 *   q, o, dout, dq : [T, Hq, D];  k, v, dk, dv : [T, Hkv, D]  (dtype).
 *   lse            : [Hq, T] float32, as written by sattn_fwd_varlen for the
 *                    same inputs, cu_seqlens, causal and scale.
 *   delta          : [Hq, T] float32 workspace (caller-owned, overwritten).
 *   cu_seqlens     : device int32 [S+1], the same table as the forward
 *                    (cu[0] = 0, non-decreasing, cu[S] = T, every length
 *                    <= max_seqlen); validated on a host copy by the caller,
 *                    clamped to [0, T] by the kernels.
 *   causal         : nonzero -> key j eligible for query i of the same
 *                    sequence iff j <= i (positions within the sequence).
 * Tokens of a sequence see only that sequence. Every token row of dq, dk, dv
 * that belongs to a sequence is written; dk, dv of a KV head sum its query
 * heads in ascending order. Two launches on `stream`, no atomics.
 * Errors as sattn_fwd_varlen, plus null or misaligned gradient buffers and
 * overlaps of any output with any input.
 */
int sattn_bwd_varlen(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, float* delta, void* dq, void* dk, void* dv, const int32_t* cu_seqlens,
                     int64_t S, int64_t T, int64_t max_seqlen, int64_t Hq, int64_t Hkv, int64_t D, int causal,
                     float scale, void* stream);

/*
 * Backward pass of sattn_fwd_sparse on equal lengths (Nq = Nk = N): the same
 * gradients as sattn_bwd with the sparse operator's eligibility ("Attention
 * algorithms and data movement", lesson 06: block sparsity with skipped
 * tiles; lesson 07: sliding windows and global tokens).
 *
 *   q, o, dout, dq : [B, Hq, N, D];  k, v, dk, dv : [B, Hkv, N, D]  (dtype).
 *   lse            : [B, Hq, N] float32, as written by sattn_fwd_sparse with
 *                    Nq = Nk = N for the same inputs, rule and scale (rows
 *                    with no eligible key carry -inf and get dq = 0).
 *   delta          : [B, Hq, N] float32 workspace (caller-owned, overwritten).
 *   win_left, win_right, n_global, block_mask, mask_heads, block_q, block_k:
 *                    exactly as in sattn_fwd_sparse (with Nq = Nk = N).
 * Key tiles outside a query tile's window band and global prefix are not
 * visited (dQ), nor query tiles outside a key tile's band (dK/dV); blocks
 * whose mask bit is clear are skipped. Two launches on `stream`, no atomics.
 * Errors as sattn_bwd plus SATTN_ERR_VALUE (window bounds < -1, n_global < 0),
 * SATTN_ERR_UNSUPPORTED (block sizes), SATTN_ERR_SHAPE (mask_heads not 1 or
 * Hq) and SATTN_ERR_ALIAS (an output over the mask).
 */
int sattn_bwd_sparse(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, float* delta, void* dq, void* dk, void* dv, int64_t B, int64_t Hq,
                     int64_t Hkv, int64_t N, int64_t D, int causal, int64_t win_left, int64_t win_right,
                     int64_t n_global, const uint8_t* block_mask, int64_t mask_heads, int64_t block_q,
                     int64_t block_k, float scale, void* stream);

/*
 * Sparse attention: sattn_fwd_cache restricted to a sliding window, global
 * tokens and a block mask ("Attention algorithms and data movement", lesson
 * 06: count active blocks, block sparsity is a changed operator tested
 * against the matching sparse reference; lesson 07: window edges and global
 * tokens united without double-counting). Exact softmax over the kept keys.
 *
 *   Shapes, alignment (query i at position p = i + Nk - Nq), GQA map and
 *   causal rule as in sattn_fwd_cache. Key j is kept for query i iff
 *     (p - win_left <= j <= p + win_right     -- a bound of -1 is unlimited
 *      or j < n_global                        -- global keys, seen by all
 *      or p < n_global)                       -- global queries see all
 *     and (block_mask is NULL or block_mask[h][i / block_q][j / block_k] != 0)
 *     and (!causal or j <= p).
 *   block_mask : device uint8 [mask_heads, ceil(Nq / block_q),
 *                ceil(Nk / block_k)], mask_heads = 1 (every head) or Hq
 *                (query head h uses slice h); NULL = no block restriction.
 *                block_q must be a positive multiple of 32, block_k of 64.
 *   win_left, win_right >= -1; n_global >= 0. Nk <= 65536.
 * A query with no kept key is an empty row: O = 0, lse = -inf. Key tiles no
 * row of a workgroup keeps are neither loaded nor computed.
 */
int sattn_fwd_sparse(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal,
                     int64_t win_left, int64_t win_right, int64_t n_global,
                     const uint8_t* block_mask, int64_t mask_heads, int64_t block_q, int64_t block_k,
                     float scale, void* stream);

/*
 * sattn_fwd_cache on strided, sliced, transposed or broadcast read-only
 * inputs, loaded in place ("Intermediate and advanced extension", workshop
 * table, strided-softmax row: inputs addressed through their row and
 * element strides, so views need no copy; "Intermediate and advanced
 * workshop validation": direct loads against copy-then-kernel).
 *
 *   q_strides  : host int64[3], element strides of q's batch, head and row
 *                dims (q[b, h, i, d] at q + b*s[0] + h*s[1] + i*s[2] + d).
 *   kv_strides : host int64[3], the same for k and v, which share them
 *                (k and v may still be different tensors).
 *   o, lse     : dense [B, Hq, Nq, D] and [B, Hq, Nq], as in sattn_fwd_cache.
 * The head dim d is contiguous. Every stride must be >= 0 and a multiple of
 * 8 elements (16 bytes); 0 broadcasts a dim. The k/v row stride must be >= D
 * (k/v rows do not overlap) and Nk * (k/v row stride) * 2 bytes < 2^31; q
 * rows may overlap.
 * Alias checks use each input's extent: the last addressed element + 1.
 * Alignment, causal rule, GQA map and empty rows as in sattn_fwd_cache.
 */
int sattn_fwd_strided(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                      const int64_t* q_strides, const int64_t* kv_strides,
                      int causal, float scale, void* stream);

/*
 * Split-KV partial states against a key/value cache, optionally causal:
 * sattn_fwd_split with the alignment of sattn_fwd_cache (query i at logical
 * position i + (Nk - Nq)). Same shapes, buffers and merge as sattn_fwd_split;
 * with causal nonzero only keys j <= i + (Nk - Nq) of each chunk count, and a
 * chunk holding no eligible key for a row stores that row's empty state
 * (part_m = -inf, part_l = 0, part_acc = 0), the identity of sattn_merge
 * ("Attention algorithms and data movement", lesson 01).
 * causal = 0 gives exactly sattn_fwd_split.
 */
int sattn_fwd_split_cache(int dtype, const void* q, const void* k, const void* v,
                          float* part_m, float* part_l, float* part_acc,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                          int64_t chunk, int causal, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SATTN_H */
