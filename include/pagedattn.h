/*
 * pagedattn.h - C ABI of libpagedattn.so: paged-KV attention for AMD MI355X
 * (gfx950).
 *
 * The calls implement the attention step of an LLM decode loop over a paged
 * KV cache, as the mini-infer pages describe it:
 *   - a fixed pool of physical KV blocks with a per-request
 *     virtual-to-physical block table (mini-infer docs,
 *     prajwal7-2002.github.io/mini-infer, "Systems Architecture" figure);
 *   - new K/V rows written straight to their physical slot, and one query
 *     token per sequence attending through the block table ("Batched Paged
 *     Decode", same page, "Core Capabilities at a Glance" table);
 *   - split-KV / flash-decoding partitioning of long contexts (zingnex.cn
 *     mini-infer thread, feature list item 7 "Flash Decoding"; MiniInfer
 *     README, "Attention Backend" table);
 *   - bounded prompt chunks attending causally to the cached prefix
 *     ("Prompt Ingestion", mini-infer docs, "Core Capabilities at a Glance").
 *
 * Conventions for every call
 *   - Tensors are caller-owned device memory, row-major and contiguous, in
 *     the layouts given per argument.  "bf16" means IEEE bfloat16 bit
 *     patterns (uint16 storage).
 *   - KV pool layout: k_cache, v_cache are [num_blocks, block_size,
 *     num_kv_heads, head_dim] bf16.  Slot s (s = block * block_size + offset)
 *     is row s of the pool viewed as [num_blocks * block_size, kv_heads *
 *     head_dim].
 *   - Grouped-query attention: q head h reads kv head h / (num_q_heads /
 *     num_kv_heads) (consecutive groups).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All device work is enqueued on it; no call synchronises, allocates or
 *     frees memory, or reads device memory on the host.
 *   - Supported shapes: head_dim 64 or 128; block_size 16 or 256;
 *     num_q_heads a multiple of num_kv_heads with a group of 1..8;
 *     num_q_heads <= PA_MAX_HEADS and num_seqs <= PA_MAX_SEQS (launch grid
 *     limits), else PA_ERR_SHAPE.
 *   - Errors are reported only through the returned status; on any status
 *     other than PA_OK from argument checking, nothing was enqueued.
 *     PA_ERR_HIP means a launch failed (hipGetLastError).  Faults inside a
 *     kernel surface asynchronously at the caller's next synchronisation.
 *   - Device-resident preconditions are NOT checked (checking would need a
 *     host sync): block ids in [0, num_blocks); context_lens[b] <=
 *     max_blocks_per_seq * block_size; valid slots unique within one call.
 *     Violating them is undefined behaviour.  pa_check_tables,
 *     pa_check_slots and pa_check_prefill (end of this header) check them
 *     on host copies, for tests and debug builds.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                      */
  PA_ERR_SHAPE = -2,       /* sizes inconsistent or out of range              */
  PA_ERR_UNSUPPORTED = -3, /* head_dim / block_size / group not supported     */
  PA_ERR_SPLITS = -4,      /* num_splits outside [0, PA_MAX_SPLITS]           */
  PA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required      */
  PA_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed      */
  PA_ERR_NO_BLOCKS = -7,   /* block manager: the pool cannot supply the blocks */
  PA_ERR_STATE = -8,       /* block manager: unknown/duplicate sequence, or a
                              forbidden state change                          */
  PA_ERR_SCRATCH = -9      /* pa_decode_noalloc: the call needs more than the
                              library's static scratch                        */
};

#define PA_MAX_SPLITS 256
#define PA_MAX_QUERY_TOKENS 8
#define PA_MAX_SEQS 65535
#define PA_MAX_HEADS 4096
/* Bytes of the static device scratch of pa_decode_noalloc (per device). */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/* Library version, as major * 10000 + minor * 100 + patch. */
int pa_version(void);

/* Human-readable name of a status code (static storage, never NULL). */
const char *pa_status_string(int status);

/*
 * Slot-mapped KV append.  For each token i < num_tokens with
 * s = slot_mapping[i] >= 0, copies k[i] (num_kv_heads * head_dim bf16) to
 * row s of k_cache and v[i] to row s of v_cache, bit for bit.  Negative slots
 * are padding and write nothing.  Source: "direct physical tensor gather with
 * zero-overhead slot mapping", mini-infer docs, "Core Capabilities at a
 * Glance" table, row "Batched Paged Decode (v0.2.1)".
 *   k, v          bf16 [num_tokens, num_kv_heads, head_dim]   (read)
 *   slot_mapping  int64 [num_tokens]                            (read)
 *   k_cache, v_cache  bf16 pools (written in place)
 * num_tokens may be 0 (nothing is enqueued).  Slots must be < num_blocks *
 * block_size (not checked; device-resident).
 */
int pa_reshape_and_cache(const void *k, const void *v, const int64_t *slot_mapping,
                         void *k_cache, void *v_cache, int64_t num_tokens, int64_t num_blocks,
                         int block_size, int num_kv_heads, int head_dim, void *stream);

/*
 * Paged decode: one query token per sequence attends to the first
 * context_lens[b] tokens of its sequence, fetched through block_tables
 * (PagedAttention over per-request block tables: psmarter/mini-infer summary,
 * "How It Works"; the unified [B, 1] paged decode of the mini-infer docs,
 * "Core Capabilities at a Glance" table, row "Batched Paged Decode"; the
 * split-KV pieces below: zingnex.cn mini-infer thread, feature list item 7,
 * and the MiniInfer README's "Attention Backend" table):
 *   out[b, h] = softmax_t(scale * q[b, h] . K_b[t, g]) V_b[t, g],  g = kv head of h,
 * with K_b[t] = k_cache[block_tables[b, t / block_size], t % block_size].
 * context_lens counts every cached token, including one appended this step.
 * A sequence with context length 0 gets a zero output.
 *
 * Split-KV: each sequence's token range is cut into contiguous pieces of
 * split_len tokens, split_len = round_up(ceil(max_blocks_per_seq *
 * block_size / S), 64), S = num_splits (0 = choose automatically, see
 * pa_decode_auto_splits).  Each piece is reduced independently to a partial
 * (normalised output, log-sum-exp) and a second kernel merges the pieces
 * with weights exp(lse_s - max lse).  With one piece per sequence the merge
 * is skipped and the first kernel writes `out` directly.
 *   q             bf16 [num_seqs, num_q_heads, head_dim]
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]
 *   context_lens  int32 [num_seqs]
 *   out           bf16 [num_seqs, num_q_heads, head_dim] (written, RNE from fp32)
 *   workspace     device scratch of at least
 *                 pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, S)
 *                 bytes for the S actually used (may be NULL when that is 0).
 *                 Calls that run concurrently must not share a workspace.
 *                 Its contents need no initialisation: the merge reads only
 *                 the pieces the split pass of the same call wrote.
 * Arithmetic: fp32 scores and accumulators from bf16 inputs; softmax weights
 * are rounded to bf16 before the weighted sum of V.
 */
int pa_decode(const void *q, const void *k_cache, const void *v_cache,
              const int32_t *block_tables, const int32_t *context_lens, float scale,
              int num_splits, void *out, int num_seqs, int num_q_heads, int num_kv_heads,
              int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
              void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step with the append fused in: for every sequence b with
 * context_lens[b] > 0, first writes new_k[b], new_v[b] (bf16 [num_seqs,
 * num_kv_heads, head_dim]) to the cache row of token context_lens[b] - 1 (the
 * slot block_tables[b, (L - 1) / block_size] * block_size + (L - 1) %
 * block_size), then computes exactly what pa_decode computes.  Equivalent to
 * pa_reshape_and_cache with those slots followed by pa_decode, in one kernel
 * launch fewer: the workgroup that reads a sequence's last token writes it
 * first.  k_cache and v_cache are written; the other arguments are as for
 * pa_decode.
 */
int pa_append_decode(const void *q, const void *new_k, const void *new_v, void *k_cache,
                     void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                     float scale, int num_splits, void *out, int num_seqs, int num_q_heads,
                     int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                     int max_blocks_per_seq, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * Multi-token decode: q_len query tokens per sequence, causal among
 * themselves, attend the paged cache in one pass - the target model's
 * parallel verification of a speculative draft of q_len - 1 tokens
 * ("Speculative Decoding: K-token draft proposals with parallel target
 * verification", mini-infer docs, "Core Capabilities at a Glance" table, row
 * "Generation Speed"; draft-model speculative decoding, zingnex.cn mini-infer
 * thread, feature list item 5).  The q_len tokens' K/V rows must already be
 * in the cache (pa_reshape_and_cache), and context_lens[b] counts them.
 * Query token j of sequence b sits at position p = context_lens[b] - q_len + j
 * and attends the keys t <= p of its sequence:
 *   out[b, j, h] = softmax_{t <= p}(scale * q[b, j, h] . K_b[t, g]) V_b[t, g].
 * A query token with p < 0 (a sequence shorter than q_len) gets a zero row.
 * q_len = 1 computes what pa_decode computes.  Split-KV as for pa_decode; the
 * pieces of a sequence serve all its query tokens, so the cache is read once
 * per step whatever q_len.
 *   q, out        bf16 [num_seqs, q_len, num_q_heads, head_dim]
 *   workspace     at least pa_decode_multi_workspace_size(num_seqs, q_len,
 *                 num_q_heads, head_dim, S) bytes for the S used.
 * Limits: 1 <= q_len <= PA_MAX_QUERY_TOKENS (else PA_ERR_SHAPE), and
 * (num_q_heads / num_kv_heads) * q_len <= 32 (else PA_ERR_UNSUPPORTED);
 * the other arguments and limits are those of pa_decode.
 */
int pa_decode_multi(const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, const int32_t *context_lens, float scale,
                    int num_splits, void *out, int num_seqs, int q_len, int num_q_heads,
                    int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                    int max_blocks_per_seq, void *workspace, size_t workspace_bytes,
                    void *stream);

/* Workspace bytes pa_decode_multi needs: fp32 partial rows
 * [num_seqs, q_len, num_q_heads, S, head_dim], then (256-byte aligned) their
 * base-2 log-sum-exp [num_seqs, q_len, num_q_heads, S].  0 when
 * num_splits <= 1 or for invalid arguments. */
size_t pa_decode_multi_workspace_size(int num_seqs, int q_len, int num_q_heads, int head_dim,
                                      int num_splits);

/*
 * FP8 KV pages.  The pools hold one byte per element: k_cache, v_cache are
 * [num_blocks, num_kv_heads, block_size, head_dim] uint8 codes of the OCP
 * 8-bit float format E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, subnormals, no infinities, 0x7F / 0xFF NaN, largest finite 448),
 * halving the pool's bytes and what a decode step reads.  The layout is
 * head-major, unlike the bf16 pools: the block_size rows of one kv head in
 * one block are contiguous, so a decode workgroup reads long sequential
 * runs; slot s is row s % block_size of block s / block_size for every kv
 * head.  K and V each carry
 * one fp32 scale for the whole pool: a code c stands for e4m3(c) * scale.
 * Source: quantised KV cache storage, "Mini-Infer: A High-Performance LLM
 * Inference Acceleration Engine for Production Environments" (zingnex.cn
 * thread, English), section "Memory Optimization and KV Cache Management";
 * the page names no format, so the format and the per-tensor scale are a
 * reading.
 *
 * pa_reshape_and_cache_fp8: the append of pa_reshape_and_cache with
 * quantisation - element x (bf16) of token i is stored at its slot as
 * e4m3(clamp(x * (1 / scale), -448, 448)), the reciprocal and the product
 * rounded to fp32, the conversion rounding to nearest even.  A NaN input
 * stores a NaN code.  k_scale, v_scale: finite, > 0, with a finite
 * reciprocal (else PA_ERR_SHAPE).  Other arguments as pa_reshape_and_cache,
 * with the pools as above.
 */
int pa_reshape_and_cache_fp8(const void *k, const void *v, const int64_t *slot_mapping,
                             void *k_cache, void *v_cache, float k_scale, float v_scale,
                             int64_t num_tokens, int64_t num_blocks, int block_size,
                             int num_kv_heads, int head_dim, void *stream);

/*
 * pa_decode over fp8 pools: computes what pa_decode computes with
 * K_b[t] = e4m3(k code) * k_scale and V_b[t] = e4m3(v code) * v_scale.  The
 * codes widen exactly to bf16 inside the kernel; k_scale joins the score
 * scale (fp32 product scale * k_scale) and v_scale multiplies the normalised
 * output.  Split-KV, workspace (pa_decode_workspace_size), outputs and limits
 * as for pa_decode; scale * k_scale * log2(e) must be finite (else
 * PA_ERR_SHAPE), and k_scale, v_scale follow pa_reshape_and_cache_fp8's rule.
 */
int pa_decode_fp8(const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *block_tables, const int32_t *context_lens, float scale,
                  float k_scale, float v_scale, int num_splits, void *out, int num_seqs,
                  int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                  int64_t num_blocks, int max_blocks_per_seq, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * pa_append_decode over fp8 pools: for every sequence b with
 * context_lens[b] > 0, first stores new_k[b], new_v[b] (bf16 [num_seqs,
 * num_kv_heads, head_dim]) quantised as pa_reshape_and_cache_fp8 quantises
 * them to the cache row of token context_lens[b] - 1, then computes what
 * pa_decode_fp8 computes - in one launch, the workgroup that reads a
 * sequence's last token writing it first.  Scales, pools and the other
 * arguments as for pa_decode_fp8.
 */
int pa_append_decode_fp8(const void *q, const void *new_k, const void *new_v, void *k_cache,
                         void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                         float scale, float k_scale, float v_scale, int num_splits, void *out,
                         int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                         int block_size, int64_t num_blocks, int max_blocks_per_seq,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_decode_multi over fp8 pools: q_len query tokens per sequence, causal
 * among themselves (the speculative verify step), with K and V dequantised
 * as for pa_decode_fp8.  q, out, workspace (pa_decode_multi_workspace_size)
 * and limits as for pa_decode_multi; scales as for pa_decode_fp8.
 */
int pa_decode_multi_fp8(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *block_tables, const int32_t *context_lens, float scale,
                        float k_scale, float v_scale, int num_splits, void *out, int num_seqs,
                        int q_len, int num_q_heads, int num_kv_heads, int head_dim,
                        int block_size, int64_t num_blocks, int max_blocks_per_seq,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * The two passes of pa_decode as separate calls, for callers that merge
 * pieces themselves (for example pieces of one sequence computed on
 * different devices) or time the passes apart.  Arguments mean what they mean
 * for pa_decode; num_splits = 0 chooses automatically, and the resolved
 * number of pieces must be at least 2 (otherwise PA_ERR_SPLITS: use
 * pa_decode, which then runs a single kernel).
 *
 * pa_decode_partials writes, for every sequence b, q head h and non-empty
 * piece s (s < ceil(context_lens[b] / split_len)), into the workspace:
 *   o_part[b, h, s, :]  fp32 [num_seqs, num_q_heads, S, head_dim] at byte 0,
 *                       the piece's softmax-normalised output;
 *   lse[b, h, s]        fp32 [num_seqs, num_q_heads, S] at byte
 *                       round_up(num_seqs * num_q_heads * S * head_dim * 4, 256),
 *                       log2 of the piece's sum of exp2(scale * log2(e) * q.k),
 *                       i.e. the base-2 log-sum-exp of the scaled scores.
 * Empty pieces are not written.  pa_decode_merge reads those partials for the
 * non-empty pieces and writes out[b, h] = sum_s 2^(lse_s - M) o_s /
 * sum_s 2^(lse_s - M), M = max_s lse_s, as bf16 (zeros when context_lens[b]
 * is 0).  Both need the same num_splits, block_size and max_blocks_per_seq so
 * that they resolve the same split_len.
 */
int pa_decode_partials(const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, const int32_t *context_lens, float scale,
                       int num_splits, int num_seqs, int num_q_heads, int num_kv_heads,
                       int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
                       void *workspace, size_t workspace_bytes, void *stream);

int pa_decode_merge(const void *workspace, size_t workspace_bytes, const int32_t *context_lens,
                    void *out, int num_splits, int num_seqs, int num_q_heads, int num_kv_heads,
                    int head_dim, int block_size, int max_blocks_per_seq, void *stream);

/* Workspace bytes pa_decode needs for a given split count (0 when
 * num_splits <= 1).  Returns 0 for invalid arguments. */
size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int head_dim, int num_splits);

/*
 * pa_decode for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, computation and results as pa_decode (the same
 * kernels, bit for bit at the same split count), minus the workspace: the
 * split partials go to a static device array of PA_NOALLOC_SCRATCH_BYTES
 * inside the library, one per device, held until the process ends.  Nothing
 * is allocated or freed, and the scratch needs no initialisation (the merge
 * reads only what the split pass of the same call wrote).
 *   - Every call on one device shares that device's scratch: calls that may
 *     run concurrently on one device (different streams, overlapping
 *     graphs) race and must be serialised by the caller.
 *   - A call whose split count needs more than PA_NOALLOC_SCRATCH_BYTES
 *     (pa_decode_workspace_size) returns PA_ERR_SCRATCH and enqueues
 *     nothing; pass a smaller num_splits, or use pa_decode.
 *   - The scratch's device address is looked up once per device, on the
 *     first call made with that device current (PA_ERR_HIP if the lookup
 *     fails).
 */
int pa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens, float scale,
                      int num_splits, void *out, int num_seqs, int num_q_heads,
                      int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                      int max_blocks_per_seq, void *stream);

/* Split count that pa_decode uses for num_splits = 0 on a device with
 * num_cus compute units.  Pure host arithmetic on the shapes (context
 * lengths are device-resident and are not read): it aims for about one
 * (sequence, kv head, piece) work unit per compute unit, so S = 1 once the
 * (sequence, kv head) pairs alone reach num_cus; the planned pieces never
 * go below 128 tokens (an explicit num_splits may ask for pieces of 64).
 * Returns a value in [1, PA_MAX_SPLITS], or a negative status for invalid
 * arguments. */
int pa_decode_plan_splits(int num_seqs, int num_kv_heads, int max_blocks_per_seq,
                          int block_size, int num_cus);

/* pa_decode_plan_splits with the compute-unit count of HIP device `device`
 * (queried once per device and cached). */
int pa_decode_auto_splits(int num_seqs, int num_kv_heads, int max_blocks_per_seq,
                          int block_size, int device);

/* Split count for a batch whose context lengths the host knows, in launch
 * order (context_lens: host int32 [num_seqs], e.g. from the block manager,
 * ordered longest first by pa_bm_order_longest_first).  The split pass
 * balances the work of a compute unit, not of a sequence (split-KV
 * partitioning, zingnex.cn mini-infer thread, feature list item 7; the
 * variable-length batches of continuous batching, MiniInfer README,
 * architecture figure, Scheduler box).  Returns pa_decode_plan_splits'
 * choice S0 when its workgroups (num_seqs * num_kv_heads * S0) exceed two per
 * compute unit.  Otherwise, for every piece count whose workgroups fit two
 * per compute unit and whose pieces are at least 128 tokens, it predicts the largest number of tokens of one kv head
 * a compute unit reads -- workgroup s * units + x (piece s of unit x) takes
 * compute unit (s * units + x) mod num_cus, and when the workgroups exceed
 * num_cus pa_decode hands the upper half of the pieces (2 s >= S) out in
 * mirrored unit order (piece s of unit units - 1 - x) -- adds 256 tokens for
 * the merge launch of any split, and returns the cheapest piece count, S0 on
 * ties.  Lengths beyond the table capacity count as the capacity.  Pure host
 * arithmetic; returns PA_ERR_NULL without lengths, PA_ERR_SHAPE for
 * num_cus > 65536, or a negative status for the shapes pa_decode_plan_splits
 * refuses. */
int pa_decode_plan_splits_lengths(const int32_t *context_lens, int num_seqs, int num_kv_heads,
                                  int max_blocks_per_seq, int block_size, int num_cus);

/* pa_decode_plan_splits_lengths with the compute-unit count of HIP device
 * `device`. */
int pa_decode_auto_splits_lengths(const int32_t *context_lens, int num_seqs, int num_kv_heads,
                                  int max_blocks_per_seq, int block_size, int device);

/*
 * Chunked prefill over the paged cache: sequence b contributes the
 * n_b = cu_seqlens_q[b + 1] - cu_seqlens_q[b] query rows
 * q[cu_seqlens_q[b] .. cu_seqlens_q[b + 1]), the last n_b tokens of a
 * sequence whose context_lens[b] tokens (cached prefix plus this chunk) are
 * all in the pool already (append the chunk's K/V first).  Query i sits at
 * position p = context_lens[b] - n_b + i and attends causally to keys
 * 0 .. p.  Source: "Bounded 512-token chunks interleaving prompt ingestion
 * with active decodes", mini-infer docs, "Core Capabilities at a Glance"
 * table, row "Prompt Ingestion (v0.2.1)".
 *   q            bf16 [total_q, num_q_heads, head_dim], total_q = cu_seqlens_q[num_seqs]
 *   cu_seqlens_q int32 [num_seqs + 1], non-decreasing, from 0
 *   out          bf16 [total_q, num_q_heads, head_dim]
 *   max_q_len    an upper bound of every n_b (sizes the launch grid); every
 *                n_b must also be <= context_lens[b] (not checked)
 *   num_splits   pieces of the key range (0 = choose automatically, see
 *                pa_prefill_plan_splits); with more than one piece a second
 *                kernel merges them by log-sum-exp, as in pa_decode
 *   workspace    at least pa_prefill_workspace_size(num_seqs, max_q_len,
 *                num_q_heads, head_dim, S) bytes for the S actually used
 *                (may be NULL when that is 0)
 * The QK^T and PV products run on the bf16 matrix cores (MFMA) with fp32
 * accumulation; softmax weights are rounded to bf16 for the PV product.
 */
int pa_prefill(const void *q, const int32_t *cu_seqlens_q, const void *k_cache,
               const void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
               float scale, int num_splits, void *out, int num_seqs, int max_q_len,
               int num_q_heads, int num_kv_heads, int head_dim, int block_size,
               int64_t num_blocks, int max_blocks_per_seq, void *workspace,
               size_t workspace_bytes, void *stream);

/*
 * pa_prefill over fp8 pools (head-major uint8 e4m3 codes, as for
 * pa_decode_fp8): K and V are the codes' values times k_scale and v_scale.
 * The codes widen exactly to bf16 inside the kernel; k_scale joins the score
 * scale, v_scale multiplies the normalised output.  Other arguments, the
 * workspace and the limits are those of pa_prefill; scales follow
 * pa_reshape_and_cache_fp8's rule and scale * k_scale * log2(e) must be
 * finite (else PA_ERR_SHAPE).
 */
int pa_prefill_fp8(const void *q, const int32_t *cu_seqlens_q, const void *k_cache,
                   const void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                   float scale, float k_scale, float v_scale, int num_splits, void *out,
                   int num_seqs, int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                   int block_size, int64_t num_blocks, int max_blocks_per_seq, void *workspace,
                   size_t workspace_bytes, void *stream);

/* Workspace bytes pa_prefill needs for a given split count (0 when
 * num_splits <= 1): each piece's normalised output rows, rounded to bf16,
 * then their fp32 log-sum-exp.  Returns 0 for invalid arguments. */
size_t pa_prefill_workspace_size(int num_seqs, int max_q_len, int num_q_heads, int head_dim,
                                 int num_splits);

/* Split count pa_prefill uses for num_splits = 0 on a device with num_cus
 * compute units: the key range is cut until the (32 query positions, kv
 * head, piece) work units number about one per compute unit.  Returns a value
 * in [1, PA_MAX_SPLITS] or a negative status. */
int pa_prefill_plan_splits(int num_seqs, int max_q_len, int num_kv_heads, int max_blocks_per_seq,
                           int block_size, int num_cus);

/*
 * Debug validation of the device-resident preconditions that the calls above
 * leave unchecked (checking them there would need a host synchronisation).
 * These run on the host, on HOST copies of the integer inputs: a caller (a
 * test, or a serving loop in a debug build) copies its tables, lengths, slots
 * or query offsets back, synchronously, and calls the check before the
 * attention call that will read them.  Plain host code: no HIP call, no
 * device access, nothing allocated on the device.
 *
 * Return value: PA_CHECK_OK when every precondition holds, else the kind of
 * the first violation found (a positive PA_CHECK_* code), with *bad_index set
 * (when bad_index is not NULL) to the offending sequence b or token i (-1 on
 * success); a negative PA_ERR_* status for invalid arguments (NULL pointers,
 * sizes out of range), with nothing checked.
 */
enum {
  PA_CHECK_OK = 0,
  PA_CHECK_LENGTH = 1,          /* context_lens[b] < 0 or > max_blocks_per_seq * block_size */
  PA_CHECK_BLOCK_ID = 2,        /* an entry block_tables[b, j] with j < ceil(L_b / block_size)
                                   lies outside [0, num_blocks)                              */
  PA_CHECK_APPEND_SHARED = 3,   /* fused append: the block receiving sequence b's new row is
                                   also read through another table entry in the same call   */
  PA_CHECK_SLOT_RANGE = 4,      /* slot_mapping[i] >= num_blocks * block_size                 */
  PA_CHECK_SLOT_DUPLICATE = 5,  /* slot_mapping[i] equals a valid slot of an earlier token    */
  PA_CHECK_QUERY_OFFSETS = 6    /* cu_seqlens_q[0] != 0, decreasing, n_b > max_q_len or
                                   n_b > context_lens[b]                                     */
};

/* Preconditions of pa_decode, pa_decode_multi, pa_decode_partials and their fp8
 * counterparts over host copies of block_tables [num_seqs, max_blocks_per_seq]
 * and context_lens [num_seqs]: every length in [0, max_blocks_per_seq *
 * block_size], every table entry a sequence reads in [0, num_blocks).  With
 * fused_append != 0 (pa_append_decode, pa_append_decode_fp8), also that the
 * block holding each non-empty sequence's last token (the row the call
 * writes) is read through no other table entry of the call, so no workgroup
 * reads a row while another writes it.  Lengths and entries are checked
 * sequence by sequence (a sequence's length before its entries); the
 * fused-append condition only once they all hold.  Requires block_size a
 * power of two, num_seqs >= 0, max_blocks_per_seq >= 1, num_blocks >= 1. */
int pa_check_tables(const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                    int max_blocks_per_seq, int block_size, int64_t num_blocks,
                    int fused_append, int64_t *bad_index);

/* Preconditions of pa_reshape_and_cache(_fp8) over a host copy of
 * slot_mapping [num_tokens]: every non-negative slot below num_blocks *
 * block_size and no valid slot repeated.  The reported token is the first one
 * (in token order) that is out of range or repeats an earlier valid slot. */
int pa_check_slots(const int64_t *slot_mapping, int64_t num_tokens, int64_t num_blocks,
                   int block_size, int64_t *bad_index);

/* Preconditions of pa_prefill(_fp8) on the query offsets, over host copies of
 * cu_seqlens_q [num_seqs + 1] and context_lens [num_seqs]: cu_seqlens_q[0] = 0,
 * non-decreasing, and every chunk n_b = cu_seqlens_q[b + 1] - cu_seqlens_q[b]
 * at most max_q_len and at most context_lens[b].  Pair it with
 * pa_check_tables for the tables and lengths. */
int pa_check_prefill(const int32_t *cu_seqlens_q, const int32_t *context_lens, int num_seqs,
                     int max_q_len, int64_t *bad_index);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
