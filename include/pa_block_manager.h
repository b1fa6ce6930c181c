/*
 * pa_block_manager.h - host-side manager of the paged KV pool: which
 * physical blocks hold which sequence's tokens.  It produces the inputs of
 * the device path in pagedattn.h: the slot_mapping of pa_reshape_and_cache
 * and the block_tables / context_lens of pa_decode, pa_decode_multi and
 * pa_prefill.  Host memory only; nothing here touches the GPU.
 *
 * What it manages (mini-infer docs, "Systems Architecture" figure, box
 * "Paged KV-Cache Memory Manager": a fixed pool of physical blocks, a
 * virtual-to-physical block table per request, a prefix cache; "Core
 * Capabilities at a Glance" table, rows "Memory Allocation", "OOM Resilience"
 * and "Prompt Caching"):
 *   - a pool of num_blocks blocks of block_size token slots; a sequence of
 *     L tokens holds ceil(L / block_size) blocks, token t in slot
 *     block_table[t / block_size] * block_size + t % block_size;
 *   - allocation takes the free block with the smallest id; when no block is
 *     free, a cached block (below) is evicted, the one released longest ago
 *     first (prefix reuse by block-level hash with LRU eviction: zingnex.cn
 *     mini-infer thread, feature list item 4);
 *   - prefix sharing (when enabled): a full block is identified by its
 *     block_size token ids and the identity of the block before it, so a
 *     block matches only under an identical prefix.  Admitting a prompt
 *     reuses the leading full blocks that match instead of allocating them;
 *     at least the prompt's last token is always left to compute.  A block
 *     becomes shareable once its sequence has moved past it - at the
 *     sequence's next pa_bm_append or at its release - by which time the
 *     prefill has written its K/V.  Released shareable blocks stay cached
 *     (reusable, evictable) until evicted;
 *   - preemption when the pool is exhausted: the running sequence with the
 *     lowest priority is released so its blocks return to the pool, the
 *     caller re-queues it as waiting (to be recomputed later);
 *   - rollback of rejected speculative tokens (pa_bm_truncate).
 *
 * Ownership: the manager owns its host memory; the caller owns every array
 * passed in or out.  Errors are return codes (the pagedattn.h status values);
 * a failed call changes nothing.  A manager is not
 * thread-safe: calls on one manager must not overlap.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stdint.h>

#include "pagedattn.h" /* status codes, including PA_ERR_NO_BLOCKS and PA_ERR_STATE */

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* A manager of num_blocks blocks of block_size tokens; a sequence may hold
 * up to max_blocks_per_seq blocks.  prefix_cache != 0 enables prefix
 * sharing.  Returns NULL for invalid arguments (num_blocks < 1,
 * block_size < 1, max_blocks_per_seq < 1) or when host memory runs out. */
pa_block_manager *pa_bm_create(int64_t num_blocks, int block_size, int max_blocks_per_seq,
                               int prefix_cache);
void pa_bm_destroy(pa_block_manager *bm);

/* Admit sequence seq_id with its prompt tokens[0 .. n) and a priority (a
 * larger value is preempted later).  *num_cached receives the number of
 * leading prompt tokens whose K/V the pool already holds (a multiple of
 * block_size, at most n - 1); slots_out[i] (n - *num_cached entries) is the
 * slot of prompt token *num_cached + i, the slot_mapping for appending the
 * prefill's K/V.  Errors: PA_ERR_NULL, PA_ERR_SHAPE (n < 1, or more than
 * max_blocks_per_seq blocks), PA_ERR_STATE (seq_id already admitted),
 * PA_ERR_NO_BLOCKS (not enough free or evictable blocks). */
int pa_bm_admit(pa_block_manager *bm, int64_t seq_id, int priority, const int32_t *tokens,
                int64_t n, int64_t *num_cached, int64_t *slots_out);

/* Extend running sequence seq_id by n tokens (a decode step's sampled token,
 * or a speculative draft).  slots_out[i] is the slot of token L + i, L the
 * length before the call.  tokens[0 .. n) are their ids (may be NULL when
 * prefix sharing is off).  Errors: PA_ERR_NULL, PA_ERR_SHAPE (n < 1 or the
 * block limit), PA_ERR_STATE (unknown seq_id), PA_ERR_NO_BLOCKS. */
int pa_bm_append(pa_block_manager *bm, int64_t seq_id, const int32_t *tokens, int64_t n,
                 int64_t *slots_out);

/* One decode step for a batch: appends tokens[i] (one token) to sequence
 * seq_ids[i] for every i < n_seqs and writes its slot to slots_out[i] - the
 * slot_mapping of the step's pa_reshape_and_cache (or the slots that
 * pa_append_decode derives from the tables).  All or nothing: when the pool
 * cannot supply every block the batch needs, PA_ERR_NO_BLOCKS and nothing
 * changes.  tokens may be NULL when prefix sharing is off.  Errors:
 * PA_ERR_NULL, PA_ERR_STATE (an unknown id, or an id listed twice; checked
 * first), PA_ERR_SHAPE (n_seqs < 0, or a sequence at its block limit). */
int pa_bm_decode_step(pa_block_manager *bm, const int64_t *seq_ids, int n_seqs,
                      const int32_t *tokens, int64_t *slots_out);

/* Shorten running sequence seq_id to new_len tokens (1 <= new_len <= its
 * length), returning the blocks past the new end (rejected draft tokens).
 * The block that will receive the next token must not be shared with another
 * sequence (PA_ERR_STATE otherwise); if it was shareable it stops being so,
 * since its later slots will be overwritten. */
int pa_bm_truncate(pa_block_manager *bm, int64_t seq_id, int64_t new_len);

/* Release sequence seq_id (finished or aborted): its blocks return to the
 * pool, shareable ones into the cache.  PA_ERR_STATE for an unknown id. */
int pa_bm_release(pa_block_manager *bm, int64_t seq_id);

/* Release the running sequence with the lowest priority (among equals, the
 * most recently admitted) and report it in *victim.  PA_ERR_STATE when no
 * sequence is running. */
int pa_bm_preempt(pa_block_manager *bm, int64_t *victim);

/* Rows of pa_decode's inputs for n_seqs running sequences, in the order of
 * seq_ids: tables_out [n_seqs, max_blocks_per_seq] int32 (entries past a
 * sequence's blocks are 0) and lens_out [n_seqs] int32.  PA_ERR_STATE for an
 * unknown id (nothing is written). */
int pa_bm_block_tables(const pa_block_manager *bm, const int64_t *seq_ids, int n_seqs,
                       int32_t *tables_out, int32_t *lens_out);

/* Launch order for a decode batch: writes to order_out the n_seqs ids of
 * seq_ids sorted by context length, longest first (equal lengths keep their
 * order in seq_ids).  A decode launch dispatches its workgroups in batch
 * order; when a batch has more (sequence, kv head) units than the GPU holds
 * at once, starting the longest sequences first keeps the last workgroups
 * short (longest-processing-time-first scheduling).  Pass order_out to
 * pa_bm_block_tables to build the rows in that order.  PA_ERR_STATE for an
 * unknown id (nothing is written); order_out must not overlap seq_ids. */
int pa_bm_order_longest_first(const pa_block_manager *bm, const int64_t *seq_ids, int n_seqs,
                              int64_t *order_out);

/* Pool accounting: blocks never used or released unshared (free), released
 * shareable blocks (cached, reusable until evicted), blocks held by running
 * sequences (used); free + cached + used = num_blocks.  *running receives the
 * number of running sequences.  Any pointer may be NULL. */
int pa_bm_stats(const pa_block_manager *bm, int64_t *free_blocks, int64_t *cached_blocks,
                int64_t *used_blocks, int64_t *running);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
