/*
 * pakv_sched.h - C ABI of libpakv's host-side page allocator and request
 * admission for the shared K/V page pool of pakv.h.
 *
 * The policy follows "Curso gratuito recorre la inferencia de LLM con videos,
 * notas y un motor funcional en C++" (news-factory.app), section "¿Cómo
 * administra el motor la memoria de la caché KV?":
 *  - one shared pool of 16-token pages, one block table per sequence and
 *    layer;
 *  - a request is admitted only when the page budget it may need is free,
 *    and that budget is reserved whole at admission (no preemption, no
 *    recomputation later);
 *  - requests that do not fit wait in arrival order (first in, first out:
 *    a request never overtakes an earlier one);
 *  - a request whose budget exceeds the whole pool is rejected with an error;
 *  - static batching admits a new group only once every running request has
 *    finished; continuous batching admits queued requests whenever the budget
 *    allows.
 * Pages are returned to the pool when a request finishes (comrad404.com
 * review of the samir-vllm README, section "Что README говорит о KV-кэше и
 * пакетном декодировании": block tables per sequence and freeing pages).
 *
 * Budget of a request with P prompt tokens and N new tokens:
 *     pages_per_layer = ceil((P + N) / 16),  budget = num_layers * pages_per_layer
 * A request submitted with a shared prefix (pa_sched_submit_shared) reuses
 * the first floor(S / 16) full pages of every layer of its parent (S shared
 * tokens) by reference and needs only the rest. Shared pages are counted
 * once in the pool; a page returns to the pool when the last request that
 * references it finishes.
 *
 * The scheduler keeps host arrays that a decode step passes (after copying
 * them to the device) to pa_kv_append / pa_decode:
 *  - block tables, int32 [num_layers][max_batch][max_pages_per_seq]: row
 *    (layer, slot) lists the physical pages of the request in batch slot
 *    `slot`, logical page order; entries past its budget, and rows of empty
 *    slots, are -1;
 *  - context lengths, int32 [max_batch]: tokens of each slot's request that
 *    are in the cache (0 for an empty slot). A request admitted with a shared
 *    prefix starts at floor(S / 16) * 16 tokens.
 * The next token of the request in slot b goes to position context_lens[b]
 * (pa_kv_append), after which pa_sched_advance(…, 1) records it.
 *
 * All functions are host code, queue no GPU work and are not thread-safe.
 * Request ids are positive and never reused by one scheduler.
 */
#ifndef PAKV_SCHED_H
#define PAKV_SCHED_H

#include <stdint.h>

#include "pakv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_sched pa_sched;

enum { PA_BATCH_CONTINUOUS = 0, PA_BATCH_STATIC = 1 };

/*
 * Create a scheduler over a pool of num_pages pages (all free), for
 * num_layers layers, at most max_batch running requests, and block-table rows
 * of max_pages_per_seq entries. mode: PA_BATCH_CONTINUOUS or
 * PA_BATCH_STATIC. All counts must be >= 1.
 */
pa_status pa_sched_create(pa_sched** out, int32_t num_pages, int32_t num_layers,
                          int32_t max_batch, int32_t max_pages_per_seq, int32_t mode);
void pa_sched_destroy(pa_sched* sched);

/*
 * Queue a request of prompt_tokens + max_new_tokens tokens (both >= 0, sum
 * >= 1). PA_ERR_CAPACITY (nothing queued) when its budget exceeds the whole
 * pool or its pages per layer exceed max_pages_per_seq: it could never run.
 */
pa_status pa_sched_submit(pa_sched* sched, int32_t prompt_tokens, int32_t max_new_tokens,
                          int64_t* request_id);

/*
 * Queue a request whose first shared_tokens prompt tokens are those of the
 * running request parent_id (shared_tokens <= the parent's context length
 * and <= prompt_tokens). Its first floor(shared_tokens / 16) pages of every
 * layer are the parent's pages, referenced from this call on (they stay in
 * the cache even if the parent finishes first). PA_ERR_STATE if the parent
 * is not running; PA_ERR_CAPACITY as for pa_sched_submit, counting only the
 * pages it does not share.
 */
pa_status pa_sched_submit_shared(pa_sched* sched, int64_t parent_id, int32_t shared_tokens,
                                 int32_t prompt_tokens, int32_t max_new_tokens,
                                 int64_t* request_id);

/*
 * Admit queued requests in arrival order while the request at the head of
 * the queue fits (its budget is free and a batch slot is empty; static mode:
 * only while no request admitted earlier is still running, then as many as
 * fit). Each admitted request gets the lowest empty batch slot and its whole
 * budget of pages, written into its block-table rows. Writes at most
 * `capacity` ids to admitted_ids (in admission order) and their count to
 * *num_admitted.
 */
pa_status pa_sched_admit(pa_sched* sched, int64_t* admitted_ids, int32_t capacity,
                         int32_t* num_admitted);

/* Batch slot of a running request, -1 for a queued one. PA_ERR_INVALID for
 * an unknown (or finished) id. */
pa_status pa_sched_slot(const pa_sched* sched, int64_t request_id, int32_t* slot);

/* Record `tokens` more tokens written to the cache of a running request.
 * PA_ERR_STATE if it is queued; PA_ERR_INVALID if its context would pass
 * prompt_tokens + max_new_tokens or tokens < 0. */
pa_status pa_sched_advance(pa_sched* sched, int64_t request_id, int32_t tokens);

/* Finish (or cancel, if still queued) a request: its batch slot empties and
 * every page it references loses that reference. */
pa_status pa_sched_finish(pa_sched* sched, int64_t request_id);

/* Host arrays described above; valid until pa_sched_destroy. */
const int32_t* pa_sched_block_tables(const pa_sched* sched);
const int32_t* pa_sched_context_lens(const pa_sched* sched);

/* Free pages, queued requests, running requests (any pointer may be NULL). */
pa_status pa_sched_stats(const pa_sched* sched, int32_t* free_pages, int32_t* queued,
                         int32_t* running);

#ifdef __cplusplus
}
#endif

#endif /* PAKV_SCHED_H */
