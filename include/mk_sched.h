/*
 * mk_sched.h -- host continuous-batching scheduler for libmk: request
 * admission, the KV page allocator and the rows of each step.
 *
 * The pages describe a serving engine that keeps many requests in flight,
 * with continuous batching over a paged KV cache and ragged sequence lengths
 * ("Cohere Publishes One-Kernel Server for North Mini Code, Claims 1.58x vLLM
 * Speedup", opening section; "Inside the Megakernel Serving Engine for North
 * Mini Code", paragraph 1; "Cohere fuses an entire decode step into one GPU
 * program", paragraph 4). This component owns that host-side state and
 * produces the arguments of mk_forward_step (include/mk.h) for every step:
 *
 *   submit -> queued -> admitted (a slot, pages) -> prompt rows -> decode rows
 *          -> finished (max_new_tokens reached) or released -> pages freed
 *
 * Policy:
 *  - Admission is first come, first served: the oldest queued request is
 *    admitted when a slot is free and the pool can hold it (with
 *    reserve_full, its whole length is reserved at admission, so an admitted
 *    request never runs out of pages; without it, pages for its prompt plus
 *    one are required and later pages come on demand). A request that cannot
 *    be admitted blocks the ones behind it (no reordering).
 *  - Every step feeds one decode row per decoding request (in slot order),
 *    then prompt rows of requests still ingesting their prompt, in slot
 *    order, up to max_rows rows in all: a prompt is ingested in chunks of
 *    consecutive rows (mk_forward_step's runs).
 *  - Pages come from a free list (LIFO; initial order given by the caller or
 *    ascending) as positions cross page boundaries and return to it when a
 *    request ends. Slots are reused lowest first, so a request that joins in
 *    a freed slot takes its row.
 *
 * Host memory only: no HIP call, no device pointer. Not thread-safe: one
 * thread at a time per scheduler. No C++ exception crosses this boundary;
 * errors return a status and set mk_last_error().
 */
#ifndef MK_SCHED_H
#define MK_SCHED_H

#include <stddef.h>
#include <stdint.h>

#include "mk.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mk_sched_config {
    int32_t max_seqs;           /* requests running at once (slots), <= max_rows */
    int32_t max_rows;           /* rows per step, <= the handle's max_batch */
    int32_t page_size;          /* tokens per page (the handle's page_size) */
    int32_t max_pages_per_seq;  /* block-table row length (the handle's) */
    int64_t n_pages;            /* pages in the pool */
    int32_t reserve_full;       /* nonzero: reserve a request's whole length at admission */
    int32_t reserved[3];
} mk_sched_config;

typedef struct mk_sched mk_sched;

/* Create a scheduler. page_order: NULL (pages 0..n_pages-1, ascending) or n_pages
 * distinct page ids in the order the free list hands them out. */
mk_status mk_sched_create(const mk_sched_config* cfg, const int32_t* page_order, mk_sched** out);
void mk_sched_destroy(mk_sched* s);

/*
 * Queue a request. cached_len tokens are taken as already in the cache (pages
 * are allocated for them at admission; a prompt ingested elsewhere, or a
 * synthetic prefill); prompt (host, prompt_len >= 1 tokens) is fed at
 * positions cached_len .., and max_new_tokens tokens are generated after it
 * (each the caller's choice from the logits of the previous row).
 * Errors: MK_ERR_INVALID (duplicate id, bad lengths), MK_ERR_CAPACITY (longer
 * than max_pages_per_seq pages).
 */
mk_status mk_sched_submit(mk_sched* s, int64_t request_id, int32_t cached_len, const int32_t* prompt,
                          int32_t prompt_len, int32_t max_new_tokens);

/* End a queued or running request now (its pages return to the free list).
 * MK_ERR_INVALID if the id is unknown. */
mk_status mk_sched_release(mk_sched* s, int64_t request_id);

/*
 * Admit what fits and lay out the next step. Writes *batch rows (0 when no
 * request is running) into caller buffers of max_rows entries:
 *   seq_ids[row]       the request's slot (equal for the rows of one prompt chunk)
 *   positions[row]     position fed
 *   block_tables[row]  max_pages_per_seq page ids (entries past the position's page are 0)
 *   tokens[row]        token fed (host)
 *   sample[row]        1 if this row's logits choose the request's next token
 *   request_ids[row]   the request (may be NULL)
 * The arrays go to mk_forward_step as they are (tokens after a copy to the
 * device). MK_ERR_CAPACITY if a running request needs a page and none is
 * free (only without reserve_full; nothing changes: release something).
 */
mk_status mk_sched_next(mk_sched* s, int32_t* batch, int32_t* seq_ids, int32_t* positions, int32_t* block_tables,
                        int32_t* tokens, int32_t* sample, int64_t* request_ids);

/*
 * After the step laid out by the last mk_sched_next has run: next_tokens[row]
 * (host, read where sample[row] == 1) is appended to that request. Requests
 * that reach max_new_tokens finish: their ids go to finished_ids (up to
 * max_finished, may be NULL) and *n_finished (may be NULL) counts them.
 * MK_ERR_INVALID if no step is pending.
 */
mk_status mk_sched_commit(mk_sched* s, const int32_t* next_tokens, int32_t* n_finished, int64_t* finished_ids,
                          int32_t max_finished);

typedef struct mk_sched_stats {
    int32_t queued, running, free_pages, reserved_pages;
    int64_t admitted, finished, steps, rows, prompt_rows;
} mk_sched_stats;
mk_status mk_sched_get_stats(const mk_sched* s, mk_sched_stats* out);

/* Tokens of a request so far (prompt, then generated): copies up to cap into
 * out (may be NULL) and sets *n. MK_ERR_INVALID if the id is unknown (finished
 * requests are kept until mk_sched_release or destroy). */
mk_status mk_sched_tokens(const mk_sched* s, int64_t request_id, int32_t* out, int32_t cap, int32_t* n);

#ifdef __cplusplus
}
#endif

#endif /* MK_SCHED_H */
