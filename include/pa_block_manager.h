/*
 * pa_block_manager.h - the host-side block manager of libpagedattn: the block
 * pool and its free list, block tables, reference counts and the prefix
 * cache, copy-on-write, preemption and swapping, and the per-step scheduler
 * that turns them into the slot mapping, block tables and copy lists the
 * device entry points of pagedattn.h consume.
 *
 * What it follows
 * ---------------
 * - The pool is cut into fixed-size blocks held in a free list; allocating
 *   takes a block from it and freeing gives the block back, both O(1); a
 *   request that holds t tokens holds ceil(t/B) blocks ("How Paged Attention
 *   and Continuous Batching Actually Work", section "Paged attention: virtual
 *   memory for the KV cache").
 * - Entry j of a request's block table backs its logical tokens [jB, jB+B);
 *   token position p lives in slot table[p / B] * B + p % B.  Every full block
 *   is keyed by its token ids chained with the key of the prefix before it; a
 *   new prompt whose leading blocks are found under those keys maps them into
 *   its table with a bumped reference count and skips their prefill; freed
 *   blocks keep their key until reused, so a shared preamble stays warm
 *   ("LLM paged attention arch", sections "The architecture: every piece
 *   explained" and "End-to-end flow").
 * - A write into a block whose reference count exceeds one first takes a
 *   fresh block, copies the shared content into it, re-points the writer's
 *   table and drops one reference ("Paged Attention as a Memory Manager",
 *   section "Prefix Caching and Copy-on-Write").
 * - Each step serves the running requests first, granting each the slots for
 *   the tokens it needs (allocate_slots), then admits waiting requests while a
 *   per-step token budget lasts, feeding a long prompt in budget-sized slices;
 *   when the pool runs dry the lowest-priority (latest-arrived) request is
 *   preempted: its KV is copied to CPU blocks for a later swap-in, or dropped
 *   and recomputed from its tokens; shared blocks only lose a reference.
 *   Admission asks for the prompt's blocks plus a margin ("How Paged Attention
 *   and Continuous Batching Actually Work", sections "Continuous batching:
 *   schedule steps, not batches" and "One step, end to end"; "LLM paged
 *   attention arch", sections "The architecture: every piece explained" and
 *   "End-to-end flow").
 *
 * Choices the pages leave open
 * ----------------------------
 *  1. Free lists are queues: allocation takes the front, a freed block joins
 *     the back; at creation they hold blocks 0 .. N-1 in order.
 *  2. A request gives its blocks back last block first.
 *  3. Priority is arrival order.  Running requests are served in arrival
 *     order; the victim is the latest-arrived running request not yet served
 *     in the step (possibly the one asking).
 *  4. A prefix matches block by block from the start and stops at the first
 *     block not found; at most floor((len-1)/B) blocks are taken from the
 *     cache, so the last prompt token is always computed.  Keys are 128-bit
 *     chained hashes; a hit also compares the block's own tokens and its
 *     parent's key, so only a 128-bit collision of a parent chain could alias.
 *  5. A block's key leaves the cache when the block is taken for new content.
 *     A block filled with a prefix that is already cached stays unkeyed.
 *  6. Copy-on-write applies when the first position a request writes in a step
 *     lies inside an existing partial block with reference count > 1.
 *  7. A block freed during a step while it is the source of one of the step's
 *     copy-on-write copies rejoins the free list when the step ends, so no
 *     block is both a copy source and a copy destination in one step.
 *  8. A swap needs one CPU block per GPU block of the victim, else the victim
 *     is recomputed.  Swapped-in blocks are private and unkeyed.
 *  9. Swapped requests, then waiting ones, are taken in arrival order and only
 *     in a step without preemption; taking stops at the first that does not
 *     fit.  Admission checks the blocks of the whole prompt plus the margin;
 *     only the blocks of the scheduled slice are allocated.
 * 10. A fork copies the parent's tokens, computed count and table, adds a
 *     reference to every block, and arrives after every earlier request.
 *
 * Conventions
 * -----------
 * - Everything here is HOST memory and host work; nothing touches a GPU.
 * - A manager owns host memory for its own state from pa_bm_create to
 *   pa_bm_destroy.  It is not thread-safe: one thread at a time per manager.
 * - Request ids are caller-chosen int64 values, unique among live requests.
 *   Token ids are int32.
 * - Every call returns a pa_status (pagedattn.h); on an error nothing changes
 *   and pa_last_error() says why.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stdint.h>

#include "pagedattn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

typedef enum pa_request_state {
  PA_REQ_WAITING = 0, /* holds no blocks; admitted (or recomputed) by a later step */
  PA_REQ_RUNNING = 1, /* holds GPU blocks for its first `computed` tokens */
  PA_REQ_SWAPPED = 2  /* its KV sits in CPU blocks until swapped in */
} pa_request_state;

typedef enum pa_preempt_mode { PA_PREEMPT_RECOMPUTE = 0, PA_PREEMPT_SWAP = 1 } pa_preempt_mode;

typedef struct pa_bm_config {
  int64_t num_gpu_blocks;   /* blocks in the device pools, in [1, 2^31 - 1] */
  int64_t num_cpu_blocks;   /* blocks in the pinned host pools, in [0, 2^31 - 1] */
  int32_t block_size;       /* tokens per block, > 0 */
  int32_t prefix_caching;   /* 1: key full blocks and share them; 0: never share by prefix */
  int32_t preempt_mode;     /* pa_preempt_mode */
  int32_t watermark_blocks; /* free blocks admission and swap-in leave untouched, >= 0 */
} pa_bm_config;

/*
 * The work one step asks of the device, valid until the manager's next
 * pa_bm_schedule or pa_bm_destroy (HOST arrays owned by the manager).  Run in
 * this order on one stream: swap-out copies (pa_swap_blocks, device to host),
 * swap-in copies (host to device), copy-on-write copies (pa_copy_blocks), the
 * KV writes of every scheduled token (pa_kv_append with slot_mapping), then
 * attention over block_tables and context_lens.
 */
typedef struct pa_step_plan {
  int32_t num_seqs;                /* scheduled requests */
  int32_t num_tokens;              /* scheduled tokens, query_start[num_seqs] */
  int32_t max_blocks;              /* width of block_tables (>= 1) */
  int32_t num_cow;                 /* copy-on-write pairs */
  int32_t num_swap_out;            /* swap-out pairs */
  int32_t num_swap_in;             /* swap-in pairs */
  int32_t num_preempted;           /* requests preempted in this step */
  const int64_t *seq_ids;          /* [num_seqs] in schedule order */
  const int32_t *query_start;      /* [num_seqs + 1]: request k owns tokens
                                      [query_start[k], query_start[k+1]) */
  const int32_t *context_lens;     /* [num_seqs]: tokens in the cache after the writes;
                                      request k's tokens sit at positions
                                      context_lens[k] - n_k .. context_lens[k] - 1 */
  const int64_t *slot_mapping;     /* [num_tokens] cache slot of every scheduled token */
  const int32_t *block_tables;     /* [num_seqs][max_blocks]; entries past
                                      ceil(context_lens[k] / block_size) are 0 */
  const int64_t *cow_pairs;        /* [num_cow][2] (source, destination) GPU blocks */
  const int64_t *swap_out_pairs;   /* [num_swap_out][2] (GPU block, CPU block) */
  const int64_t *swap_in_pairs;    /* [num_swap_in][2] (CPU block, GPU block) */
  const int64_t *preempted_ids;    /* [num_preempted] in preemption order */
  const int32_t *preempted_modes;  /* [num_preempted] pa_preempt_mode actually applied */
} pa_step_plan;

typedef struct pa_bm_stats {
  int64_t free_gpu_blocks;
  int64_t free_cpu_blocks;
  int64_t cached_blocks;           /* keys in the prefix cache */
  int64_t running, waiting, swapped;
  /* totals since creation: the telemetry the pages name (block use,
     preemptions, prefix hits) */
  int64_t preemptions;
  int64_t swapped_out_blocks;
  int64_t swapped_in_blocks;
  int64_t cow_copies;
  int64_t prefix_hit_tokens;       /* prompt tokens taken from the cache at admission */
  int64_t admitted_tokens;         /* tokens of every admitted (or re-admitted) request */
} pa_bm_stats;

typedef struct pa_request_info {
  int32_t state;                   /* pa_request_state */
  int32_t reserved;
  int64_t arrival;                 /* 0, 1, 2, ... in order of add_request and fork */
  int64_t num_tokens;              /* prompt plus appended tokens */
  int64_t computed;                /* tokens whose KV is in the cache (GPU or CPU) */
  int64_t num_blocks;              /* GPU blocks held */
  int64_t num_cpu_blocks;          /* CPU blocks held */
} pa_request_info;

/* Creates a manager with every block free.  PA_ERR_SHAPE for sizes out of
 * range, PA_ERR_NOMEM if its host memory cannot be allocated. */
int pa_bm_create(const pa_bm_config *config, pa_block_manager **out);

/* Frees the manager and everything it owns (NULL is ignored). */
void pa_bm_destroy(pa_block_manager *bm);

/* A new waiting request with its prompt (num_tokens > 0).  PA_ERR_ID if the id
 * is live; PA_ERR_SHAPE if ceil(num_tokens/B) exceeds num_gpu_blocks minus
 * the watermark (it could never be admitted).  A request that later grows past
 * that size cannot be re-admitted after a preemption; finish it first. */
int pa_bm_add_request(pa_block_manager *bm, int64_t rid, const int32_t *tokens,
                      int64_t num_tokens);

/* Appends tokens (normally the one just sampled) to a live request; their KV
 * is computed by a later step. */
int pa_bm_append_tokens(pa_block_manager *bm, int64_t rid, const int32_t *tokens,
                        int64_t num_tokens);

/* Appends tokens[i] to request rids[i] for i < n: one sampled token for each of
 * many requests in one call.  Every id is checked first; on an error nothing
 * is appended. */
int pa_bm_append_batch(pa_block_manager *bm, const int64_t *rids, const int32_t *tokens,
                       int64_t n);

/* Parallel sampling: `child` starts as a copy of the running `parent` that
 * shares all its blocks.  PA_ERR_STATE unless the parent is running. */
int pa_bm_fork(pa_block_manager *bm, int64_t parent, int64_t child);

/* Ends a request in any state and gives back its GPU and CPU blocks at once. */
int pa_bm_finish(pa_block_manager *bm, int64_t rid);

/* One scheduling step under a budget of token_budget (> 0) tokens; fills *plan. */
int pa_bm_schedule(pa_block_manager *bm, int64_t token_budget, pa_step_plan *plan);

int pa_bm_get_stats(const pa_block_manager *bm, pa_bm_stats *out);

int pa_bm_request_info(const pa_block_manager *bm, int64_t rid, pa_request_info *out);

/* The request's GPU block table (cpu = 0) or its CPU blocks (cpu = 1): writes
 * min(count, capacity) ids to out and the full count to *count. */
int pa_bm_blocks(const pa_block_manager *bm, int64_t rid, int32_t cpu, int32_t *out,
                 int64_t capacity, int64_t *count);

/* Reference count of every GPU block, [num_gpu_blocks] into out. */
int pa_bm_refcounts(const pa_block_manager *bm, int32_t *out, int64_t capacity);

/* The GPU (cpu = 0) or CPU (cpu = 1) free list from front to back. */
int pa_bm_free_list(const pa_block_manager *bm, int32_t cpu, int32_t *out, int64_t capacity,
                    int64_t *count);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
