/*
 * pa_sched.h — C ABI of libpa's host runtime: the KV block manager, the
 * iteration-level scheduler and the engine loop that drives the pa_* kernels
 * (include/pa.h) once per iteration.
 *
 * What the pages fix:
 *   - "Module 4 · Batching, Scheduling, and Paging" (datasystem.school):
 *       section "Static batching: the batch waits for its slowest member" —
 *         a fixed batch is released only when its longest member finishes;
 *       section "Continuous batching: reschedule every iteration" — finished
 *         sequences leave and waiting requests are admitted every iteration;
 *         Orca reserves the maximum response length per admitted request;
 *       section "PagedAttention" — the host owns the tables; a sequence
 *         gets a new block at the moment its last one is full, gives all of
 *         them back when it ends, and is pushed out (to be recomputed) when
 *         device memory runs short;
 *       section "Block sharing" — the samples of one prompt point at the
 *         prompt's blocks, a shared block is duplicated before a write that
 *         would make the samples differ, and a per-block count of sharers
 *         decides when the block is free again.
 *   - "Paging the KV Cache" (lecture 6), section "The waste hiding inside
 *     memory" — a max-length reservation per request fragments memory.
 *   - worksonmygpu.com continuous-batching post, sections "Iteration-level
 *     scheduling" and "The prefill/decode mix" — one iteration is one token
 *     per running sequence, and prompt prefill shares iterations with decode
 *     under a policy that bounds one iteration's work.
 *
 * The policy details the pages leave open (token budget per iteration, decode
 * first, chunked prefill, first-come-first-served admission without skipping,
 * which request is evicted, stack-ordered free list, prompt copies under
 * reservation) are stated with pa_sched_step below.
 *
 * Ownership and threads. A pa_sched or pa_engine object is created and
 * destroyed by these calls and used from one host thread at a time. The
 * scheduler touches host memory only. The engine owns a small pinned-host and
 * device ring for its per-iteration index packets (allocated at creation,
 * freed at destruction) and borrows every other buffer from the caller.
 */
#ifndef PA_SCHED_H
#define PA_SCHED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PA_POLICY_PAGED = 0,   /* continuous batching, blocks allocated on fill, eviction */
  PA_POLICY_RESERVE = 1, /* continuous batching, ceil(max_len / bs) blocks reserved per sample */
  PA_POLICY_STATIC = 2   /* static batches with the same reservation */
};

enum {
  PA_SCHED_FINISHED = 64, /* pa_sched_step / pa_engine_step: every request has finished */
  PA_ERR_STATE = 65       /* invariant broken: a lone request does not fit, or no progress */
};

typedef struct {
  int32_t num_blocks; /* blocks in the pool */
  int32_t block_size;
  int32_t max_seqs;   /* batch slots: samples that may run at once */
  int32_t max_tokens; /* tokens one iteration may process: decode + prefill */
  int32_t max_chunk;  /* longest prefill chunk */
  int32_t max_len;    /* longest context a sample may reach: prompt + output - 1 */
  int32_t policy;     /* PA_POLICY_* */
  int32_t num_host_blocks; /* PAGED only: host blocks for swapping evicted requests
                              (0: an evicted request is dropped and recomputed) */
  int32_t prefix_caching;  /* PAGED only, nonzero: reuse full prefix blocks across requests */
} pa_sched_config;

typedef struct pa_sched pa_sched;

/*
 * pa_sched_create — a scheduler over `num_requests` requests.
 *   free_order      [num_blocks] every block id once: the order in which blocks
 *                   are first handed out (later, a released block is the next
 *                   one handed out).
 *   prompt_lens     [num_requests] >= 1
 *   arrival         [num_requests] first iteration at which the request may be
 *                   admitted, non-decreasing (requests are queued in index order)
 *   sample_offsets  [num_requests + 1] request r has samples
 *                   sample_offsets[r] .. sample_offsets[r+1]-1 (at least one)
 *   output_lens     [sample_offsets[num_requests]] tokens each sample
 *                   generates, >= 1 (the first comes from the prompt's prefill)
 *   prefix_ids      [num_requests] or NULL: the shared prompt prefix a request
 *                   names (-1: none); requests naming one id share its first
 *                   prefix_lens[r] prompt tokens ("Module 4", section "Block
 *                   sharing", on sharing identical prefixes across requests)
 *   prefix_lens     [num_requests] or NULL: 0 <= prefix_lens[r] <= prompt_lens[r]
 * Returns PA_OK and *out, or PA_ERR_NULL / PA_ERR_SHAPE (bad config, bad
 * free_order, or a request that exceeds max_len, max_seqs or the pool even
 * when alone).
 */
int pa_sched_create(const pa_sched_config* cfg, const int32_t* free_order, int32_t num_requests,
                    const int32_t* prompt_lens, const int32_t* arrival,
                    const int32_t* sample_offsets, const int32_t* output_lens,
                    const int32_t* prefix_ids, const int32_t* prefix_lens, pa_sched** out);
void pa_sched_destroy(pa_sched* s);

/* Words (int32) a plan packet may take for this scheduler. */
int64_t pa_sched_plan_capacity(const pa_sched* s);

/* Blocks currently free. */
int32_t pa_sched_num_free(const pa_sched* s);

/*
 * pa_sched_step — plan one iteration and apply it to the scheduler's state.
 *
 * An iteration, in order:
 *   1. Copies owed from the previous iteration (reservation policies: the
 *      prompt's blocks into each further sample's reserved blocks) are
 *      emitted first.
 *   2. Requests whose arrival iteration has come join the waiting queue.
 *   3. PAGED: while the free blocks cannot cover what the running requests
 *      take this iteration — one block per decode sample whose last block is
 *      full or shared, plus the blocks of each continuing prefill chunk —
 *      the most recently admitted running request is evicted: its blocks are
 *      released and it goes back to the head of the queue. With host blocks
 *      configured, a decoding victim whose distinct blocks fit the free host
 *      blocks is swapped out (each distinct block, in sample then table order,
 *      to the next free host block) and keeps its progress; otherwise it
 *      restarts from its prompt.
 *   4. Decode: every unfinished sample of the running requests (admission
 *      order, then sample order) appends the KV of its last token, one slot
 *      (allocated when its last block is full; a shared block is copied
 *      first), and produces its next token; each takes one token of the
 *      iteration's budget of max_tokens.
 *   5. Prefill: each running request still in prefill gets its next chunk of
 *      min(remaining prompt, max_chunk, budget left) tokens.
 *   6. Admission (not after an eviction; STATIC only when no batch was
 *      running at the start of the iteration): a swapped head comes back when
 *      its unfinished samples fit the free slots and its blocks the free
 *      device blocks (one new block per host block, its samples sharing as
 *      before, host blocks released in order; no prefill, no budget). Else the
 *      head of the queue is admitted while it fits the free slots (its samples count from
 *      admission on), the budget (continuous policies only: a static batch is
 *      formed whole and its later members start prefill in later iterations),
 *      and the pool (PAGED: the blocks of its first chunk; reservation
 *      policies: ceil(max_len/bs) blocks per sample, taken now), and gets its
 *      first chunk if budget is left. The chunk that completes a
 *      prompt produces every sample's first token; PAGED samples then share
 *      the prompt's blocks.
 *   7. Samples that produced their last token release their blocks and slot
 *      (STATIC: the whole batch releases when its last sample is done).
 *
 * Prefix caching (PAGED, prefix_caching nonzero): a full block inside a
 * request's prefix, once prefilled, enters a cache under (prefix id, block
 * index); the cache holds a reference to it. An admitted request takes the
 * cached blocks of its prefix from block 0 up to the first miss (never its
 * whole prompt) and prefills only the rest. Entries are kept in
 * least-recently-used order (a hit or an entry moves to the back); when a
 * block is needed and none is free, the oldest entry that only the cache
 * holds gives its block up. Such blocks count as free in every fit test.
 *
 * The plan packet written to `buf` (int32 words):
 *   header [16]: 0 iteration, 1 tokens generated, 2 copies, 3 slots (tokens
 *     appended), 4 prefill tokens, 5 chunks, 6 decodes, 7 admitted,
 *     8 preempted, 9 finished, 10 MB = ceil(max_len/bs) (table row width),
 *     11 longest chunk, 12 swap-outs, 13 swap-ins, 14..15 zero;
 *   then: copies [copies][2] (src, dst); slots [slots] (prefill tokens in
 *     chunk order, then decode tokens in decode order); chunk_req [chunks];
 *     chunk_qsl [chunks+1] (query start of each chunk, then the prefill token
 *     count); chunk_ctx [chunks] (context after the chunk); chunk_tables
 *     [chunks][MB]; dec_req [decodes]; dec_sample [decodes]; dec_ctx [decodes]
 *     (context after the append); dec_tables [decodes][MB]; admitted;
 *     preempted; finished (request ids); swap_out [swap-outs][2] (device
 *     block, host block); swap_in [swap-ins][2] (host block, device block).
 *     Table rows are zero-padded. On the GPU the swap-outs run first, then
 *     the swap-ins, then the copies, appends and attention.
 * `buf` may be NULL (the plan is applied but not written); otherwise `cap`
 * must be at least pa_sched_plan_capacity(). *used receives the words
 * written. Returns PA_OK, PA_SCHED_FINISHED (nothing planned), PA_ERR_NULL,
 * PA_ERR_SHAPE (cap too small; the state is unchanged) or PA_ERR_STATE.
 */
int pa_sched_step(pa_sched* s, int32_t* buf, int64_t cap, int64_t* used);

/*
 * The engine: a scheduler driving the kernels of include/pa.h on one stream.
 * With host blocks configured it also owns that many pinned host blocks and
 * moves swapped blocks with pa_swap_blocks.
 * Every iteration's packet goes host -> device with one asynchronous copy
 * from a pinned ring slot, then pa_copy_blocks and pa_append_kv are
 * enqueued, then the attention: pa_mixed_attention when the iteration has
 * both prefill chunks and decodes, else pa_prefill_chunk or pa_decode (an
 * iteration of decodes only runs its append and decode as one
 * pa_decode_append). There are no model weights:
 * queries and new K/V rows come from caller buffers, row i of the
 * iteration's tokens (prefill tokens first, then decode tokens) reading row i
 * of k_rows / v_rows, prefill token i reading row i of q_prefill and decode i
 * reading row i of q_decode. The host never waits for the device except to
 * reuse a ring slot whose copy has not finished.
 *
 *   kv_pool     one layer's pool (include/pa.h layout), num_blocks of the
 *               scheduler's config
 *   q_prefill   [max_tokens][num_q_heads][head_dim]
 *   q_decode    [max_seqs][num_q_heads][head_dim]
 *   k_rows, v_rows [max_tokens][num_kv_heads][head_dim]
 *   out_prefill [max_tokens][num_q_heads][head_dim]
 *   out_decode  [max_seqs][num_q_heads][head_dim]
 *   workspace   pa_decode workspace for (max_seqs, num_q_heads, head_dim,
 *               max_len), zero-filled before first use
 * The scheduler stays owned by the caller and must outlive the engine.
 */
typedef struct pa_engine pa_engine;

typedef struct {
  int64_t iterations;
  int64_t generated;      /* tokens produced, including those of evicted attempts */
  int64_t prefill_tokens; /* prompt tokens processed, including recomputation */
  int64_t decode_tokens;
  int64_t decode_context_tokens; /* sum of the decodes' context lengths (tokens attended) */
  int64_t copies;
  int64_t evictions;
  int64_t swapped_blocks; /* blocks swapped out (each comes back in once) */
  double host_us;         /* host time spent planning and enqueueing */
  double wait_us;         /* host time spent waiting for a ring slot (the device is behind) */
} pa_engine_stats;

int pa_engine_create(pa_sched* s, void* kv_pool, int32_t num_kv_heads, int32_t num_q_heads,
                     int32_t head_dim, int32_t dtype, float scale, const void* q_prefill,
                     const void* q_decode, const void* k_rows, const void* v_rows,
                     void* out_prefill, void* out_decode, void* workspace,
                     size_t workspace_bytes, void* stream, pa_engine** out);
void pa_engine_destroy(pa_engine* e);

/* One iteration: plan it (copying the packet to `buf` when it is not NULL,
 * as pa_sched_step does) and enqueue its work. Returns as pa_sched_step, or
 * a pa_* kernel status. */
int pa_engine_step(pa_engine* e, int32_t* buf, int64_t cap, int64_t* used);

/* Iterations until every request has finished, then a stream synchronisation.
 * Statistics accumulate over every step of this engine. */
int pa_engine_run(pa_engine* e, pa_engine_stats* stats);

#ifdef __cplusplus
}
#endif

#endif /* PA_SCHED_H */
