/*
 * pa.h — C ABI of libpa: paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the pages this library is built from:
 *   - "Module 4 · Batching, Scheduling, and Paging" (datasystem.school),
 *     section "PagedAttention": a sequence's cache lives in equal-sized
 *     blocks scattered over one pool, and a table per sequence names the
 *     physical block behind each of its logical blocks, so attention reads K
 *     and V by looking each block up in that table. Section "Block sharing":
 *     before a sample writes into a block it shares with other samples, the
 *     block is duplicated.
 *   - "Paging the KV Cache" (lecture 6), section "The waste hiding inside
 *     memory": the cache grows token by token.
 *   - worksonmygpu.com continuous-batching post, section "Selective batching":
 *     each request's query attends only over that request's own tokens with
 *     softmax(Q K^T / sqrt(d_k)) V; section "The prefill/decode mix": prefill
 *     chunks run in the same iteration as decode steps.
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every call
 * ---------------------------------------------------------------------------
 * Pointers. Every buffer pointer is a device pointer (HIP device memory) owned
 * by the caller; pool, query, K/V-row and output pointers must be 16-byte
 * aligned (kernels move 16-byte vectors). libpa allocates nothing, frees nothing and keeps no global
 * state; calls on different streams with disjoint buffers are independent.
 *
 * Streams. `stream` is a hipStream_t passed as void* (NULL = the null stream).
 * Every call only enqueues work on `stream` and returns: no host
 * synchronisation, no device-to-host read. Calls that depend on each other
 * must be issued in order on one stream: copy_blocks, then append_kv, then
 * decode / prefill_chunk.
 *
 * Element type. `dtype` is PA_F32 (float) or PA_BF16 (bfloat16). Queries,
 * pool, new K/V rows and outputs share it. Scores, softmax and accumulation
 * are float32; bfloat16 outputs are rounded to nearest even.
 *
 * KV pool layout (one layer). The pool is `num_blocks` blocks of
 * `2 * num_kv_heads * block_size * head_dim` elements each. Block j holds its
 * K half, then its V half; each half is `num_kv_heads` tiles of
 * `block_size * head_dim` elements, one per kv head:
 *   K tile: [head_dim/8][block_size][8]  (8-element slices of each token's
 *                                         vector; slice c of all slots is
 *                                         contiguous)
 *   V tile: [block_size/4][head_dim][4]  (4-token slices of each dimension)
 * With E = 2*Hkv*bs*d and T = bs*d, K element (block j, kv head g, slot s,
 * dim i) is at
 *   j*E + g*T + ((i/8)*bs + s)*8 + i%8,
 * and V element (j, g, s, i) at
 *   j*E + Hkv*T + g*T + ((s/4)*d + i)*4 + s%4.
 * Logical token t of a sequence with table row R lives in block R[t / bs] at
 * slot t % bs. A slot number is `block * block_size + offset`.
 *
 * Supported shapes: head_dim in {64, 128}; block_size in {16, 32};
 * num_q_heads = G * num_kv_heads with G in {1, 2, 4, 8}; query head h reads
 * kv head h / G.
 *
 * Errors. Arguments are validated on the host before anything is enqueued;
 * a non-zero return means nothing was enqueued. Device-side *contents* are
 * the caller's contract: block ids and slots must lie in [0, num_blocks) and
 * [0, num_blocks*block_size); context lengths in [0, max_blocks_per_seq *
 * block_size]. Kernels clamp out-of-range block ids and lengths so that they
 * never access memory outside the buffers, but the result is then unspecified.
 * A launch failure returns PA_ERR_LAUNCH.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* inconsistent or negative sizes */
  PA_ERR_UNSUPPORTED = 3, /* head_dim / block_size / group size / dtype not built */
  PA_ERR_WORKSPACE = 4,   /* workspace too small */
  PA_ERR_LAUNCH = 5,      /* the HIP launch failed */
  PA_ERR_ALIAS = 6,       /* output overlaps an input it must not overlap */
  PA_ERR_ALIGN = 7,       /* a data pointer is not 16-byte aligned */
  PA_ERR_HOST = 8         /* host pool is not pinned, device-mapped host memory */
};

/* Tokens per split-K partition of pa_decode. A sequence of n tokens is cut at
 * multiples of PA_DECODE_PARTITION; the cut never depends on the rest of the
 * batch, so a sequence's output does not depend on batch composition. */
#define PA_DECODE_PARTITION 1024

/*
 * pa_append_kv — write each new token's K and V into its block slot.
 * ("Paging the KV Cache", "The waste hiding inside memory": the cache grows
 * one token at a time; "Module 4", "PagedAttention": the slot's block comes
 * from the sequence's table.)
 *
 *   kv_pool      [num_blocks * E] pool, modified in place
 *   k_new, v_new [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping [num_tokens] int32: token i goes to slot slot_mapping[i];
 *                a negative slot skips the token (padding).
 * Copies are bitwise. Two tokens with the same slot in one call: undefined.
 * num_tokens == 0 is a valid no-op.
 */
int pa_append_kv(void* kv_pool, const void* k_new, const void* v_new,
                 const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                 int32_t dtype, void* stream);

/*
 * pa_copy_blocks — copy-on-write of whole blocks.
 * ("Module 4", section "Block sharing": on the first divergent write to a
 * shared block, the block is copied.)
 *
 *   block_pairs [num_pairs][2] int32 (src, dst): block dst becomes a bitwise
 *               copy of block src (K and V halves, all heads, all slots).
 * Every dst must be distinct and no dst may be the src of another pair
 * (otherwise undefined). num_pairs == 0 is a valid no-op.
 */
int pa_copy_blocks(void* kv_pool, const int32_t* block_pairs, int32_t num_pairs,
                   int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t dtype, void* stream);

/*
 * pa_decode_workspace_size — bytes of workspace pa_decode needs for a batch of
 * `num_seqs` sequences whose longest context is at most `max_context_len`.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                int32_t max_context_len);

/*
 * pa_decode — one decode step of paged attention for a ragged batch.
 * (worksonmygpu.com continuous-batching post, "Selective batching": per
 * request softmax(q K^T * scale) V over that request's own tokens; "Module 4",
 * "PagedAttention": K and V gathered through the block table.)
 *
 *   out           [num_seqs][num_q_heads][head_dim]  (must not overlap q)
 *   q             [num_seqs][num_q_heads][head_dim]
 *   block_tables  [num_seqs][max_blocks_per_seq] int32 physical block ids;
 *                 entries at or past ceil(n/bs) never address the pool (entry
 *                 0 of every row is read to choose the cache policy below,
 *                 whatever it holds).
 *   context_lens  [num_seqs] int32: sequence b attends to its logical tokens
 *                 0 .. context_lens[b]-1 (including a token appended this
 *                 step). A zero length gives a zero output row. Slots past
 *                 the context are never used, even when they hold NaN.
 *   max_context_len  host-side upper bound of context_lens (sizes the grid).
 *   scale         multiplies q.K (1/sqrt(head_dim) for standard attention).
 *   workspace     device buffer of at least pa_decode_workspace_size() bytes,
 *                 ZERO-FILLED before its first use. It holds work-queue
 *                 counters, which every call returns to zero, and partial
 *                 results. The counters' place does not depend on the batch
 *                 shape, so one workspace serves any sequence of calls on one
 *                 stream; calls that may run concurrently need separate
 *                 workspaces.
 * Sequences longer than PA_DECODE_PARTITION are split into partitions whose
 * partial softmax states are merged in partition order: inside the same
 * kernel for bfloat16 batches of up to 2048 sequences, by a second kernel on
 * the same stream otherwise.
 * Cache behaviour: a call whose K+V exceeds 256 MiB and in which no sequence
 * starts with its predecessor's first block streams K/V with nontemporal
 * loads (they are not kept in the caches); other calls load them cached. The
 * results are bit-identical either way.
 */
int pa_decode(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
              const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
              int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
              int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
              int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_shared — pa_decode for a batch whose sequences share leading
 * blocks, with the caller saying which. ("Module 4", "Block sharing": the
 * samples of one prompt point at the same physical blocks for the prompt.)
 *
 * Same arguments, checks and results as pa_decode (bit-identical outputs),
 * plus
 *   share_prev  device int32 [num_seqs], or NULL (then exactly pa_decode):
 *               share_prev[b] = the number of leading tokens of sequence b
 *               that sit in the same physical blocks as sequence b-1's
 *               (0 or negative: none; share_prev[0] is not read).
 * The hint only decides which sequences are computed together, never what is
 * computed: consecutive sequences that share whole PA_DECODE_PARTITION-token
 * partitions (and each have at least one partition of their own after them)
 * are stacked, up to 16 query rows, into one MFMA tile, so each shared block
 * is read once per stack instead of once per sequence. Every shared block id
 * is checked against each stacked sequence's own table before it is used; a
 * wrong hint only costs speed. bfloat16 batches of at most 2048 sequences
 * use it; other calls run pa_decode as it is.
 */
int pa_decode_shared(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
                     const int32_t* context_lens, const int32_t* share_prev, int32_t num_seqs,
                     int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, float scale, int32_t dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * pa_decode_append — one decode step: each sequence's new token is appended,
 * then every sequence attends over its context including that token.
 * ("Paging the KV Cache", "The waste hiding inside memory": the cache grows by
 * one token per generated token; worksonmygpu.com continuous-batching post,
 * "Selective batching": each request's attention over its own tokens.)
 *
 * The same results as pa_append_kv(kv_pool, k_new, v_new, slot_mapping,
 * num_seqs, ...) followed by pa_decode(...) on the same stream, bit for bit,
 * for calls in which slot_mapping[b] is the pool slot of position
 * context_lens[b]-1 in sequence b's table (as a scheduler's append gives).
 * Arguments as pa_decode, plus
 *   k_new, v_new  [num_seqs][num_kv_heads][head_dim], 16-byte aligned: the
 *                 key and value of position context_lens[b]-1 of sequence b.
 *   slot_mapping  [num_seqs] int32: the pool slot they are written to
 *                 (negative: not written; the attention still uses them).
 * The pool holds every new token when the call's work completes, as after
 * pa_append_kv; the call's own attention takes the new tokens from k_new and
 * v_new, not from the pool. bfloat16 batches of at most 2048 sequences run as
 * one kernel, which writes the new tokens after its loads; other calls run
 * the append and then the decode. Errors as pa_decode, and PA_ERR_NULL /
 * PA_ERR_ALIGN for k_new, v_new or slot_mapping.
 */
int pa_decode_append(void* out, const void* q, void* kv_pool, const int32_t* block_tables,
                     const int32_t* context_lens, const void* k_new, const void* v_new,
                     const int32_t* slot_mapping, int32_t num_seqs, int32_t max_blocks_per_seq,
                     int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                     int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill_chunk — attention of prefill chunks over a paged cache.
 * (worksonmygpu.com continuous-batching post, "The prefill/decode mix":
 * prompt chunks share the iteration with decode steps.)
 *
 * Chunk c's queries are rows query_start_loc[c] .. query_start_loc[c+1]-1 of
 * q; they are the last L_c of the chunk's context_lens[c] tokens, whose K/V
 * must already be appended. Query i of the chunk sits at position
 * a = context_lens[c] - L_c + i and attends to tokens 0..a (causal within the
 * chunk, full over earlier cached tokens).
 *
 *   out            [total_q_tokens][num_q_heads][head_dim]  (must not overlap q)
 *   q              [total_q_tokens][num_q_heads][head_dim]
 *   block_tables   [num_chunks][max_blocks_per_seq] int32
 *   context_lens   [num_chunks] int32, each >= its chunk length
 *   query_start_loc [num_chunks + 1] int32 device array, non-decreasing,
 *                  query_start_loc[0] = 0, query_start_loc[num_chunks] =
 *                  total_q_tokens
 *   max_chunk_len  host-side upper bound of the chunk lengths (sizes the grid)
 */
int pa_prefill_chunk(void* out, const void* q, const void* kv_pool,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* query_start_loc, int32_t num_chunks,
                     int32_t total_q_tokens, int32_t max_chunk_len,
                     int32_t max_blocks_per_seq, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                     int32_t dtype, void* stream);

enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 };

/*
 * pa_swap_blocks — move whole blocks between the device pool and a pool in
 * pinned host memory. ("Module 4 · Batching, Scheduling, and Paging",
 * section "PagedAttention": when HBM is exhausted a request is evicted, its
 * KV swapped to CPU memory or dropped and recomputed later.)
 *
 *   host_pool       num_host_blocks blocks of the same size and layout as the
 *                   device pool's, in pinned host memory that the device
 *                   addresses directly (hipHostMalloc, or a pinned torch
 *                   tensor); anything else returns PA_ERR_HOST.
 *   block_pairs     device int32 [num_pairs][2] (src, dst):
 *                   PA_SWAP_OUT copies device block src to host block dst,
 *                   PA_SWAP_IN copies host block src to device block dst.
 * Pairs must not write a block another pair of the call reads or writes.
 * The copy is a kernel reading and writing the host pool over the host link;
 * like every call it only enqueues on `stream`. Out-of-range ids are skipped.
 */
int pa_swap_blocks(void* kv_pool, void* host_pool, const int32_t* block_pairs, int32_t num_pairs,
                   int32_t direction, int32_t num_blocks, int32_t num_host_blocks,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                   void* stream);

/*
 * pa_mixed_attention — one iteration's decode batch and prefill chunks
 * together. (worksonmygpu.com continuous-batching post, "The prefill/decode
 * mix makes scheduling harder, not easier": prefill chunks and decode steps
 * share an iteration.)
 *
 * Computes exactly what pa_decode (dec_* arguments, workspace) and
 * pa_prefill_chunk (pre_* arguments) compute on the same pool, with the same
 * conventions, shapes, errors and results; either side may be empty
 * (num_seqs == 0, or num_chunks == 0). For bfloat16 batches of at most 2048
 * sequences and at most 1024 (chunk, position-block) prefill tiles both run
 * in one persistent launch (plus the decode split-K merge): workgroups take
 * decode items and prefill tiles from two shared work lists, so the
 * HBM-bound decode and the MFMA-bound prefill overlap on every CU. Otherwise
 * the two launches run in turn. Outputs must not overlap each other or either
 * query buffer (PA_ERR_ALIAS). The workspace is pa_decode's, for the decode
 * side's shape; its counters also serve the prefill work list.
 */
int pa_mixed_attention(void* dec_out, const void* dec_q, const int32_t* dec_block_tables,
                       const int32_t* dec_context_lens, int32_t num_seqs,
                       int32_t dec_max_blocks_per_seq, int32_t max_context_len, void* pre_out,
                       const void* pre_q, const int32_t* pre_block_tables,
                       const int32_t* pre_context_lens, const int32_t* query_start_loc,
                       int32_t num_chunks, int32_t total_q_tokens, int32_t max_chunk_len,
                       int32_t pre_max_blocks_per_seq, const void* kv_pool, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, float scale, int32_t dtype, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Bytes of the device array that pa_decode_noalloc uses as its workspace
 * (one array per device, held until the process ends). */
#define PA_DECODE_SCRATCH_BYTES (64u << 20)

/*
 * pa_decode_noalloc — pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, or harnesses that
 * forbid allocation. Same arguments, semantics, validation and results as
 * pa_decode (bit-identical outputs), without the workspace arguments: the
 * split-K partials and the work-queue counters live in a device array of
 * PA_DECODE_SCRATCH_BYTES owned by the library, whose address is looked up at
 * the first call on each device. Nothing is allocated or freed by any call.
 *
 * Limit: the batch's partials, packed in the call's element type, must fit:
 *   256 + round256(num_seqs * num_q_heads * P * head_dim * e)
 *       + round256(num_seqs * num_q_heads * P * 8) <= PA_DECODE_SCRATCH_BYTES,
 * with P = ceil(max_context_len / PA_DECODE_PARTITION) (at least 1), e = 4
 * for PA_F32 and 2 for PA_BF16; otherwise PA_ERR_WORKSPACE and nothing is
 * enqueued. (The 256-sequence, 64-query-head, head_dim 128, 8192-token bf16
 * batch needs about 34 MB.)
 *
 * Every call on one device shares that device's array, and each call leaves
 * its counters at zero. Calls that may overlap in time on one device (on
 * different streams, or from different host threads without ordering) race
 * on the array and give undefined results: order them on one stream, or use
 * pa_decode with separate workspaces.
 */
int pa_decode_noalloc(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                      int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                      int32_t dtype, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* pa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
