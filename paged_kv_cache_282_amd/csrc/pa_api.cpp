// libpa host API: argument validation and dispatch. See include/pa.h for the
// contract of every entry point. Nothing here allocates, synchronises or reads
// device memory; every check runs on the host before anything is enqueued.
#include "pa.h"
#include "pa_sched.h"

#include <hip/hip_runtime.h>

#include "pa_launch.h"

static_assert(pa::kPartition == PA_DECODE_PARTITION,
              "the kernels' split-K partition must be the one the workspace is sized for");

namespace {

bool supported_dims(int32_t head_dim, int32_t block_size) {
  return (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32);
}

bool supported_dtype(int32_t dtype) { return dtype == PA_F32 || dtype == PA_BF16; }

size_t elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : 2; }

int check_pool(int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
               int32_t dtype) {
  if (num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return PA_ERR_SHAPE;
  if (!supported_dtype(dtype) || !supported_dims(head_dim, block_size)) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int check_heads(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return PA_ERR_SHAPE;
  const int32_t g = num_q_heads / num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return na && nb && pa < pb + nb && pb < pa + na;
}

pa::PoolShape shape(int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size) {
  pa::PoolShape ps;
  ps.num_blocks = num_blocks;
  ps.num_kv_heads = num_kv_heads;
  ps.head_dim = head_dim;
  ps.block_size = block_size;
  return ps;
}

int status_of(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

int pa_append_kv(void* kv_pool, const void* k_new, const void* v_new,
                 const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                 void* stream) {
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (int s = check_pool(num_blocks, num_kv_heads, head_dim, block_size, dtype)) return s;
  if (num_tokens == 0) return PA_OK;
  if (!kv_pool || !k_new || !v_new || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(kv_pool) || !aligned16(k_new) || !aligned16(v_new)) return PA_ERR_ALIGN;
  if (int64_t(num_blocks) * block_size > INT32_MAX) return PA_ERR_SHAPE;
  return status_of(pa::launch_append(kv_pool, k_new, v_new, slot_mapping, num_tokens,
                                     shape(num_blocks, num_kv_heads, head_dim, block_size), dtype,
                                     static_cast<hipStream_t>(stream)));
}

int pa_copy_blocks(void* kv_pool, const int32_t* block_pairs, int32_t num_pairs,
                   int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t dtype, void* stream) {
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (int s = check_pool(num_blocks, num_kv_heads, head_dim, block_size, dtype)) return s;
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > 65535) return PA_ERR_SHAPE;  // grid.y limit
  if (!kv_pool || !block_pairs) return PA_ERR_NULL;
  if (!aligned16(kv_pool)) return PA_ERR_ALIGN;
  return status_of(pa::launch_copy(kv_pool, block_pairs, num_pairs,
                                   shape(num_blocks, num_kv_heads, head_dim, block_size), dtype,
                                   static_cast<hipStream_t>(stream)));
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                int32_t max_context_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  return pa::DecodeWorkspace::layout(num_seqs, num_q_heads, head_dim,
                                     pa::decode_max_parts(max_context_len))
      .total;
}

}  // extern "C"

namespace {

// Host checks of a decode batch with at least one sequence (pool and heads
// already checked), apart from its workspace.
int check_decode_batch(void* out, const void* q, const void* kv_pool,
                       const int32_t* block_tables, const int32_t* context_lens,
                       int32_t num_seqs, int32_t max_blocks_per_seq, int32_t max_context_len,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t dtype) {
  if (!out || !q || !kv_pool || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(kv_pool)) return PA_ERR_ALIGN;
  if (max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (int64_t(max_context_len) > int64_t(max_blocks_per_seq) * block_size) return PA_ERR_SHAPE;
  const int64_t parts = pa::decode_max_parts(max_context_len);
  if (int64_t(num_seqs) * num_kv_heads * parts > (int64_t(1) << 30)) return PA_ERR_SHAPE;
  if (int64_t(num_seqs) * num_kv_heads > INT32_MAX) return PA_ERR_SHAPE;  // merge grid
  const size_t qbytes = size_t(num_seqs) * num_q_heads * head_dim * elem_bytes(dtype);
  if (overlaps(out, qbytes, q, qbytes)) return PA_ERR_ALIAS;
  return PA_OK;
}

// The same, with a caller's workspace.
int check_decode(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
                 const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                 int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                 int32_t head_dim, int32_t block_size, int32_t dtype, void* workspace,
                 size_t workspace_bytes) {
  if (!workspace) return PA_ERR_NULL;
  if (!aligned16(workspace)) return PA_ERR_ALIGN;
  if (int s = check_decode_batch(out, q, kv_pool, block_tables, context_lens, num_seqs,
                                 max_blocks_per_seq, max_context_len, num_q_heads, num_kv_heads,
                                 head_dim, block_size, dtype))
    return s;
  if (workspace_bytes < pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len))
    return PA_ERR_WORKSPACE;
  return PA_OK;
}

// Host checks of a prefill batch with at least one chunk and token.
int check_prefill(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
                  const int32_t* context_lens, const int32_t* query_start_loc,
                  int32_t num_chunks, int32_t total_q_tokens, int32_t max_chunk_len,
                  int32_t max_blocks_per_seq, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t dtype) {
  if (!out || !q || !kv_pool || !block_tables || !context_lens || !query_start_loc)
    return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(kv_pool)) return PA_ERR_ALIGN;
  if (max_blocks_per_seq <= 0 || max_chunk_len <= 0 || max_chunk_len > total_q_tokens)
    return PA_ERR_SHAPE;
  if (num_chunks > 65535 || num_kv_heads > 65535) return PA_ERR_SHAPE;  // grid y/z limits
  const size_t qbytes = size_t(total_q_tokens) * num_q_heads * head_dim * elem_bytes(dtype);
  if (overlaps(out, qbytes, q, qbytes)) return PA_ERR_ALIAS;
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_decode(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
              const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
              int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
              int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
              int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0) return PA_ERR_SHAPE;
  if (int s = check_pool(num_blocks, num_kv_heads, head_dim, block_size, dtype)) return s;
  if (int s = check_heads(num_q_heads, num_kv_heads)) return s;
  if (num_seqs == 0) return PA_OK;
  if (int s = check_decode(out, q, kv_pool, block_tables, context_lens, num_seqs,
                           max_blocks_per_seq, max_context_len, num_q_heads, num_kv_heads,
                           head_dim, block_size, dtype, workspace, workspace_bytes))
    return s;
  return status_of(pa::launch_decode(out, q, kv_pool, block_tables, context_lens, num_seqs,
                                     max_blocks_per_seq, max_context_len, num_q_heads,
                                     shape(num_blocks, num_kv_heads, head_dim, block_size), scale,
                                     dtype, workspace, static_cast<hipStream_t>(stream)));
}

int pa_decode_shared(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
                     const int32_t* context_lens, const int32_t* share_prev, int32_t num_seqs,
                     int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, float scale, int32_t dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0) return PA_ERR_SHAPE;
  if (int s = check_pool(num_blocks, num_kv_heads, head_dim, block_size, dtype)) return s;
  if (int s = check_heads(num_q_heads, num_kv_heads)) return s;
  if (num_seqs == 0) return PA_OK;
  if (int s = check_decode(out, q, kv_pool, block_tables, context_lens, num_seqs,
                           max_blocks_per_seq, max_context_len, num_q_heads, num_kv_heads,
                           head_dim, block_size, dtype, workspace, workspace_bytes))
    return s;
  return status_of(pa::launch_decode(out, q, kv_pool, block_tables, context_lens, num_seqs,
                                     max_blocks_per_seq, max_context_len, num_q_heads,
                                     shape(num_blocks, num_kv_heads, head_dim, block_size), scale,
                                     dtype, workspace, static_cast<hipStream_t>(stream),
                                     share_prev));
}

int pa_decode_append(void* out, const void* q, void* kv_pool, const int32_t* block_tables,
                     const int32_t* context_lens, const void* k_new, const void* v_new,
                     const int32_t* slot_mapping, int32_t num_seqs, int32_t max_blocks_per_seq,
                     int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                     int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0) return PA_ERR_SHAPE;
  if (int s = check_pool(num_blocks, num_kv_heads, head_dim, block_size, dtype)) return s;
  if (int s = check_heads(num_q_heads, num_kv_heads)) return s;
  if (num_seqs == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return PA_ERR_ALIGN;
  if (int64_t(num_blocks) * block_size > INT32_MAX) return PA_ERR_SHAPE;
  if (int s = check_decode(out, q, kv_pool, block_tables, context_lens, num_seqs,
                           max_blocks_per_seq, max_context_len, num_q_heads, num_kv_heads,
                           head_dim, block_size, dtype, workspace, workspace_bytes))
    return s;
  return status_of(pa::launch_decode_append(
      out, q, kv_pool, block_tables, context_lens, k_new, v_new, slot_mapping, num_seqs,
      max_blocks_per_seq, max_context_len, num_q_heads,
      shape(num_blocks, num_kv_heads, head_dim, block_size), scale, dtype, workspace,
      static_cast<hipStream_t>(stream)));
}

int pa_decode_noalloc(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                      int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                      int32_t dtype, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0) return PA_ERR_SHAPE;
  if (int s = check_pool(num_blocks, num_kv_heads, head_dim, block_size, dtype)) return s;
  if (int s = check_heads(num_q_heads, num_kv_heads)) return s;
  if (num_seqs == 0) return PA_OK;
  // the library's array stands in for the workspace: every other check of
  // pa_decode, then the packed layout against the array's size
  const size_t need = pa::DecodeWorkspace::layout(num_seqs, num_q_heads, head_dim,
                                                  pa::decode_max_parts(max_context_len),
                                                  elem_bytes(dtype))
                          .total;
  if (int s = check_decode_batch(out, q, kv_pool, block_tables, context_lens, num_seqs,
                                 max_blocks_per_seq, max_context_len, num_q_heads, num_kv_heads,
                                 head_dim, block_size, dtype))
    return s;
  if (need > pa::kDecodeScratchBytes) return PA_ERR_WORKSPACE;
  return status_of(pa::launch_decode_noalloc(
      out, q, kv_pool, block_tables, context_lens, num_seqs, max_blocks_per_seq, max_context_len,
      num_q_heads, shape(num_blocks, num_kv_heads, head_dim, block_size), scale, dtype,
      static_cast<hipStream_t>(stream)));
}

int pa_prefill_chunk(void* out, const void* q, const void* kv_pool,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* query_start_loc, int32_t num_chunks,
                     int32_t total_q_tokens, int32_t max_chunk_len,
                     int32_t max_blocks_per_seq, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                     int32_t dtype, void* stream) {
  if (num_chunks < 0 || total_q_tokens < 0 || max_chunk_len < 0 || max_blocks_per_seq < 0)
    return PA_ERR_SHAPE;
  if (int s = check_pool(num_blocks, num_kv_heads, head_dim, block_size, dtype)) return s;
  if (int s = check_heads(num_q_heads, num_kv_heads)) return s;
  if (num_chunks == 0 || total_q_tokens == 0) return PA_OK;
  if (int s = check_prefill(out, q, kv_pool, block_tables, context_lens, query_start_loc,
                            num_chunks, total_q_tokens, max_chunk_len, max_blocks_per_seq,
                            num_q_heads, num_kv_heads, head_dim, dtype))
    return s;
  return status_of(pa::launch_prefill(out, q, kv_pool, block_tables, context_lens,
                                      query_start_loc, num_chunks, total_q_tokens, max_chunk_len,
                                      max_blocks_per_seq, num_q_heads,
                                      shape(num_blocks, num_kv_heads, head_dim, block_size),
                                      scale, dtype, static_cast<hipStream_t>(stream)));
}

int pa_swap_blocks(void* kv_pool, void* host_pool, const int32_t* block_pairs, int32_t num_pairs,
                   int32_t direction, int32_t num_blocks, int32_t num_host_blocks,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                   void* stream) {
  if (num_pairs < 0 || num_host_blocks < 0) return PA_ERR_SHAPE;
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN) return PA_ERR_SHAPE;
  if (int s = check_pool(num_blocks, num_kv_heads, head_dim, block_size, dtype)) return s;
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > 65535) return PA_ERR_SHAPE;  // grid.y limit
  if (!kv_pool || !host_pool || !block_pairs) return PA_ERR_NULL;
  if (!aligned16(kv_pool) || !aligned16(host_pool)) return PA_ERR_ALIGN;
  // The host pool must be pinned memory the device can address; its device
  // address is looked up (the same value under unified addressing).
  void* host_dev = nullptr;
  if (hipHostGetDevicePointer(&host_dev, host_pool, 0) != hipSuccess || !host_dev) {
    (void)hipGetLastError();  // leave no error behind for a later launch check
    return PA_ERR_HOST;
  }
  return status_of(pa::launch_swap(kv_pool, host_dev, block_pairs, num_pairs,
                                   direction == PA_SWAP_OUT, num_host_blocks,
                                   shape(num_blocks, num_kv_heads, head_dim, block_size), dtype,
                                   static_cast<hipStream_t>(stream)));
}

int pa_mixed_attention(void* dec_out, const void* dec_q, const int32_t* dec_block_tables,
                       const int32_t* dec_context_lens, int32_t num_seqs,
                       int32_t dec_max_blocks_per_seq, int32_t max_context_len, void* pre_out,
                       const void* pre_q, const int32_t* pre_block_tables,
                       const int32_t* pre_context_lens, const int32_t* query_start_loc,
                       int32_t num_chunks, int32_t total_q_tokens, int32_t max_chunk_len,
                       int32_t pre_max_blocks_per_seq, const void* kv_pool, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, float scale, int32_t dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || dec_max_blocks_per_seq < 0 || max_context_len < 0 || num_chunks < 0 ||
      total_q_tokens < 0 || max_chunk_len < 0 || pre_max_blocks_per_seq < 0)
    return PA_ERR_SHAPE;
  if (int s = check_pool(num_blocks, num_kv_heads, head_dim, block_size, dtype)) return s;
  if (int s = check_heads(num_q_heads, num_kv_heads)) return s;
  const bool dec = num_seqs > 0, pre = num_chunks > 0 && total_q_tokens > 0;
  if (dec) {
    if (int s = check_decode(dec_out, dec_q, kv_pool, dec_block_tables, dec_context_lens,
                             num_seqs, dec_max_blocks_per_seq, max_context_len, num_q_heads,
                             num_kv_heads, head_dim, block_size, dtype, workspace,
                             workspace_bytes))
      return s;
  }
  if (pre) {
    if (int s = check_prefill(pre_out, pre_q, kv_pool, pre_block_tables, pre_context_lens,
                              query_start_loc, num_chunks, total_q_tokens, max_chunk_len,
                              pre_max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim,
                              dtype))
      return s;
  }
  if (dec && pre) {  // neither output may overlap the other call's output or query
    const size_t e = elem_bytes(dtype);
    const size_t db = size_t(num_seqs) * num_q_heads * head_dim * e;
    const size_t pb = size_t(total_q_tokens) * num_q_heads * head_dim * e;
    if (overlaps(dec_out, db, pre_out, pb) || overlaps(dec_out, db, pre_q, pb) ||
        overlaps(pre_out, pb, dec_q, db))
      return PA_ERR_ALIAS;
  }
  if (!dec && !pre) return PA_OK;
  return status_of(pa::launch_mixed(
      dec_out, dec_q, kv_pool, dec_block_tables, dec_context_lens, num_seqs,
      dec_max_blocks_per_seq, max_context_len, pre_out, pre_q, pre_block_tables,
      pre_context_lens, query_start_loc, pre ? num_chunks : 0, total_q_tokens,
      pre ? max_chunk_len : 0, pre_max_blocks_per_seq, num_q_heads,
      shape(num_blocks, num_kv_heads, head_dim, block_size), scale, dtype, workspace,
      static_cast<hipStream_t>(stream)));
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case PA_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, group size or dtype";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_ALIAS: return "output overlaps an input";
    case PA_ERR_ALIGN: return "a data pointer is not 16-byte aligned";
    case PA_ERR_HOST: return "host pool is not pinned, device-mapped host memory";
    case PA_SCHED_FINISHED: return "every request has finished";
    case PA_ERR_STATE: return "scheduler invariant broken (a lone request does not fit, or no progress)";
    default: return "unknown status";
  }
}

}  // extern "C"
