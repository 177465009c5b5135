// Internal interface between the host API (pa_api.cpp) and the device code
// (pa_kernels.hip). Arguments are validated by the caller; these functions only
// size grids and launch on `stream`. Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Split-K partition (tokens). The public header's macro is the one definition:
// the workspace size, the grid and every kernel use this constant.
constexpr int kPartition = PA_DECODE_PARTITION;
constexpr int kWaves = 4;         // waves per workgroup in the attention kernels
constexpr int kStep = 32;         // tokens per wave step

struct PoolShape {
  int64_t num_blocks;
  int num_kv_heads;
  int head_dim;
  int block_size;
  int64_t block_elems() const { return 2LL * num_kv_heads * block_size * head_dim; }
};

// Workspace carve-up for pa_decode (256-byte aligned): the work-queue counters
// at offset 0 (a place that does not depend on the batch shape), then per
// (sequence, query head, partition) the partition's unnormalised output O[d]
// and its (M, L). The counters must be zero before the first call; every call
// returns them to zero. Partial results need no initialisation.
struct DecodeWorkspace {
  size_t queue_off, o_off, ml_off, total;
  // o_elem_bytes: bytes per partial-output element. pa_decode sizes its
  // caller's workspace for float (4) whatever the call's type; the
  // allocation-free entry point packs a bf16 call's partials at 2 bytes each.
  static DecodeWorkspace layout(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim,
                                int64_t max_parts, size_t o_elem_bytes = sizeof(float)) {
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    DecodeWorkspace w;
    w.queue_off = 0;
    w.o_off = 256;
    // partial outputs are float or bf16 (the call's type)
    size_t o_bytes = size_t(num_seqs) * num_q_heads * max_parts * head_dim * o_elem_bytes;
    w.ml_off = w.o_off + up(o_bytes);
    size_t ml_bytes = size_t(num_seqs) * num_q_heads * max_parts * 2 * sizeof(float);
    w.total = w.ml_off + up(ml_bytes);
    return w;
  }
};

inline int64_t decode_max_parts(int64_t max_context_len) {
  int64_t p = (max_context_len + kPartition - 1) / kPartition;
  return p < 1 ? 1 : p;
}

hipError_t launch_append(void* pool, const void* k_new, const void* v_new, const int32_t* slots,
                         int num_tokens, const PoolShape& ps, int dtype, hipStream_t stream);

hipError_t launch_copy(void* pool, const int32_t* pairs, int num_pairs, const PoolShape& ps,
                       int dtype, hipStream_t stream);

// Whole blocks between the device pool and a device-mapped host pool: out
// copies pool[pair.src] to host[pair.dst], in copies host[pair.src] to
// pool[pair.dst].
hipError_t launch_swap(void* pool, void* host_dev, const int32_t* pairs, int num_pairs, bool out,
                       int64_t num_host_blocks, const PoolShape& ps, int dtype,
                       hipStream_t stream);

// share: nullptr, or the caller's sharing hint of pa_decode_shared (device
// int32 per sequence).
hipError_t launch_decode(void* out, const void* q, const void* pool, const int32_t* tables,
                         const int32_t* lens, int num_seqs, int max_blocks_per_seq,
                         int max_context_len, int num_q_heads, const PoolShape& ps, float scale,
                         int dtype, void* workspace, hipStream_t stream,
                         const int32_t* share = nullptr);

// pa_decode_append: the decode step's append and its decode. bfloat16 batches
// of up to kMaxScanSeqs sequences run in one launch; other calls launch the
// append, then the decode.
hipError_t launch_decode_append(void* out, const void* q, void* pool, const int32_t* tables,
                                const int32_t* lens, const void* k_new, const void* v_new,
                                const int32_t* slots, int num_seqs, int max_blocks_per_seq,
                                int max_context_len, int num_q_heads, const PoolShape& ps,
                                float scale, int dtype, void* workspace, hipStream_t stream);

// pa_decode with the library's own scratch array as the workspace (no
// allocation). The caller has checked that the packed layout (partials in the
// call's type) fits kDecodeScratchBytes.
constexpr size_t kDecodeScratchBytes = PA_DECODE_SCRATCH_BYTES;
hipError_t launch_decode_noalloc(void* out, const void* q, const void* pool, const int32_t* tables,
                                 const int32_t* lens, int num_seqs, int max_blocks_per_seq,
                                 int max_context_len, int num_q_heads, const PoolShape& ps,
                                 float scale, int dtype, hipStream_t stream);

hipError_t launch_prefill(void* out, const void* q, const void* pool, const int32_t* tables,
                          const int32_t* lens, const int32_t* qsl, int num_chunks,
                          int total_q_tokens, int max_chunk_len, int max_blocks_per_seq, int num_q_heads,
                          const PoolShape& ps, float scale, int dtype, hipStream_t stream);

// Decode batch and prefill chunks in one persistent launch (bf16, batches the
// fused kernel takes), else the two launches in turn.
hipError_t launch_mixed(void* dec_out, const void* dec_q, const void* pool,
                        const int32_t* dec_tables, const int32_t* dec_lens, int num_seqs,
                        int dec_max_blocks, int max_context_len, void* pre_out,
                        const void* pre_q, const int32_t* pre_tables, const int32_t* pre_lens,
                        const int32_t* qsl, int num_chunks, int total_q_tokens, int max_chunk_len,
                        int pre_max_blocks, int num_q_heads, const PoolShape& ps, float scale,
                        int dtype, void* workspace, hipStream_t stream);

}  // namespace pa
