// Internal launchers between the C-ABI layer (pkv_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Store: one thread per 16-byte chunk of a K or V row.
hipError_t launch_store(const uint16_t* key, int64_t key_stride, const uint16_t* value,
                        int64_t value_stride, uint16_t* k_cache, uint16_t* v_cache,
                        const int32_t* slot_mapping, int32_t num_tokens, int64_t num_slots,
                        int32_t row_elems, hipStream_t stream);

// Rows [from, to) of a bucketed decode step's metadata become padding:
// slot_mapping -1, context_lens 0.
hipError_t launch_pad_batch(int32_t* slot_mapping, int32_t* context_lens, int32_t from,
                            int32_t to, hipStream_t stream);

// Staged row writes: apply a packed buffer (rows[n], starts[n], off[n+1],
// values[total]) to a device int32 table.
hipError_t launch_apply_writes(int32_t* table, int64_t row_stride, int32_t num_rows,
                               int32_t num_cols, const int32_t* packed, int32_t n, int32_t total,
                               hipStream_t stream);

// Step metadata from device-resident request state, one launch; B <= kMetaMaxBatch.
constexpr int32_t kMetaMaxBatch = 4096;
hipError_t launch_metadata(int32_t B, const int32_t* idx_mapping, const int32_t* num_computed,
                           const int32_t* num_scheduled, const int32_t* block_table,
                           int32_t num_reqs, int64_t table_stride, int32_t block_size,
                           int32_t max_blocks_per_seq, int32_t max_tokens, int32_t* cu_seqlens_q,
                           int32_t* cu_seqlens_k, int32_t* context_lens, int64_t* positions,
                           int32_t* slot_mapping, int32_t* block_tables, int32_t* max_seqlens,
                           hipStream_t stream);

// Gumbel-max sampling: chunk scores into workspace (B x chunks of 8 bytes),
// then one wavefront per row picks the token.
int32_t sample_chunk_size(bool bf16);
hipError_t launch_sample(int64_t* tokens, const void* logits, bool bf16, int64_t row_stride,
                         int32_t B, int32_t V, const float* temps, const int64_t* seeds,
                         const int64_t* offsets, void* workspace, hipStream_t stream);

// The no-allocation sampling entry point's fixed scratch: this many 8-byte
// chunk keys (1 MiB) per device, in a file-scope device array of
// pkv_sample.hip.  sample_scratch_address gives the current device's copy
// (looked up once per device, under a lock).
constexpr int64_t kSampleScratchKeys = (int64_t)1 << 17;
hipError_t sample_scratch_address(void** address);

// The store fused into a decode call (all null otherwise): the new token of
// sequence b, at position context_lens[b] - 1, has its K/V rows at
// key + b * key_stride and value + b * value_stride ([H_kv, d] each).  The
// wavefront that computes the segment's last tile reads that row from there
// instead of the cache, and writes it into the cache (the row is in no other
// tile, and no other wavefront of the call reads it).
struct NewToken {
  const uint16_t* key;
  const uint16_t* value;
  int64_t key_stride;
  int64_t value_stride;
};

// Decode launch plan: one wavefront per resident slot of the current device.
struct DecodePlan {
  int32_t num_waves;       // 0 when the shape has no kernel
  size_t workspace_bytes;  // partial slots per share + one record per (sequence, KV head)
};
DecodePlan decode_plan(int32_t B, int32_t H_q, int32_t H_kv, int32_t d, int32_t block_size,
                       int32_t max_blocks_per_seq);

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int32_t B, int32_t H_q, int32_t H_kv,
                         int32_t d, int32_t num_blocks, int32_t block_size,
                         int32_t max_blocks_per_seq, float softmax_scale, void* workspace,
                         const DecodePlan& plan, const NewToken& new_token, hipStream_t stream);

// Query tiles of a prefill call (the grid's y extent, at most 65535).
int64_t prefill_query_tiles(int32_t max_seqlen_q, int32_t G);
constexpr int64_t kPrefillMaxQueryTiles = 65535;
// K/V rows of one 64-key tile are addressed with 32-bit byte offsets from the
// tile's first row, so a row stride (elements) may be at most 2^24.
constexpr int64_t kPrefillMaxRowStride = (int64_t)1 << 24;

hipError_t launch_prefill(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                          const uint16_t* v_cache, const int32_t* block_tables,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t B,
                          int32_t total_q, int32_t max_seqlen_q, int32_t H_q, int32_t H_kv,
                          int32_t d, int32_t num_blocks, int32_t block_size,
                          int32_t max_blocks_per_seq, float softmax_scale, hipStream_t stream);

// Varlen causal prefill over packed (non-paged) K/V rows; strides in elements.
hipError_t launch_prefill_packed(uint16_t* out, const uint16_t* q, int64_t q_stride,
                                 const uint16_t* k, int64_t k_stride, const uint16_t* v,
                                 int64_t v_stride, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int32_t B, int32_t total_q,
                                 int32_t total_k, int32_t max_seqlen_q, int32_t H_q, int32_t H_kv,
                                 int32_t d, float softmax_scale, hipStream_t stream);

}  // namespace pkv
