// C ABI of libpkv: argument checks on the host, then kernel launches.
// Declarations and the full contract are in include/pkv.h.
#include "pkv.h"

#include <limits.h>
#include <math.h>

#include <algorithm>
#include <vector>

#include "pkv_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2_ge16(int32_t x) { return x >= 16 && (x & (x - 1)) == 0; }

bool supported_d(int32_t d) { return d == 64 || d == 128; }

bool supported_group(int32_t H_q, int32_t H_kv) {
  const int32_t g = H_q / H_kv;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

// The decode schedule counts (sequence, KV head, 16-token tile) units in
// int32: the most a table of this width can describe must fit.
bool decode_units_fit(int32_t B, int32_t H_kv, int32_t block_size, int32_t max_blocks_per_seq) {
  const int64_t tiles = ((int64_t)max_blocks_per_seq * block_size + 15) / 16;
  return (int64_t)B * H_kv * tiles <= INT32_MAX;
}

// The prefill kernels take the running maximum of the raw scores and scale
// it afterwards, which is only the maximum of the scaled scores for a
// positive scale.
bool positive_finite(float x) { return isfinite(x) && x > 0.0f; }

pkv_status launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ELAUNCH; }

// Checks shared by the two attention calls.
pkv_status check_attention(const void* out, const void* q, const void* k_cache,
                           const void* v_cache, const void* block_tables, int32_t H_q,
                           int32_t H_kv, int32_t d, int32_t num_blocks, int32_t block_size,
                           int32_t max_blocks_per_seq) {
  if (!out || !q || !k_cache || !v_cache || !block_tables) return PKV_EINVAL;
  if (H_q <= 0 || H_kv <= 0 || d <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return PKV_EINVAL;
  if (H_q % H_kv != 0 || !pow2_ge16(block_size)) return PKV_EINVAL;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PKV_EINVAL;
  if ((int64_t)num_blocks * block_size > INT32_MAX) return PKV_EINVAL;  // slots are int32
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_EINVAL;
  if (!supported_d(d) || !supported_group(H_q, H_kv)) return PKV_EUNSUPPORTED;
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_EINVAL: return "PKV_EINVAL: invalid argument";
    case PKV_EUNSUPPORTED: return "PKV_EUNSUPPORTED: unsupported head size or group size";
    case PKV_ELAUNCH: return "PKV_ELAUNCH: kernel launch failed";
    case PKV_ESCRATCH:
      return "PKV_ESCRATCH: the call needs more scratch than the fixed array of the "
             "no-allocation entry point holds";
    default: return "unknown pkv status";
  }
}

int pkv_version(void) { return 100; }

pkv_status pkv_prepare_metadata(int32_t B, const int32_t* num_cached, const int32_t* num_new,
                                const int32_t* block_offsets, const int32_t* block_ids,
                                int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t* slot_mapping, int32_t* context_lens,
                                int32_t* cu_seqlens_q, int32_t* cu_seqlens_k,
                                int32_t* block_tables, int32_t* max_seqlen_q,
                                int32_t* max_seqlen_k) {
  if (B < 0 || !pow2_ge16(block_size) || max_blocks_per_seq < 0) return PKV_EINVAL;
  if (!cu_seqlens_q || !cu_seqlens_k || !max_seqlen_q || !max_seqlen_k) return PKV_EINVAL;
  if (B > 0 && (!num_cached || !num_new || !block_offsets || !context_lens ||
                (max_blocks_per_seq > 0 && !block_tables)))
    return PKV_EINVAL;
  int shift = 0;
  while ((1 << shift) < block_size) ++shift;
  const int32_t mask = block_size - 1;
  int64_t cq = 0, ck = 0;
  int32_t mq = 0, mk = 0;
  cu_seqlens_q[0] = 0;
  cu_seqlens_k[0] = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t c = num_cached[b], n = num_new[b];
    if (c < 0 || n < 0 || c + n > INT32_MAX) return PKV_EINVAL;
    const int64_t lo = block_offsets[b], hi = block_offsets[b + 1];
    const int64_t owned = hi - lo;
    const int64_t needed = (c + n + block_size - 1) >> shift;
    if (lo < 0 || owned < needed || owned > max_blocks_per_seq) return PKV_EINVAL;
    if (owned > 0 && !block_ids) return PKV_EINVAL;
    int32_t* row = block_tables + (int64_t)b * max_blocks_per_seq;
    for (int64_t j = 0; j < max_blocks_per_seq; ++j) {
      int32_t id = -1;
      if (j < owned) {
        id = block_ids[lo + j];
        if (id < 0 || (int64_t)id * block_size + mask > INT32_MAX) return PKV_EINVAL;
      }
      row[j] = id;
    }
    if (n > 0 && !slot_mapping) return PKV_EINVAL;
    for (int64_t p = c; p < c + n; ++p)  // position p of the sequence
      slot_mapping[cq + (p - c)] = row[p >> shift] * block_size + (int32_t)(p & mask);
    cq += n;
    ck += c + n;
    if (cq > INT32_MAX || ck > INT32_MAX) return PKV_EINVAL;
    cu_seqlens_q[b + 1] = (int32_t)cq;
    cu_seqlens_k[b + 1] = (int32_t)ck;
    context_lens[b] = (int32_t)(c + n);
    if (n > mq) mq = (int32_t)n;
    if (c + n > mk) mk = (int32_t)(c + n);
  }
  *max_seqlen_q = mq;
  *max_seqlen_k = mk;
  return PKV_OK;
}

pkv_status pkv_store(const void* key, int64_t key_stride, const void* value,
                     int64_t value_stride, void* k_cache, void* v_cache,
                     const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                     int32_t block_size, int32_t H_kv, int32_t d, hipStream_t stream) {
  if (num_tokens < 0 || num_blocks <= 0 || H_kv <= 0 || d <= 0 || !pow2_ge16(block_size))
    return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PKV_EINVAL;
  const int64_t row = (int64_t)H_kv * d;
  if (row % 8 != 0 || row > INT32_MAX / 2) return PKV_EINVAL;
  if (key_stride < row || value_stride < row || key_stride % 8 || value_stride % 8)
    return PKV_EINVAL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_EINVAL;
  const int64_t slots = (int64_t)num_blocks * block_size;
  if (slots > INT64_MAX / row) return PKV_EINVAL;
  return launch_status(pkv::launch_store(
      static_cast<const uint16_t*>(key), key_stride, static_cast<const uint16_t*>(value),
      value_stride, static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
      slot_mapping, num_tokens, slots, (int32_t)row, stream));
}

size_t pkv_decode_workspace_size(int32_t B, int32_t H_q, int32_t H_kv, int32_t d,
                                 int32_t block_size, int32_t max_blocks_per_seq) {
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || d <= 0 || max_blocks_per_seq <= 0 ||
      !pow2_ge16(block_size) || H_q % H_kv != 0)
    return 0;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return 0;
  if (!decode_units_fit(B, H_kv, block_size, max_blocks_per_seq)) return 0;
  return pkv::decode_plan(B, H_q, H_kv, d, block_size, max_blocks_per_seq).workspace_bytes;
}

pkv_status pkv_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                      int32_t H_q, int32_t H_kv, int32_t d, int32_t num_blocks,
                      int32_t block_size, int32_t max_blocks_per_seq, float softmax_scale,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B <= 0 || !context_lens || !isfinite(softmax_scale)) return PKV_EINVAL;
  pkv_status st = check_attention(out, q, k_cache, v_cache, block_tables, H_q, H_kv, d,
                                  num_blocks, block_size, max_blocks_per_seq);
  if (st != PKV_OK) return st;
  if ((int64_t)B * H_kv > INT32_MAX) return PKV_EINVAL;
  if (!decode_units_fit(B, H_kv, block_size, max_blocks_per_seq)) return PKV_EUNSUPPORTED;
  const pkv::DecodePlan plan = pkv::decode_plan(B, H_q, H_kv, d, block_size, max_blocks_per_seq);
  if (plan.num_waves <= 0) return PKV_EUNSUPPORTED;
  if (!workspace || workspace_bytes < plan.workspace_bytes || !aligned16(workspace))
    return PKV_EINVAL;
  return launch_status(pkv::launch_decode(
      static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
      static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), block_tables,
      context_lens, B, H_q, H_kv, d, num_blocks, block_size, max_blocks_per_seq, softmax_scale,
      workspace, plan, pkv::NewToken{}, stream));
}

pkv_status pkv_store_decode(void* out, const void* q, const void* key, int64_t key_stride,
                            const void* value, int64_t value_stride, void* k_cache,
                            void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t B, int32_t H_q, int32_t H_kv,
                            int32_t d, int32_t num_blocks, int32_t block_size,
                            int32_t max_blocks_per_seq, float softmax_scale, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (B <= 0 || !context_lens || !isfinite(softmax_scale)) return PKV_EINVAL;
  if (!key || !value) return PKV_EINVAL;
  pkv_status st = check_attention(out, q, k_cache, v_cache, block_tables, H_q, H_kv, d,
                                  num_blocks, block_size, max_blocks_per_seq);
  if (st != PKV_OK) return st;
  const int64_t row = (int64_t)H_kv * d;
  if (key_stride < row || value_stride < row || key_stride % 8 || value_stride % 8)
    return PKV_EINVAL;
  if (!aligned16(key) || !aligned16(value)) return PKV_EINVAL;
  if ((int64_t)B * H_kv > INT32_MAX) return PKV_EINVAL;
  if (!decode_units_fit(B, H_kv, block_size, max_blocks_per_seq)) return PKV_EUNSUPPORTED;
  const pkv::DecodePlan plan = pkv::decode_plan(B, H_q, H_kv, d, block_size, max_blocks_per_seq);
  if (plan.num_waves <= 0) return PKV_EUNSUPPORTED;
  if (!workspace || workspace_bytes < plan.workspace_bytes || !aligned16(workspace))
    return PKV_EINVAL;
  const pkv::NewToken nt{static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
                         key_stride, value_stride};
  return launch_status(pkv::launch_decode(
      static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
      static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), block_tables,
      context_lens, B, H_q, H_kv, d, num_blocks, block_size, max_blocks_per_seq, softmax_scale,
      workspace, plan, nt, stream));
}

pkv_status pkv_prefill_varlen(void* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t B, int32_t total_q, int32_t max_seqlen_q,
                              int32_t max_seqlen_k, int32_t H_q, int32_t H_kv, int32_t d,
                              int32_t num_blocks, int32_t block_size,
                              int32_t max_blocks_per_seq, float softmax_scale,
                              hipStream_t stream) {
  (void)max_seqlen_k;
  if (B < 0 || total_q < 0 || max_seqlen_q < 0) return PKV_EINVAL;
  if (B == 0 || max_seqlen_q == 0 || total_q == 0) return PKV_OK;
  if (!cu_seqlens_q || !cu_seqlens_k || !positive_finite(softmax_scale)) return PKV_EINVAL;
  pkv_status st = check_attention(out, q, k_cache, v_cache, block_tables, H_q, H_kv, d,
                                  num_blocks, block_size, max_blocks_per_seq);
  if (st != PKV_OK) return st;
  if (B > 65535) return PKV_EINVAL;
  if (pkv::prefill_query_tiles(max_seqlen_q, H_q / H_kv) > pkv::kPrefillMaxQueryTiles)
    return PKV_EUNSUPPORTED;
  if ((int64_t)H_kv * d > pkv::kPrefillMaxRowStride) return PKV_EUNSUPPORTED;
  return launch_status(pkv::launch_prefill(
      static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
      static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), block_tables,
      cu_seqlens_q, cu_seqlens_k, B, total_q, max_seqlen_q, H_q, H_kv, d, num_blocks, block_size,
      max_blocks_per_seq, softmax_scale, stream));
}

pkv_status pkv_prefill_varlen_packed(void* out, const void* q, int64_t q_stride, const void* k,
                                     int64_t k_stride, const void* v, int64_t v_stride,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     int32_t B, int32_t total_q, int32_t total_k,
                                     int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t H_q,
                                     int32_t H_kv, int32_t d, float softmax_scale,
                                     hipStream_t stream) {
  (void)max_seqlen_k;
  if (B < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0) return PKV_EINVAL;
  if (B == 0 || max_seqlen_q == 0 || total_q == 0) return PKV_OK;
  if (!out || !q || !k || !v || !cu_seqlens_q || !cu_seqlens_k) return PKV_EINVAL;
  if (!positive_finite(softmax_scale)) return PKV_EINVAL;
  if (H_q <= 0 || H_kv <= 0 || d <= 0 || H_q % H_kv != 0 || total_k <= 0) return PKV_EINVAL;
  if (B > 65535) return PKV_EINVAL;
  const int64_t qrow = (int64_t)H_q * d, kvrow = (int64_t)H_kv * d;
  if (q_stride < qrow || k_stride < kvrow || v_stride < kvrow) return PKV_EINVAL;
  if (q_stride % 8 || k_stride % 8 || v_stride % 8) return PKV_EINVAL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k) || !aligned16(v)) return PKV_EINVAL;
  if (!supported_d(d) || !supported_group(H_q, H_kv)) return PKV_EUNSUPPORTED;
  if (pkv::prefill_query_tiles(max_seqlen_q, H_q / H_kv) > pkv::kPrefillMaxQueryTiles)
    return PKV_EUNSUPPORTED;
  if (k_stride > pkv::kPrefillMaxRowStride || v_stride > pkv::kPrefillMaxRowStride)
    return PKV_EUNSUPPORTED;
  return launch_status(pkv::launch_prefill_packed(
      static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q), q_stride,
      static_cast<const uint16_t*>(k), k_stride, static_cast<const uint16_t*>(v), v_stride,
      cu_seqlens_q, cu_seqlens_k, B, total_q, total_k, max_seqlen_q, H_q, H_kv, d, softmax_scale,
      stream));
}

pkv_status pkv_pack_row_writes(int32_t n, const int32_t* rows, const int32_t* starts,
                               const int32_t* lens, const int32_t* values, int32_t num_rows,
                               int32_t num_cols, int32_t* packed, int64_t packed_capacity,
                               int64_t* packed_size) {
  if (n < 0 || !packed_size || num_rows < 0 || num_cols < 0) return PKV_EINVAL;
  if (n > 0 && (!rows || !starts || !lens)) return PKV_EINVAL;
  int64_t total = 0;
  for (int32_t w = 0; w < n; ++w) {
    if (lens[w] < 0 || rows[w] < 0 || rows[w] >= num_rows || starts[w] < 0) return PKV_EINVAL;
    if ((int64_t)starts[w] + lens[w] > num_cols) return PKV_EINVAL;
    total += lens[w];
  }
  if (total > INT32_MAX || (total > 0 && !values)) return PKV_EINVAL;
  // no element may be written twice: sort the non-empty writes by (row, start)
  std::vector<int32_t> order;
  order.reserve((size_t)n);
  for (int32_t w = 0; w < n; ++w)
    if (lens[w] > 0) order.push_back(w);
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return rows[a] != rows[b] ? rows[a] < rows[b] : starts[a] < starts[b];
  });
  for (size_t i = 1; i < order.size(); ++i) {
    const int32_t a = order[i - 1], b = order[i];
    if (rows[a] == rows[b] && (int64_t)starts[a] + lens[a] > starts[b]) return PKV_EINVAL;
  }
  const int64_t size = 3 * (int64_t)n + 1 + total;
  *packed_size = size;
  if (!packed || packed_capacity < size) return PKV_EINVAL;
  int32_t* off = packed + 2 * (int64_t)n;
  int32_t* vals = off + n + 1;
  off[0] = 0;
  for (int32_t w = 0; w < n; ++w) {
    packed[w] = rows[w];
    packed[n + w] = starts[w];
    off[w + 1] = off[w] + lens[w];
  }
  for (int64_t i = 0; i < total; ++i) vals[i] = values[i];
  return PKV_OK;
}

pkv_status pkv_apply_row_writes(int32_t* table, int64_t row_stride, int32_t num_rows,
                                int32_t num_cols, const int32_t* packed, int32_t n,
                                int32_t total, hipStream_t stream) {
  if (n < 0 || total < 0 || num_rows < 1 || num_cols < 1 || row_stride < num_cols)
    return PKV_EINVAL;
  if (n == 0 || total == 0) return PKV_OK;
  if (!table || !packed) return PKV_EINVAL;
  return launch_status(
      pkv::launch_apply_writes(table, row_stride, num_rows, num_cols, packed, n, total, stream));
}

pkv_status pkv_prepare_metadata_device(int32_t B, const int32_t* idx_mapping,
                                       const int32_t* num_computed, const int32_t* num_scheduled,
                                       const int32_t* block_table, int32_t num_reqs,
                                       int64_t table_stride, int32_t block_size,
                                       int32_t max_blocks_per_seq, int32_t max_tokens,
                                       int32_t* cu_seqlens_q, int32_t* cu_seqlens_k,
                                       int32_t* context_lens, int64_t* positions,
                                       int32_t* slot_mapping, int32_t* block_tables,
                                       int32_t* max_seqlens, hipStream_t stream) {
  if (B < 0 || max_tokens < 0 || !pow2_ge16(block_size) || max_blocks_per_seq < 1 ||
      table_stride < max_blocks_per_seq || num_reqs < 1)
    return PKV_EINVAL;
  if (!cu_seqlens_q || !cu_seqlens_k) return PKV_EINVAL;
  if (B > 0 && (!num_computed || !num_scheduled || !block_table || !context_lens ||
                (max_tokens > 0 && !slot_mapping)))
    return PKV_EINVAL;
  if (B > pkv::kMetaMaxBatch) return PKV_EUNSUPPORTED;
  return launch_status(pkv::launch_metadata(
      B, idx_mapping, num_computed, num_scheduled, block_table, num_reqs, table_stride,
      block_size, max_blocks_per_seq, max_tokens, cu_seqlens_q, cu_seqlens_k, context_lens,
      positions, slot_mapping, block_tables, max_seqlens, stream));
}

size_t pkv_sample_workspace_size(int32_t B, int32_t V) {
  if (B < 1 || V < 1) return 0;
  const int64_t chunk = pkv::sample_chunk_size(false);  // the smaller chunk: the most chunks
  return (size_t)B * (size_t)((V + chunk - 1) / chunk) * sizeof(uint64_t);
}

pkv_status pkv_sample_gumbel(int64_t* tokens, const void* logits, int32_t logits_bf16,
                             int64_t row_stride, int32_t B, int32_t V,
                             const float* temperatures, const int64_t* seeds,
                             const int64_t* offsets, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  if (B < 0 || V < 1 || row_stride < V) return PKV_EINVAL;
  if (row_stride % (logits_bf16 ? 8 : 4) != 0) return PKV_EINVAL;
  if (B == 0) return PKV_OK;
  if (!tokens || !logits || !seeds || !workspace || !aligned16(logits)) return PKV_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 8 != 0) return PKV_EINVAL;  // 64-bit chunk keys
  if (B > 65535) return PKV_EINVAL;  // one grid row per batch row
  if (workspace_bytes < pkv_sample_workspace_size(B, V)) return PKV_EINVAL;
  return launch_status(pkv::launch_sample(tokens, logits, logits_bf16 != 0, row_stride, B, V,
                                          temperatures, seeds, offsets, workspace, stream));
}

pkv_status pkv_sample_gumbel_noalloc(int64_t* tokens, const void* logits, int32_t logits_bf16,
                                     int64_t row_stride, int32_t B, int32_t V,
                                     const float* temperatures, const int64_t* seeds,
                                     const int64_t* offsets, hipStream_t stream) {
  if (B < 0 || V < 1 || row_stride < V) return PKV_EINVAL;
  if (row_stride % (logits_bf16 ? 8 : 4) != 0) return PKV_EINVAL;
  if (B == 0) return PKV_OK;
  if (!tokens || !logits || !seeds || !aligned16(logits)) return PKV_EINVAL;
  if (B > 65535) return PKV_EINVAL;  // one grid row per batch row
  const int64_t chunk = pkv::sample_chunk_size(logits_bf16 != 0);
  if ((int64_t)B * ((V + chunk - 1) / chunk) > pkv::kSampleScratchKeys) return PKV_ESCRATCH;
  void* scratch = nullptr;
  if (pkv::sample_scratch_address(&scratch) != hipSuccess) return PKV_ELAUNCH;
  return launch_status(pkv::launch_sample(tokens, logits, logits_bf16 != 0, row_stride, B, V,
                                          temperatures, seeds, offsets, scratch, stream));
}

}  // extern "C"
