// store_kvcache: scatter the new tokens' K/V rows into the paged cache through
// slot_mapping (devpress "nano-vllm解读", KV-cache write; AIInfraGuide 3.6,
// section 2: slot -1 writes nothing).
//
// Pure data movement, HBM-bound: each thread moves one 16-byte chunk of one K
// or V row with a single 128-bit load and store.  Consecutive threads cover
// consecutive chunks of a row, so every wavefront reads and writes whole
// contiguous 1 KiB spans of a row (a 2 KiB row for H_kv*d = 1024 is two waves).
//
// Also here: the padding kernel of a bucketed (graph-captured) decode step,
// which marks the rows between the batch and its bucket as padding.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

__global__ __launch_bounds__(256) void store_kernel(
    const uint16_t* __restrict__ key, int64_t key_stride, const uint16_t* __restrict__ value,
    int64_t value_stride, uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, int32_t num_tokens, int64_t num_slots,
    int32_t chunks_per_row, int64_t total_chunks, int32_t row_elems) {
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= total_chunks) return;
  const int32_t per_token = 2 * chunks_per_row;
  const int32_t tok = (int32_t)(item / per_token);
  const int32_t rem = (int32_t)(item - (int64_t)tok * per_token);
  const bool is_v = rem >= chunks_per_row;
  const int32_t chunk = is_v ? rem - chunks_per_row : rem;
  const int32_t slot = slot_mapping[tok];
  if (slot < 0 || (int64_t)slot >= num_slots) return;  // -1 = padding; others out of range
  const uint16_t* src = (is_v ? value + (int64_t)tok * value_stride : key + (int64_t)tok * key_stride);
  uint16_t* dst = (is_v ? v_cache : k_cache) + (int64_t)slot * row_elems;
  st16(dst + chunk * 8, ld16(src + chunk * 8));
}

hipError_t launch_store(const uint16_t* key, int64_t key_stride, const uint16_t* value,
                        int64_t value_stride, uint16_t* k_cache, uint16_t* v_cache,
                        const int32_t* slot_mapping, int32_t num_tokens, int64_t num_slots,
                        int32_t row_elems, hipStream_t stream) {
  const int32_t chunks = row_elems / 8;
  const int64_t total = (int64_t)num_tokens * 2 * chunks;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(store_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, key, key_stride,
                     value, value_stride, k_cache, v_cache, slot_mapping, num_tokens, num_slots,
                     chunks, total, row_elems);
  return hipGetLastError();
}

// Padding rows of a bucketed decode step: slot -1 (the store skips the row)
// and context length 0 (the decode writes a zero row).
__global__ __launch_bounds__(256) void pad_batch_kernel(int32_t* __restrict__ slot_mapping,
                                                        int32_t* __restrict__ context_lens,
                                                        int32_t from, int32_t to) {
  const int32_t i = from + (int32_t)(blockIdx.x * 256 + threadIdx.x);
  if (i >= to) return;
  slot_mapping[i] = -1;
  context_lens[i] = 0;
}

hipError_t launch_pad_batch(int32_t* slot_mapping, int32_t* context_lens, int32_t from,
                            int32_t to, hipStream_t stream) {
  if (to <= from) return hipSuccess;
  const unsigned blocks = (unsigned)((to - from + 255) / 256);
  hipLaunchKernelGGL(pad_batch_kernel, dim3(blocks), dim3(256), 0, stream, slot_mapping,
                     context_lens, from, to);
  return hipGetLastError();
}

}  // namespace pkv
