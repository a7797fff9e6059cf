// store_kvcache: scatter the new tokens' K/V rows into the paged cache through
// slot_mapping (devpress "nano-vllm解读", KV-cache write; AIInfraGuide 3.6,
// section 2: slot -1 writes nothing).
//
// Pure data movement, HBM-bound: each thread moves one 16-byte chunk of one K
// or V row with a single 128-bit load and store.  A workgroup covers one
// token's K and V rows (more groups when they exceed 256 chunks); consecutive
// threads take consecutive chunks, so every wavefront reads and writes whole
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
    const int32_t* __restrict__ slot_mapping, int64_t num_slots, int32_t chunks_per_row,
    int32_t row_elems) {
  // grid (token, chunk group): no division to find either; rows of more than
  // 65535 groups of 256 chunks loop over the groups
  const int32_t tok = (int32_t)blockIdx.x;
  for (int64_t rem = (int64_t)blockIdx.y * 256 + threadIdx.x; rem < 2 * (int64_t)chunks_per_row;
       rem += (int64_t)gridDim.y * 256) {
    const bool is_v = rem >= chunks_per_row;
    const int64_t chunk = is_v ? rem - chunks_per_row : rem;
    // the source row exists for every token, so its load goes out together
    // with the slot's instead of waiting for the slot check (the empty asm
    // keeps the compiler from sinking it below the check)
    const uint16_t* src =
        (is_v ? value + (int64_t)tok * value_stride : key + (int64_t)tok * key_stride);
    int32_t slot = slot_mapping[tok];
    u32x4 row = ld16(src + chunk * 8);
    asm volatile("" : "+v"(row), "+v"(slot));
    if (slot < 0 || (int64_t)slot >= num_slots) return;  // -1 = padding; others out of range
    uint16_t* dst = (is_v ? v_cache : k_cache) + (int64_t)slot * row_elems;
    st16(dst + chunk * 8, row);
  }
}

hipError_t launch_store(const uint16_t* key, int64_t key_stride, const uint16_t* value,
                        int64_t value_stride, uint16_t* k_cache, uint16_t* v_cache,
                        const int32_t* slot_mapping, int32_t num_tokens, int64_t num_slots,
                        int32_t row_elems, hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  const int32_t chunks = row_elems / 8;
  const int64_t g = (2 * (int64_t)chunks + 255) / 256;
  const unsigned groups = (unsigned)(g < 65535 ? g : 65535);
  hipLaunchKernelGGL(store_kernel, dim3((unsigned)num_tokens, groups), dim3(256), 0, stream, key,
                     key_stride, value, value_stride, k_cache, v_cache, slot_mapping, num_slots,
                     chunks, row_elems);
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
