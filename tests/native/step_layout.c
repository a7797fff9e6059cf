/* Prints the size and field offsets of pkv_decode_step as the C compiler
 * lays it out, for comparison with the Python binding's ctypes mirror. */
#include <stddef.h>
#include <stdio.h>

#include "pkv.h"

#define FIELD(f) printf(#f " %zu\n", offsetof(pkv_decode_step, f))

int main(void) {
  printf("size %zu\n", sizeof(pkv_decode_step));
  FIELD(layers); FIELD(max_batch); FIELD(H_q); FIELD(H_kv); FIELD(d);
  FIELD(num_blocks); FIELD(block_size); FIELD(max_blocks_per_seq); FIELD(softmax_scale);
  FIELD(slot_mapping); FIELD(context_lens); FIELD(block_tables);
  FIELD(q); FIELD(key); FIELD(value); FIELD(key_stride); FIELD(value_stride);
  FIELD(k_cache); FIELD(v_cache); FIELD(out); FIELD(workspace); FIELD(workspace_bytes);
  return 0;
}
