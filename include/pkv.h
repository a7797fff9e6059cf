/*
 * pkv.h -- C ABI of libpkv: attention over a block-paged KV cache on AMD
 * MI355X (gfx950).
 *
 * The calls follow the problem as the source pages state it:
 *  - devpress.csdn.net "nano-vllm解读", section "PagedAttention是如何实现的":
 *    the decode call's arguments (q as [reqs, H, d]; k_cache/v_cache as
 *    [max_blocks, block_size, H_kv, d]; int32 cache lengths; an int32
 *    [reqs, max_len_blocks] block table right-padded with -1;
 *    softmax_scale = 1/sqrt(d)), and the store kernel that writes each new
 *    token's K/V at the row slot_mapping[i] of the cache viewed as
 *    [num_blocks * block_size, H_kv * d];
 *  - the same page, section "如何适配不同请求不同序列长度": varlen causal
 *    prefill with queries stacked along the token axis and addressed by
 *    cumulative lengths cu_seqlens_q / cu_seqlens_k (+ max_seqlen_q/k);
 *  - caomaolufei.github.io AIInfraGuide 3.6, section 2 ("prepare_prefill /
 *    prepare_decode"): how slot_mapping, context_lens (the stored token
 *    included), cu_seqlens and the -1-padded block tables are built, and
 *    that a slot of -1 writes nothing; section 4: one pool
 *    [2, layers, num_blocks, block_size, H_kv, d] whose per-layer slices are
 *    the k_cache/v_cache arguments.
 *
 * Conventions shared by every call:
 *  - bf16 tensors are passed as device pointers to raw 16-bit bfloat16 data,
 *    16-byte aligned, in the row-major layouts stated per call.
 *  - Grouped-query attention: query head h reads KV head h / (H_q / H_kv)
 *    (contiguous groups).  The pages give K/V H_kv heads but do not state the
 *    grouping; this is the reading used on both sides of every parity test.
 *  - The caller owns all memory.  The library never allocates, frees or
 *    synchronises: every device call only enqueues work on `stream` and
 *    returns.  Calls on one stream run in order, so a store followed by an
 *    attention call on the same stream sees the stored rows.
 *  - Errors are reported by the return code only.  Scalar arguments are
 *    checked on the host before anything is enqueued.  Device-resident
 *    metadata (slots, block ids, lengths, cu_seqlens) cannot be checked
 *    without a synchronisation; the kernels clamp or skip out-of-range values
 *    so that no access leaves the caller's buffers, but the results of such
 *    calls are unspecified.  Preconditions: every block id a read key maps to
 *    lies in [0, num_blocks); non-(-1) slots lie in [0, num_blocks*block_size)
 *    and are unique; context_lens[b] <= max_blocks_per_seq * block_size;
 *    cu_seqlens are non-decreasing with 0 <= nq <= nk per sequence.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_EINVAL = 1,       /* an argument violates a documented constraint */
  PKV_EUNSUPPORTED = 2, /* valid, but not a shape the library has kernels for */
  PKV_ELAUNCH = 3,      /* the HIP runtime reported an error at launch */
  PKV_ESCRATCH = 4      /* more scratch than pkv_sample_gumbel_noalloc's fixed array holds */
} pkv_status;

/* Static, human-readable name of a status code. */
const char* pkv_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int pkv_version(void);

/*
 * Host metadata for one attention step (AIInfraGuide 3.6, section 2).
 *
 * Input, per sequence b (host memory):
 *   num_cached[b]   tokens already in the cache (c)
 *   num_new[b]      tokens this step stores and queries (n; 1 for decode)
 *   block_offsets   [B+1] CSR offsets into block_ids
 *   block_ids       physical block ids of sequence b in logical order at
 *                   block_ids[block_offsets[b] .. block_offsets[b+1])
 * Output (host memory, caller-allocated):
 *   slot_mapping    [sum n]  slot of new token i of sequence b: position
 *                   p = c + i, slot = block_ids_b[p / block_size] * block_size
 *                   + p % block_size
 *   context_lens    [B]      c + n
 *   cu_seqlens_q    [B+1]    prefix sums of n
 *   cu_seqlens_k    [B+1]    prefix sums of c + n
 *   block_tables    [B, max_blocks_per_seq]  ids, right-padded with -1
 *   max_seqlen_q, max_seqlen_k   maxima of n and c + n (0 when B == 0)
 * PKV_EINVAL: B < 0; a null pointer (with B > 0); block_size not a power of
 * two >= 16; c or n negative; fewer blocks than ceil((c+n)/block_size) or
 * more than max_blocks_per_seq; a negative block id; int32 overflow of a sum.
 * Outputs are unspecified after an error.
 */
pkv_status pkv_prepare_metadata(int32_t B, const int32_t* num_cached, const int32_t* num_new,
                                const int32_t* block_offsets, const int32_t* block_ids,
                                int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t* slot_mapping, int32_t* context_lens,
                                int32_t* cu_seqlens_q, int32_t* cu_seqlens_k,
                                int32_t* block_tables, int32_t* max_seqlen_q,
                                int32_t* max_seqlen_k);

/*
 * Store (devpress page, KV-cache write): for i in [0, num_tokens) with
 * slot_mapping[i] != -1, copy the H_kv*d bf16 values of key[i] and value[i]
 * bit for bit to row slot_mapping[i] of k_cache and v_cache.
 *   key, value   device, [num_tokens, H_kv, d] bf16; head and d contiguous,
 *                token stride key_stride / value_stride elements (>= H_kv*d,
 *                multiple of 8), e.g. views into a fused QKV projection.
 *   k_cache, v_cache   device, [num_blocks, block_size, H_kv, d] bf16, contiguous.
 *   slot_mapping device, [num_tokens] int32; -1 = padding, nothing written.
 * Slots outside [-1, num_blocks*block_size) are skipped by the kernel.
 * num_tokens == 0 enqueues nothing and returns PKV_OK.
 * PKV_EINVAL: null pointers (num_tokens > 0), num_tokens < 0, non-positive
 * sizes, block_size not a power of two >= 16, a stride below H_kv*d or not a
 * multiple of 8, pointers not 16-byte aligned, int64 overflow of the pool size.
 */
pkv_status pkv_store(const void* key, int64_t key_stride, const void* value,
                     int64_t value_stride, void* k_cache, void* v_cache,
                     const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                     int32_t block_size, int32_t H_kv, int32_t d, hipStream_t stream);

/*
 * Bytes of device workspace pkv_decode needs for these sizes on the current
 * HIP device: two fp32 partial results (max, sum, d-vector) per query head of
 * a group for every share of the work schedule (2W + 14*ceil(W/2) shares
 * for the W resident wavefronts of the device), a 16-byte record per (sequence, KV head), and a
 * 256-byte line holding the schedule's share counter.  Query it with the
 * device current that will run the decode.  0 for invalid or unsupported
 * sizes.
 */
size_t pkv_decode_workspace_size(int32_t B, int32_t H_q, int32_t H_kv, int32_t d,
                                 int32_t block_size, int32_t max_blocks_per_seq);

/*
 * Paged decode attention (devpress page, "PagedAttention是如何实现的";
 * AIInfraGuide 3.6, section 2):
 *   out[b, h, :] = softmax_j( q[b,h,:] . K_b[j, h/G, :] * softmax_scale ) V_b[j, h/G, :]
 * over j in [0, context_lens[b]), where key j of sequence b is row
 * j % block_size of physical block block_tables[b][j / block_size].
 *   out, q        device, [B, H_q, d] bf16, contiguous (out rounded to nearest even)
 *   k_cache, v_cache   device, [num_blocks, block_size, H_kv, d] bf16, contiguous
 *   block_tables  device, [B, max_blocks_per_seq] int32, -1 padded (never read)
 *   context_lens  device, [B] int32, the just-stored token included; 0 gives a
 *                 zero output row; values above max_blocks_per_seq*block_size
 *                 are clamped to it
 *   workspace     device, >= pkv_decode_workspace_size(...) bytes, 16-byte
 *                 aligned, zero-filled before its first use (e.g. hipMemset).
 *                 Each call leaves it ready for the next one; calls that share
 *                 a workspace must run in stream order, never concurrently.
 *                 After a PKV_ELAUNCH it must be zero-filled again.
 * The causal mask of the pages' call is a no-op for one query per sequence.
 * The work (every 16-token tile of every (sequence, KV head)) is cut into
 * shares: one static share per resident wavefront of the device (all of the
 * work for calls of up to 64 tiles per wavefront, else 7/10 of it (4/5 for
 * G >= 4) up to 128 tiles per wavefront and 2/5 above), then shrinking shares that wavefronts
 * take from an atomic counter as they finish, so all of them stop at nearly
 * the same time.  K and V are read with non-temporal loads (each byte once).
 * Pieces of a sequence that span shares are merged with a log-sum-exp rescale
 * in a second kernel, in share order, so the result does not depend on which
 * wavefront took which share: results are deterministic run to run on one
 * device.
 * PKV_EINVAL: null pointers, non-positive sizes, H_q % H_kv != 0, block_size
 * not a power of two >= 16, misaligned pointers, too small a workspace, a
 * softmax_scale that is not finite.
 * PKV_EUNSUPPORTED: d not in {64, 128}; H_q/H_kv not in {1, 2, 4, 8};
 * B * H_kv * ceil(max_blocks_per_seq * block_size / 16) > INT32_MAX.
 */
pkv_status pkv_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                      int32_t H_q, int32_t H_kv, int32_t d, int32_t num_blocks,
                      int32_t block_size, int32_t max_blocks_per_seq, float softmax_scale,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);


/*
 * The store of a decode step fused into its attention call (devpress page,
 * KV-cache write then "PagedAttention是如何实现的"): the same result as
 * pkv_store of each sequence's new token followed by pkv_decode, in one
 * launch fewer.  Sequence b's new token sits at position p = context_lens[b] - 1
 * (its slot: row p % block_size of block block_tables[b][p / block_size]);
 * its K/V rows are key[b] and value[b].  The call writes them there, bit for
 * bit, and attends over positions [0, context_lens[b]) as pkv_decode does
 * (the new token's row is read from key/value, not from the cache).
 * Sequences with context_lens[b] <= 0 store nothing and give zero rows.
 *   key, value    device, [B, H_kv, d] bf16; head and d contiguous, sequence
 *                 stride key_stride / value_stride elements (>= H_kv*d,
 *                 multiple of 8), e.g. views into a fused QKV projection.
 *   the rest      as pkv_decode (same workspace size).
 * Preconditions as pkv_decode's, plus: the new token's block belongs to
 * sequence b alone (no other sequence of the call reads it), as a block that
 * is being written never holds a shared prefix.
 * PKV_EINVAL: pkv_decode's cases, null key/value, a stride below H_kv*d or
 * not a multiple of 8, key/value not 16-byte aligned.
 * PKV_EUNSUPPORTED: as pkv_decode.
 */
pkv_status pkv_store_decode(void* out, const void* q, const void* key, int64_t key_stride,
                            const void* value, int64_t value_stride, void* k_cache,
                            void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t B, int32_t H_q, int32_t H_kv,
                            int32_t d, int32_t num_blocks, int32_t block_size,
                            int32_t max_blocks_per_seq, float softmax_scale, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * Varlen causal prefill over the paged cache (devpress page, "如何适配不同请求
 * 不同序列长度"; AIInfraGuide 3.6, section 2).  Sequence b has
 * nq = cu_seqlens_q[b+1]-cu_seqlens_q[b] new queries and
 * nk = cu_seqlens_k[b+1]-cu_seqlens_k[b] keys, c = nk - nq of them cached.
 * Query i of sequence b sits at absolute position c + i and attends keys
 * 0 .. c + i (causal, bottom-right aligned), read through block_tables[b]:
 *   out[cu_q[b]+i, h, :] = softmax_j<=c+i( q . K_b[j, h/G] * scale ) V_b[j, h/G]
 * Only the differences of cu_seqlens_k are used: keys always come from the cache,
 * so the new tokens' K/V must have been stored first (pkv_store, same stream).
 *   out, q        device, [total_q, H_q, d] bf16, contiguous; total_q = cu_seqlens_q[B]
 *   cu_seqlens_q, cu_seqlens_k   device, [B+1] int32, cu_seqlens_q[0] == 0
 *   max_seqlen_q  host bound on nq (sizes the grid; sequences beyond it are cut)
 *   max_seqlen_k  host bound on nk (informational; keys are clamped to the table)
 *   other arguments as for pkv_decode.
 * Query rows at or beyond total_q are never written.
 * Precision: q.k products and all sums in fp32.  Every finite bf16 V is
 * accepted: the probabilities and V first enter the PV product as fp16; a
 * workgroup whose rows come out non-finite (a V value beyond fp16's range,
 * |v| >= 2^16) or all below 2^-14 in magnitude (where fp16 subnormals of tiny
 * V values would show) computes its tiles again with V in bf16 and the
 * probabilities split into bf16 high and low parts (about 2^-16 relative).
 * As in pkv_decode, the fp32 sums bound the result: sum_j p_j |v_j| with
 * max_j p_j = 1 must stay below fp32's largest value.
 * PKV_EINVAL / PKV_EUNSUPPORTED as for pkv_decode, plus total_q < 0,
 * max_seqlen_q < 0, B > 65535 or a softmax_scale that is not finite and
 * positive (PKV_EINVAL), and max_seqlen_q above
 * 65535 query tiles of 128 / G positions or H_kv * d above 2^24
 * (PKV_EUNSUPPORTED).  B == 0, total_q == 0 or max_seqlen_q == 0 enqueues
 * nothing.
 */
pkv_status pkv_prefill_varlen(void* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t B, int32_t total_q, int32_t max_seqlen_q,
                              int32_t max_seqlen_k, int32_t H_q, int32_t H_kv, int32_t d,
                              int32_t num_blocks, int32_t block_size,
                              int32_t max_blocks_per_seq, float softmax_scale,
                              hipStream_t stream);

/*
 * Varlen causal prefill over packed, non-paged K/V (devpress page, "如何适配
 * 不同请求不同序列长度": the varlen call without a block table, keys of all
 * sequences stacked on the token axis and addressed by cu_seqlens_k).
 * Sequence b has nq = cu_seqlens_q[b+1]-cu_seqlens_q[b] queries and
 * nk = cu_seqlens_k[b+1]-cu_seqlens_k[b] keys (nq <= nk; nq == nk is the
 * no-prefix case); query i sits at position nk - nq + i and attends keys
 * 0 .. nk - nq + i (causal, bottom-right aligned):
 *   out[cu_q[b]+i, h, :] = softmax_j( q . k[cu_k[b]+j, h/G] * scale ) v[cu_k[b]+j, h/G]
 *   q      device, [total_q, H_q, d] bf16 rows q_stride elements apart
 *   k, v   device, [total_k, H_kv, d] bf16 rows k_stride / v_stride elements apart
 *          (heads and d contiguous; e.g. views of a fused QKV projection)
 *   out    device, [total_q, H_q, d] bf16, contiguous
 *   cu_seqlens_q, cu_seqlens_k   device, [B+1] int32, cu_seqlens_q[0] == 0,
 *          cu_seqlens_q[B] == total_q, cu_seqlens_k[B] <= total_k
 *   max_seqlen_q  host bound on nq (sizes the grid; sequences beyond it are cut)
 *   max_seqlen_k  host bound on nk (informational)
 * Key rows outside [0, total_k) are never read (rows are clamped; the results
 * of calls that violate the cu_seqlens preconditions are unspecified).
 * Precision as for pkv_prefill_varlen (every finite bf16 V).
 * PKV_EINVAL: null pointers, non-positive sizes, H_q % H_kv != 0, a stride
 * below the row size or not a multiple of 8, misaligned pointers, B < 0,
 * B > 65535, total_q < 0, total_k < 0, total_k == 0 with work to do, or a
 * softmax_scale that is not finite and positive.
 * PKV_EUNSUPPORTED: d not in {64, 128}, H_q/H_kv not in {1, 2, 4, 8},
 * max_seqlen_q above 65535 query tiles of 128 / G positions, or k_stride or
 * v_stride above 2^24 elements.
 * B == 0, total_q == 0 or max_seqlen_q == 0 enqueues nothing.
 */
pkv_status pkv_prefill_varlen_packed(void* out, const void* q, int64_t q_stride, const void* k,
                                     int64_t k_stride, const void* v, int64_t v_stride,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     int32_t B, int32_t total_q, int32_t total_k,
                                     int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t H_q,
                                     int32_t H_kv, int32_t d, float softmax_scale,
                                     hipStream_t stream);

/*
 * Gumbel-max sampling (devpress page, "Gumbel-Max采样"; docs.vllm.com.cn,
 * "Model Runner V2 设计文档", section 6, the Gumbel sampling kernel).  For
 * row b of the logits, with temperature T = temperatures[b]:
 *   token[b] = argmax_i ( logits[b, i] / T + g_{b,i} ),  g = -ln(-ln u),
 * which draws token i with probability softmax(logits[b] / T)_i without
 * forming the softmax.  T <= 0 selects the plain argmax of logits[b] (no
 * noise).  Ties go to the smallest index.
 * The uniform u_{b,i} comes from a stateless counter-based generator,
 * Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
 * Easy as 1, 2, 3", SC 2011): key = (low, high 32 bits of seeds[b]), counter
 * = (i / 4, low, high 32 bits of offsets[b], 0); word i % 4 of the result, x,
 * gives u = ((x >> 9) + 0.5) * 2^-23, strictly inside (0, 1).  The same
 * (seed, offset) always gives the same draw; callers advance the offset per
 * step.
 * Arithmetic: fp32.  logits[b, i] / T is the correctly rounded quotient
 * (for tiny quotients, below 2^-80, its last bits may differ); g is
 * -ln(ln 2) - ln 2 * log2(-log2 u) on the hardware base-2 logarithm, within a
 * few ulp of an fp32 -ln(-ln u); the score is their fp32 sum.  Scores that
 * differ by less than this rounding (about 1e-5) may be ordered either way.
 *   logits       device [B, V], fp32 (logits_bf16 == 0) or bf16 (!= 0), rows
 *                row_stride elements apart, 16-byte aligned rows
 *   temperatures device [B] fp32, or null for T = 1
 *   seeds        device [B] int64;  offsets: device [B] int64, or null for 0
 *   tokens       device [B] int64, written
 *   workspace    device, pkv_sample_workspace_size(B, V) bytes, 8-byte
 *                aligned (no contents carried between calls; calls that
 *                share one must run in stream order, never concurrently)
 * Logits must be finite (NaN and infinities are unspecified).
 * PKV_EINVAL: B < 0, B > 65535, V < 1, row_stride < V or not a multiple of
 * 8 (bf16) / 4 (fp32), null pointers, misaligned logits or workspace
 * (B > 0), a short workspace.
 * B == 0 enqueues nothing.
 */
/* Workspace bytes pkv_sample_gumbel needs: 8 per row per 4096-logit chunk
 * (0 for B < 1 or V < 1). */
size_t pkv_sample_workspace_size(int32_t B, int32_t V);

pkv_status pkv_sample_gumbel(int64_t* tokens, const void* logits, int32_t logits_bf16,
                             int64_t row_stride, int32_t B, int32_t V,
                             const float* temperatures, const int64_t* seeds,
                             const int64_t* offsets, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * pkv_sample_gumbel without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, draws and results as
 * pkv_sample_gumbel (the same kernels, bit-identical tokens); the chunk keys
 * go to a fixed scratch array inside the library instead of a workspace:
 * 2^17 keys of 8 bytes (1 MiB) per device, held from the library's first use
 * on that device until the process ends.  The first call on each device
 * looks up that device's copy (no allocation); nothing in it needs clearing,
 * since every key a call reads is written by the same call.
 * Limit: B * ceil(V / chunk) <= 131072 keys, chunk = 8192 logits for bf16 and
 * 4096 for fp32 (e.g. V = 151936: B <= 6898 bf16, B <= 3449 fp32); larger
 * calls return PKV_ESCRATCH and enqueue nothing.
 * Every call on one device shares that device's array: calls that can
 * overlap on one device (other streams, other host threads) race and give
 * unspecified tokens; keep them in one stream's order.
 * Errors as for pkv_sample_gumbel (without the workspace checks), plus
 * PKV_ESCRATCH, and PKV_ELAUNCH if the scratch address cannot be found.
 */
pkv_status pkv_sample_gumbel_noalloc(int64_t* tokens, const void* logits, int32_t logits_bf16,
                                     int64_t row_stride, int32_t B, int32_t V,
                                     const float* temperatures, const int64_t* seeds,
                                     const int64_t* offsets, hipStream_t stream);

/*
 * Staged row writes into a device int32 table (docs.vllm.com.cn, "Model
 * Runner V2 设计文档", section 4, StagedWriteTensor): the table stays on the
 * device; the host stages ragged writes (row, start, values), packs them
 * into one contiguous buffer, copies that buffer to the device and launches
 * one kernel that applies every write.  Used for block tables, whose rows
 * grow by a few ids per step.
 *
 * Packed layout (int32, n writes, `total` values):
 *   [0, n)              row of each write
 *   [n, 2n)             first column of each write
 *   [2n, 3n+1)          offsets: write w's values are values[off[w] .. off[w+1]),
 *                       off[0] == 0, off[n] == total
 *   [3n+1, 3n+1+total)  the values, write after write
 * Size: 3n + 1 + total int32.
 */

/*
 * Host: packs n writes (write w puts lens[w] values, taken in order from
 * `values` after those of the writes before it, into row rows[w] from column
 * starts[w] on) into `packed` (host memory of packed_capacity int32).
 * *packed_size receives 3n + 1 + total.
 * PKV_EINVAL: n < 0; null pointers (n > 0); a write outside [0, num_rows) x
 * [0, num_cols); a negative length; two writes that cover one element (the
 * order of overlapping writes would be unspecified); a capacity below the
 * packed size; int32 overflow of the total.
 */
pkv_status pkv_pack_row_writes(int32_t n, const int32_t* rows, const int32_t* starts,
                               const int32_t* lens, const int32_t* values, int32_t num_rows,
                               int32_t num_cols, int32_t* packed, int64_t packed_capacity,
                               int64_t* packed_size);

/*
 * Device: applies a packed buffer (device memory, the layout above) to
 * table[num_rows, num_cols] (device, int32, rows row_stride elements apart).
 * One thread per value; elements outside the table are skipped.  n == 0 or
 * total == 0 enqueues nothing.
 * PKV_EINVAL: null pointers (with work to do), n < 0, total < 0,
 * num_rows < 1, num_cols < 1, row_stride < num_cols.
 */
pkv_status pkv_apply_row_writes(int32_t* table, int64_t row_stride, int32_t num_rows,
                                int32_t num_cols, const int32_t* packed, int32_t n,
                                int32_t total, hipStream_t stream);

/*
 * Step metadata built on the device (docs.vllm.com.cn, "Model Runner V2
 * 设计文档", section 5: inputs prepared by GPU kernels from state kept on the
 * GPU), with the meaning of pkv_prepare_metadata (AIInfraGuide 3.6,
 * section 2).  Batch row b is the request in row r = idx_mapping[b] of the
 * persistent state: c = num_computed[r] tokens already cached, n =
 * num_scheduled[b] new tokens this step, physical block ids in
 * block_table[r, 0 ..].
 * Inputs (device):
 *   idx_mapping     [B] int32 rows of the persistent state (null: row b)
 *   num_computed    [num_reqs] int32
 *   num_scheduled   [B] int32
 *   block_table     [num_reqs, table_stride] int32
 * Outputs (device):
 *   cu_seqlens_q, cu_seqlens_k   [B+1]  prefix sums of n and of c + n
 *   context_lens    [B]       c + n
 *   positions       [max_tokens] int64: c + i for new token i (may be null)
 *   slot_mapping    [max_tokens] int32: block_table[r, p / bs] * bs + p % bs
 *                   for position p = c + i; -1 if that id is negative
 *   block_tables    [B, max_blocks_per_seq] int32: the ids covering the c + n
 *                   tokens, then -1 (may be null)
 *   max_seqlens     [2] int32: max n, max (c + n) (may be null)
 * Token rows at or beyond min(sum n, max_tokens) are not written.  One
 * kernel launch.  Preconditions (device data, not checked): 0 <= r <
 * num_reqs, c >= 0, n >= 0, ceil((c + n) / bs) <= max_blocks_per_seq <=
 * table_stride, sums within int32.
 * PKV_EINVAL: B < 0, null required pointers (B > 0), num_reqs < 1,
 * block_size not a power of two >= 16, max_blocks_per_seq < 1,
 * table_stride < max_blocks_per_seq, max_tokens < 0.
 * PKV_EUNSUPPORTED: B > 4096 (the prefix sums are kept in LDS).
 * B == 0 writes cu_seqlens_q[0] = cu_seqlens_k[0] = 0 only.
 */
pkv_status pkv_prepare_metadata_device(int32_t B, const int32_t* idx_mapping,
                                       const int32_t* num_computed, const int32_t* num_scheduled,
                                       const int32_t* block_table, int32_t num_reqs,
                                       int64_t table_stride, int32_t block_size,
                                       int32_t max_blocks_per_seq, int32_t max_tokens,
                                       int32_t* cu_seqlens_q, int32_t* cu_seqlens_k,
                                       int32_t* context_lens, int64_t* positions,
                                       int32_t* slot_mapping, int32_t* block_tables,
                                       int32_t* max_seqlens, hipStream_t stream);

/*
 * Graph-captured decode step with batch buckets (devpress page,
 * "CUDAGraph优化"; AIInfraGuide 3.6, section 5).  A decode step is, for every
 * layer l, pkv_store of the batch's new K/V rows into layer l's caches
 * followed by pkv_decode over them.  Its kernels, launch shapes and their
 * order depend only on the batch size, so one graph is captured per batch
 * bucket over static buffers sized for max_batch rows, and a step of `batch`
 * rows replays the smallest bucket >= batch with the rows beyond `batch`
 * padded: slot -1 (the store skips them) and context length 0 (their outputs
 * are zero rows).
 *
 * Buckets: 1, 2, 4, 8, then every multiple of 16 up to max_batch, then
 * max_batch itself when it is not already one (the pages' list stops at the
 * last multiple of 16; adding max_batch lets every batch up to it replay).
 * Batches above max_batch (above 512 in the pages) run eagerly: the caller
 * issues pkv_store / pkv_decode itself.
 */
typedef struct pkv_decode_graph pkv_decode_graph;

/*
 * The step a graph set captures: for each layer l, one pkv_store_decode call
 * over the batch's rows (row b's new token, key[l][b] and value[l][b], goes to
 * position context_lens[b] - 1 through block_tables, the slot the pages'
 * decode metadata puts in slot_mapping, and is attended with the rest).  All
 * pointers are device pointers except the per-layer arrays themselves (host
 * arrays of `layers` device pointers, read at create time; the graphs bake in
 * the device addresses, so the buffers must stay allocated and in place while
 * the graph set exists).
 *   slot_mapping   [max_batch] int32   the batch's slots (rows [0, batch)
 *                                      written by the caller, for its own
 *                                      use: the step stores through the
 *                                      table); the replay sets the padding
 *                                      rows [batch, bucket) to -1
 *   context_lens   [max_batch] int32   rows [0, batch) written by the caller
 *                                      before each replay; the replay writes
 *                                      0 to the padding rows [batch, bucket)
 *   block_tables   [max_batch, max_blocks_per_seq] int32
 *   q[l], out[l]   [max_batch, H_q, d] bf16, contiguous
 *   key[l], value[l]   [max_batch, H_kv, d] bf16 rows key_stride /
 *                  value_stride elements apart (as for pkv_store)
 *   k_cache[l], v_cache[l]   [num_blocks, block_size, H_kv, d] bf16
 *   workspace      pkv_decode_workspace_size(max_batch, ...) bytes or more,
 *                  zero-filled before create, used by nothing else while
 *                  the graph set exists (every layer of every replay uses it
 *                  in stream order).
 */
typedef struct pkv_decode_step {
  int32_t layers;
  int32_t max_batch;
  int32_t H_q, H_kv, d;
  int32_t num_blocks, block_size, max_blocks_per_seq;
  float softmax_scale;
  int32_t* slot_mapping;
  int32_t* context_lens;
  const int32_t* block_tables;
  const void* const* q;
  const void* const* key;
  const void* const* value;
  int64_t key_stride, value_stride;
  void* const* k_cache;
  void* const* v_cache;
  void* const* out;
  void* workspace;
  size_t workspace_bytes;
} pkv_decode_step;

/*
 * Bucket a batch of `batch` rows replays for a graph set of max_batch rows:
 * the smallest bucket >= batch; -1 when batch < 1, batch > max_batch or
 * max_batch is outside [1, 512].  Host only.
 */
int32_t pkv_decode_graph_bucket(int32_t max_batch, int32_t batch);

/*
 * Captures one graph per bucket on the current HIP device.  Blocking set-up
 * call: it waits for all work already enqueued on the device (so the caller's
 * fills of the static buffers and the workspace, on any stream, are done),
 * then writes slot -1 and context length 0 to all max_batch rows,
 * runs the step once eagerly on those all-padding rows (which loads every
 * kernel and writes zero rows to out[*][0, max_batch)), captures the graphs
 * on a stream of its own and waits for that stream.  On success *graph owns
 * the graphs; release them with pkv_decode_graph_destroy.
 * PKV_EINVAL: null pointers, layers < 1, max_batch outside [1, 512], a
 * workspace smaller than needed, or any argument pkv_store_decode would
 * reject.  PKV_EUNSUPPORTED as for pkv_decode.  PKV_ELAUNCH: the HIP
 * runtime failed (nothing is left allocated).
 */
pkv_status pkv_decode_graph_create(const pkv_decode_step* step, pkv_decode_graph** graph);

/*
 * Enqueues one decode step of `batch` rows on `stream`: a small kernel that
 * writes slot -1 and context length 0 to rows [batch, bucket) (none when
 * batch is a bucket), then the bucket's graph.  The caller has written rows
 * [0, batch) of the static metadata, q, key and value, in stream order.
 * Afterwards out[l] rows [0, batch) hold the attention outputs, rows
 * [batch, bucket) are zero, rows beyond the bucket are untouched.  Replays
 * of one graph set share its workspace: they must be ordered (one stream, or
 * events).  batch == 0 enqueues nothing.
 * PKV_EINVAL: null graph, batch < 0 or batch > max_batch.  PKV_ELAUNCH: the
 * HIP runtime failed.
 */
pkv_status pkv_decode_graph_replay(pkv_decode_graph* graph, int32_t batch, hipStream_t stream);

/*
 * The same step issued eagerly on `stream` (the pages' enforce_eager branch):
 * for each layer, pkv_store_decode over rows [0, batch) of the step's
 * buffers, with no padding.  Not blocking.  Same errors as
 * pkv_decode_graph_create for the step, plus batch outside [0, max_batch].
 */
pkv_status pkv_decode_step_run(const pkv_decode_step* step, int32_t batch, hipStream_t stream);

/* Waits for the device to finish all enqueued work (so no replay is still
 * running), then releases the graphs.  Null is a no-op. */
void pkv_decode_graph_destroy(pkv_decode_graph* graph);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
