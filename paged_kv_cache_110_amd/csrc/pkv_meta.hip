// Step metadata on the device, and staged row writes into device tables
// (docs.vllm.com.cn, "Model Runner V2 设计文档": section 4, StagedWriteTensor;
// section 5, inputs prepared on the GPU from state kept on the GPU).  The
// arithmetic is that of the host metadata step (AIInfraGuide 3.6, section 2):
// prefix sums of new and total tokens, position c + i of new token i, slot
// block_table[p / bs] * bs + p % bs, -1-padded block tables.
//
// Integer work of a few kilobytes per step: latency-bound, so everything runs
// in one launch.  Every block rebuilds the batch's prefix sums in LDS (B is at
// most 4096) and then takes a grid-stride share of the token rows and of the
// block-table entries.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kMetaThreads = 256;
constexpr int kMetaPerThread = kMetaMaxBatch / kMetaThreads;

__device__ __forceinline__ int meta_wave_scan(int x, int lane) {  // inclusive
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// ------------------------------------------------------------- row writes

// Packed layout: rows[n], starts[n], off[n+1], values[total].
__global__ __launch_bounds__(kMetaThreads) void apply_writes_kernel(
    int32_t* __restrict__ table, int64_t row_stride, int32_t num_rows, int32_t num_cols,
    const int32_t* __restrict__ packed, int32_t n, int32_t total) {
  const int32_t* rows = packed;
  const int32_t* starts = packed + n;
  const int32_t* off = packed + 2 * (int64_t)n;
  const int32_t* vals = off + n + 1;
  const int64_t step = (int64_t)gridDim.x * kMetaThreads;
  for (int64_t i = (int64_t)blockIdx.x * kMetaThreads + threadIdx.x; i < total; i += step) {
    int lo = 0, hi = n;  // off[lo] <= i < off[hi]: the last write starting at or before i
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= i) lo = mid;
      else hi = mid;
    }
    const int32_t r = rows[lo];
    const int64_t c = (int64_t)starts[lo] + (i - off[lo]);
    if (r >= 0 && r < num_rows && c >= 0 && c < num_cols) table[r * row_stride + c] = vals[i];
  }
}

hipError_t launch_apply_writes(int32_t* table, int64_t row_stride, int32_t num_rows,
                               int32_t num_cols, const int32_t* packed, int32_t n, int32_t total,
                               hipStream_t stream) {
  const int64_t want = ((int64_t)total + kMetaThreads - 1) / kMetaThreads;
  const unsigned blocks = (unsigned)(want < 1024 ? want : 1024);
  hipLaunchKernelGGL(apply_writes_kernel, dim3(blocks), dim3(kMetaThreads), 0, stream, table,
                     row_stride, num_rows, num_cols, packed, n, total);
  return hipGetLastError();
}

// ------------------------------------------------------------- step metadata

__global__ __launch_bounds__(kMetaThreads) void metadata_kernel(
    int32_t B, const int32_t* __restrict__ idx_mapping, const int32_t* __restrict__ num_computed,
    const int32_t* __restrict__ num_scheduled, const int32_t* __restrict__ block_table,
    int32_t num_reqs, int64_t table_stride, int32_t bs_log2, int32_t maxb, int32_t max_tokens,
    int32_t* __restrict__ cu_q_out, int32_t* __restrict__ cu_k_out,
    int32_t* __restrict__ ctx_out, int64_t* __restrict__ pos_out, int32_t* __restrict__ slot_out,
    int32_t* __restrict__ bt_out, int32_t* __restrict__ max_out) {
  __shared__ int32_t cq[kMetaMaxBatch + 1];  // cu_seqlens_q
  __shared__ int32_t ck[kMetaMaxBatch + 1];  // cu_seqlens_k
  __shared__ int32_t cached[kMetaMaxBatch];  // c of batch row b
  __shared__ int32_t req[kMetaMaxBatch];     // persistent row of batch row b
  __shared__ int32_t part[2][kMetaThreads / 64];
  __shared__ int32_t mx[2][kMetaThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid % 64, wave = tid / 64;
  const int bs = 1 << bs_log2;

  // 1. each thread owns kMetaPerThread consecutive batch rows
  int nq[kMetaPerThread], nk[kMetaPerThread];
  int sq = 0, sk = 0, mq = 0, mk = 0;
#pragma unroll
  for (int k = 0; k < kMetaPerThread; ++k) {
    const int b = tid * kMetaPerThread + k;
    int n = 0, c = 0;
    if (b < B) {
      int r = idx_mapping ? idx_mapping[b] : b;
      r = r < 0 ? 0 : (r >= num_reqs ? num_reqs - 1 : r);
      c = num_computed[r];
      n = num_scheduled[b];
      c = c < 0 ? 0 : c;
      n = n < 0 ? 0 : n;
      cached[b] = c;
      req[b] = r;
    }
    nq[k] = n;
    nk[k] = c + n;
    sq += n;
    sk += c + n;
    mq = n > mq ? n : mq;
    mk = c + n > mk ? c + n : mk;
  }
  // 2. block-wide exclusive scan of the per-thread sums
  const int iq = meta_wave_scan(sq, lane), ik = meta_wave_scan(sk, lane);
  int wq = mq, wk = mk;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int a = __shfl_xor(wq, off, 64), b = __shfl_xor(wk, off, 64);
    wq = a > wq ? a : wq;
    wk = b > wk ? b : wk;
  }
  if (lane == 63) {
    part[0][wave] = iq;
    part[1][wave] = ik;
  }
  if (lane == 0) {
    mx[0][wave] = wq;
    mx[1][wave] = wk;
  }
  __syncthreads();
  int bq = 0, bk = 0;
  for (int w = 0; w < wave; ++w) {
    bq += part[0][w];
    bk += part[1][w];
  }
  int rq = bq + iq - sq, rk = bk + ik - sk;  // exclusive prefix at this thread's first row
#pragma unroll
  for (int k = 0; k < kMetaPerThread; ++k) {
    const int b = tid * kMetaPerThread + k;
    if (b <= B) {  // entry B is the total
      cq[b] = rq;
      ck[b] = rk;
    }
    rq += nq[k];
    rk += nk[k];
  }
  if (B == kMetaMaxBatch && tid == kMetaThreads - 1) {  // the total of a full batch
    cq[B] = rq;
    ck[B] = rk;
  }
  __syncthreads();

  // 3. per-sequence outputs (block 0)
  if (blockIdx.x == 0) {
    for (int b = tid; b <= B; b += kMetaThreads) {
      cu_q_out[b] = cq[b];
      cu_k_out[b] = ck[b];
      if (b < B) ctx_out[b] = ck[b + 1] - ck[b];
    }
    if (tid == 0 && max_out) {
      int a = 0, c = 0;
      for (int w = 0; w < kMetaThreads / 64; ++w) {
        a = mx[0][w] > a ? mx[0][w] : a;
        c = mx[1][w] > c ? mx[1][w] : c;
      }
      max_out[0] = a;
      max_out[1] = c;
    }
  }
  if (B == 0) return;

  // 4. token rows: position and slot of new token t
  const int total = cq[B] < max_tokens ? cq[B] : max_tokens;
  const int64_t step = (int64_t)gridDim.x * kMetaThreads;
  for (int64_t t = (int64_t)blockIdx.x * kMetaThreads + tid; t < total; t += step) {
    int lo = 0, hi = B;  // cq[lo] <= t < cq[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cq[mid] <= t) lo = mid;
      else hi = mid;
    }
    const int64_t p = (int64_t)cached[lo] + (t - cq[lo]);
    const int64_t j = p >> bs_log2;
    int32_t slot = -1;
    if (j < maxb) {
      const int32_t id = block_table[req[lo] * table_stride + j];
      const int64_t s = (int64_t)id * bs + (p & (bs - 1));
      if (id >= 0 && s <= INT32_MAX) slot = (int32_t)s;
    }
    slot_out[t] = slot;
    if (pos_out) pos_out[t] = p;
  }

  // 5. block tables of the batch: the ids covering c + n tokens, then -1
  if (!bt_out) return;
  const int64_t entries = (int64_t)B * maxb;
  for (int64_t e = (int64_t)blockIdx.x * kMetaThreads + tid; e < entries; e += step) {
    const int b = (int)(e / maxb);
    const int j = (int)(e - (int64_t)b * maxb);
    const int len = ck[b + 1] - ck[b];
    const int need = (int)(((int64_t)len + bs - 1) >> bs_log2);
    bt_out[e] = j < need ? block_table[req[b] * table_stride + j] : -1;
  }
}

hipError_t launch_metadata(int32_t B, const int32_t* idx_mapping, const int32_t* num_computed,
                           const int32_t* num_scheduled, const int32_t* block_table,
                           int32_t num_reqs, int64_t table_stride, int32_t block_size,
                           int32_t max_blocks_per_seq, int32_t max_tokens, int32_t* cu_seqlens_q,
                           int32_t* cu_seqlens_k, int32_t* context_lens, int64_t* positions,
                           int32_t* slot_mapping, int32_t* block_tables, int32_t* max_seqlens,
                           hipStream_t stream) {
  int bs_log2 = 0;
  while ((1 << bs_log2) < block_size) ++bs_log2;
  const int64_t work = (int64_t)max_tokens > (int64_t)B * max_blocks_per_seq
                           ? (int64_t)max_tokens
                           : (int64_t)B * max_blocks_per_seq;
  int64_t blocks = (work + kMetaThreads - 1) / kMetaThreads;
  blocks = blocks < 1 ? 1 : (blocks > 256 ? 256 : blocks);
  hipLaunchKernelGGL(metadata_kernel, dim3((unsigned)blocks), dim3(kMetaThreads), 0, stream, B,
                     idx_mapping, num_computed, num_scheduled, block_table, num_reqs,
                     table_stride, bs_log2, max_blocks_per_seq, max_tokens, cu_seqlens_q,
                     cu_seqlens_k, context_lens, positions, slot_mapping, block_tables,
                     max_seqlens);
  return hipGetLastError();
}

}  // namespace pkv
