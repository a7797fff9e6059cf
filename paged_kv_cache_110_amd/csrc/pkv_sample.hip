// Gumbel-max sampling over logits (devpress "nano-vllm解读", "Gumbel-Max采样";
// docs.vllm.com.cn, "Model Runner V2 设计文档", section 6): the token of row b
// is argmax_i (logits[b, i] / T_b + g_{b,i}) with g = -ln(-ln u) and u from a
// stateless counter-based generator, Philox4x32-10 (Salmon, Moraes, Dror and
// Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011), keyed by the
// row's seed and counted by (vocabulary index / 4, the row's offset).
//
// Two launches.  sample_chunk_kernel: one workgroup per (chunk of the
// vocabulary, row); every thread holds 4 x 16 bytes of logits (32 bf16 or 16
// fp32 values), the workgroup finds the chunk's largest logit, and only groups
// of 4 logits that can still win (see kPruneSpan) get their Philox block and
// noise; each wavefront packs its surviving groups into a list in LDS and
// shares them out over its lanes, unless most groups survive.  The best
// (score, index) is kept as one ordered 64-bit key; the workgroup's best key
// goes to the workspace.
// sample_reduce_kernel: one wavefront per row takes the best chunk key and
// writes the token.  Keys order by score, then by smaller index.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kSampleThreads = 256;
constexpr int kSampleSteps = 4;  // 16-byte loads per thread per chunk

template <bool BF16>
struct SampleShape {
  static constexpr int kPerLoad = BF16 ? 8 : 4;  // logits per 16-byte load
  static constexpr int kChunk = kSampleThreads * kPerLoad * kSampleSteps;
};

int32_t sample_chunk_size(bool bf16) {
  return bf16 ? SampleShape<true>::kChunk : SampleShape<false>::kChunk;
}

// Philox4x32-10: ten rounds of two 32x32->64 products, the high halves xored
// into the other counter words with the round key, the key bumped by the
// Weyl constants after every round.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)kM0 * c[0];
    const uint64_t p1 = (uint64_t)kM1 * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
    k0 += kW0;
    k1 += kW1;
  }
}

// g = -ln(-ln u), u = ((x >> 9) + 0.5) * 2^-23 (exact in fp32, inside (0, 1)).
// logf, not the hardware log2: near u = 1 the inner logarithm is tiny and
// must keep its relative accuracy, since those draws give the largest g.
__device__ __forceinline__ float gumbel_of(uint32_t x) {
  const float u = ((float)(x >> 9) + 0.5f) * 0x1p-23f;
  return -logf(-logf(u));
}

// Ordered key: larger score first, then smaller index.
__device__ __forceinline__ uint64_t score_key(float s, uint32_t idx) {
  uint32_t b = __float_as_uint(s);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)k, off, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(k >> 32), off, 64);
    k = umax64(k, ((uint64_t)hi << 32) | lo);
  }
  return k;
}

// Exact pruning.  u lies in [2^-24, 1 - 2^-24], so every g lies in
// [-2.81156, 16.63553]: a logit x with x / T + 16.63553 below m / T - 2.81156,
// m the chunk's largest logit, scores below the chunk's best whatever the
// draws, and its noise need not be computed.  kPruneSpan = 19.5 > 19.44709
// leaves 0.05 for the rounding of the fp32 scores (plus a relative term for
// very large |m / T|), so pruning never changes the chunk's best key.
constexpr float kPruneSpan = 19.5f;

template <bool BF16>
__global__ __launch_bounds__(kSampleThreads) void sample_chunk_kernel(
    const uint16_t* __restrict__ logits, int64_t row_stride, int32_t V, int32_t nchunks,
    const float* __restrict__ temps, const int64_t* __restrict__ seeds,
    const int64_t* __restrict__ offsets, uint64_t* __restrict__ partial) {
  using S = SampleShape<BF16>;
  constexpr int NX = kSampleSteps * S::kPerLoad;  // logits per thread
  constexpr int NG = NX / 4;                       // groups of 4 (one Philox block each)
  const int b = blockIdx.y;
  const int chunk = blockIdx.x;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const float T = temps ? temps[b] : 1.0f;
  const bool greedy = !(T > 0.0f);
  const uint64_t seed = (uint64_t)seeds[b];
  const uint64_t off = offsets ? (uint64_t)offsets[b] : 0ull;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const uint32_t c1 = (uint32_t)off, c2 = (uint32_t)(off >> 32);
  // row base in 16-bit units (fp32 rows are twice as long)
  const uint16_t* row = logits + (int64_t)b * row_stride * (BF16 ? 1 : 2);
  // index of this thread's first logit of step st (S::kPerLoad consecutive logits)
  auto first = [&](int st) -> int64_t {
    return (int64_t)chunk * S::kChunk + ((int64_t)st * kSampleThreads + threadIdx.x) * S::kPerLoad;
  };
  auto load_logit = [&](int64_t i) -> float {
    return BF16 ? __uint_as_float((uint32_t)row[i] << 16) : reinterpret_cast<const float*>(row)[i];
  };

  // 1. every logit of the thread (-inf past the end of the row), and their max
  float x[NX];
  float mt = -INFINITY;
#pragma unroll
  for (int st = 0; st < kSampleSteps; ++st) {
    const int64_t i0 = first(st);
    float* xs = x + st * S::kPerLoad;
    if (i0 + S::kPerLoad <= V) {
      const u32x4 w = ld16(row + i0 * (BF16 ? 1 : 2));
      if (BF16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          xs[2 * k] = bf16_lo(w[k]);
          xs[2 * k + 1] = bf16_hi(w[k]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) xs[k] = __uint_as_float(w[k]);
      }
    } else {  // the row's ragged end
#pragma unroll
      for (int e = 0; e < S::kPerLoad; ++e) xs[e] = i0 + e < V ? load_logit(i0 + e) : -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < S::kPerLoad; ++e) mt = fmaxf(mt, xs[e]);
  }
  auto index_of = [&](int j) -> int64_t { return first(j / S::kPerLoad) + j % S::kPerLoad; };

  __shared__ uint64_t red[kSampleThreads / 64];
  __shared__ float redf[kSampleThreads / 64];
  __shared__ int32_t work[kSampleThreads / 64][64 * NG];  // compacted groups, per wavefront
  uint64_t best = 0;
  // scores one group of 4 consecutive logits (first index i, values v[4])
  auto score_group = [&](int64_t i, const float (&v)[4]) {
    uint32_t r[4] = {(uint32_t)(i >> 2), c1, c2, 0u};
    philox4x32_10(r, k0, k1);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (i + e < V) best = umax64(best, score_key(v[e] / T + gumbel_of(r[e]), (uint32_t)(i + e)));
  };

  if (greedy) {
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      const int64_t i = index_of(j);
      if (i < V) best = umax64(best, score_key(x[j], (uint32_t)i));
    }
  } else {
    // 2. the chunk's largest logit, and the pruning threshold in logit units
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o, 64));
    if (lane == 0) redf[wave] = mt;
    __syncthreads();
    float m = redf[0];
#pragma unroll
    for (int w = 1; w < kSampleThreads / 64; ++w) m = fmaxf(m, redf[w]);
    const float ms = m / T;
    float thr = (ms - kPruneSpan - 1e-5f * fabsf(ms)) * T;
    if (!(fabsf(thr) < INFINITY)) thr = -INFINITY;  // m / T overflowed: no pruning
    // 3. groups with a logit at or above the threshold
    uint32_t gmask = 0;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      bool keep = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) keep |= x[4 * g + e] >= thr;
      gmask |= keep ? (1u << g) : 0u;
    }
    const int cnt = __popc(gmask);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const int total = __shfl(incl, 63, 64);
    if (total * 2 > 64 * NG) {
      // most groups survive: score them where they are
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (gmask & (1u << g)) {
          const float v[4] = {x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
          score_group(index_of(4 * g), v);
        }
      }
    } else {
      // 4. compact the surviving groups of the wavefront, then share them out
      int slot = incl - cnt;
#pragma unroll
      for (int g = 0; g < NG; ++g)
        if (gmask & (1u << g)) work[wave][slot++] = (int32_t)index_of(4 * g);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int e = lane; e < total; e += 64) {
        const int64_t i = work[wave][e];
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = i + k < V ? load_logit(i + k) : -INFINITY;
        score_group(i, v);
      }
    }
  }
  best = wave_max_key(best);
  if (lane == 0) red[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kSampleThreads / 64; ++w) best = umax64(best, red[w]);
    partial[(int64_t)b * nchunks + chunk] = best;
  }
}

__global__ __launch_bounds__(64) void sample_reduce_kernel(const uint64_t* __restrict__ partial,
                                                           int32_t nchunks,
                                                           int64_t* __restrict__ tokens) {
  const int b = blockIdx.x;
  uint64_t best = 0;
  for (int c = threadIdx.x; c < nchunks; c += 64) best = umax64(best, partial[(int64_t)b * nchunks + c]);
  best = wave_max_key(best);
  if (threadIdx.x == 0) tokens[b] = (int64_t)(0xFFFFFFFFu - (uint32_t)best);
}

hipError_t launch_sample(int64_t* tokens, const void* logits, bool bf16, int64_t row_stride,
                         int32_t B, int32_t V, const float* temps, const int64_t* seeds,
                         const int64_t* offsets, void* workspace, hipStream_t stream) {
  const int32_t chunk = sample_chunk_size(bf16);
  const int32_t nchunks = (V + chunk - 1) / chunk;
  uint64_t* partial = static_cast<uint64_t*>(workspace);
  const dim3 grid((unsigned)nchunks, (unsigned)B);
  const uint16_t* lg = static_cast<const uint16_t*>(logits);
  if (bf16)
    hipLaunchKernelGGL(sample_chunk_kernel<true>, grid, dim3(kSampleThreads), 0, stream, lg,
                       row_stride, V, nchunks, temps, seeds, offsets, partial);
  else
    hipLaunchKernelGGL(sample_chunk_kernel<false>, grid, dim3(kSampleThreads), 0, stream, lg,
                       row_stride, V, nchunks, temps, seeds, offsets, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sample_reduce_kernel, dim3((unsigned)B), dim3(64), 0, stream, partial,
                     nchunks, tokens);
  return hipGetLastError();
}

}  // namespace pkv
