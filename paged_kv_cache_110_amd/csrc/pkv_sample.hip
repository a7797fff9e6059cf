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
// shares them out over its lanes, unless most groups survive.  Each thread
// keeps its best (score, index); the workgroup reduces them as ordered 64-bit
// keys and its best key goes to the workspace.
// sample_reduce_kernel: one wavefront per row takes the best chunk key and
// writes the token.  Keys order by score, then by smaller index.
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "pkv_internal.h"

// Fixed scratch of the no-allocation entry point: the chunk keys of one call
// (kSampleScratchKeys x 8 bytes), one copy per device, held until the process
// ends.  Host code must never pass this name to a kernel: on the host it is a
// stand-in, not the device address, which sample_scratch_address looks up.
static __device__ __align__(256) uint64_t scratch[pkv::kSampleScratchKeys];

namespace pkv {

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_address[kMaxScratchDevices];  // per device, set on first use
}  // namespace

hipError_t sample_scratch_address(void** address) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_address[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_address[dev] = p;
  }
  *address = g_scratch_address[dev];
  return hipSuccess;
}

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
// Weyl constants after every round.  Each three-way xor is one v_bitop3_b32
// (truth table 0x96); the key schedule stays in scalar registers.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)kM0 * c[0];
    const uint64_t p1 = (uint64_t)kM1 * c[2];
    const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c[1], k0);
    const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c[3], k1);
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
    k0 += kW0;
    k1 += kW1;
  }
}

// g = -ln(-ln u), u = ((x >> 9) + 0.5) * 2^-23 (exact in fp32, inside (0, 1)),
// taken as -ln(ln 2) - ln 2 * log2(-log2 u): two hardware base-2 logarithms
// (v_log_f32, relative error about 1 ulp, accurate near 1 as well) and one
// fma.  Neither logarithm sees a denormal or a value outside (0, 24], so the
// library logf's range handling is not needed.  The result differs from an
// fp32 -ln(-ln u) by a few units in the last place at most.
__device__ __forceinline__ float gumbel_of(uint32_t x) {
  constexpr float kLn2 = 0.693147180559945309f;
  constexpr float kNegLnLn2 = 0.366512920581664327f;  // -ln(ln 2)
  const float u = fmaf((float)(x >> 9), 0x1p-23f, 0x1p-24f);
  const float w = -__builtin_amdgcn_logf(u);  // -log2 u, in [8.6e-8, 24]
  return fmaf(-kLn2, __builtin_amdgcn_logf(w), kNegLnLn2);
}

// x / T.  FAST: the product with r = 1/T (correctly rounded) plus one fma
// correction of its residual.  For temperatures in [2^-32, 2^32] and |x| and
// |x| / T in [2^-80, 2^126) it gave the IEEE quotient on every pair checked
// (each finite bf16 value and random fp32 values, at over 600 temperatures);
// below 2^-80 its last bits may differ, far below the noise added to it.  The
// kernel takes it only for chunks whose largest logit keeps every quotient
// that can win below 2^126.
template <bool FAST>
__device__ __forceinline__ float div_t(float x, float T, float r) {
  if constexpr (FAST) {
    const float q = x * r;
    return fmaf(fmaf(-q, T, x), r, q);
  } else {
    return x / T;
  }
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
  // the thread's best candidate; equal scores go to the smaller index
  float bs = -INFINITY;
  uint32_t bi = 0xFFFFFFFFu;
  // (bitwise, so that the update compiles to selects, not branches)
  auto consider = [&](bool valid, float s, uint32_t i) {
    const bool take = valid & ((s > bs) | ((s == bs) & (i < bi)));
    bs = take ? s : bs;
    bi = take ? i : bi;
  };
  // scores one group of 4 consecutive logits (first index i, values v[4]).
  // IN_ORDER: the thread meets its indices in increasing order and logits past
  // the row's end hold -inf, so a strict "greater" keeps the first of equal
  // scores and never takes an index past the end (-inf / T + g is -inf, or
  // NaN on the multiply path, and neither beats the initial -inf).
  auto score_group = [&](auto fast, auto in_order, uint32_t i, const float (&v)[4], float T,
                         float rT) {
    uint32_t r[4] = {i >> 2, c1, c2, 0u};
    philox4x32_10(r, k0, k1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float s = div_t<decltype(fast)::value>(v[e], T, rT) + gumbel_of(r[e]);
      if constexpr (decltype(in_order)::value) {
        const bool take = s > bs;
        bs = take ? s : bs;
        bi = take ? i + e : bi;
      } else {
        consider(i + e < (uint32_t)V, s, i + e);
      }
    }
  };

  if (greedy) {
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      const int64_t i = index_of(j);
      consider(i < V, x[j], (uint32_t)i);
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
    if (total * 2 <= 64 * NG) {
      // few groups survive: compact them (first index of each) for sharing out
      int slot = incl - cnt;
#pragma unroll
      for (int g = 0; g < NG; ++g)
        if (gmask & (1u << g)) work[wave][slot++] = (int32_t)index_of(4 * g);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // 4. score the surviving groups, in place or from the compacted list.  The
    // multiply-and-correct division needs T in [2^-32, 2^32] and a chunk whose
    // largest logit is at most 2^64 in size: every quotient that can win then
    // stays finite (a logit below -2^96 may give NaN, which never wins, where
    // the quotient would be hugely negative and lose as well).
    auto run = [&](auto fast) {
      const float rT = 1.0f / T;
      if (total * 2 > 64 * NG) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          if (gmask & (1u << g)) {
            const float v[4] = {x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
            score_group(fast, std::true_type{}, (uint32_t)index_of(4 * g), v, T, rT);
          }
        }
      } else {
        for (int e = lane; e < total; e += 64) {
          const int64_t i = work[wave][e];
          float v[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = i + k < V ? load_logit(i + k) : -INFINITY;
          score_group(fast, std::false_type{}, (uint32_t)i, v, T, rT);
        }
      }
    };
    const bool fast_div = T >= 0x1p-32f && T <= 0x1p32f && fabsf(m) <= 0x1p64f;
    if (fast_div)
      run(std::true_type{});
    else
      run(std::false_type{});
  }
  uint64_t best = bi == 0xFFFFFFFFu ? 0ull : score_key(bs, bi);
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
  // key 0: no candidate at all (possible only with NaN logits); token 0
  if (threadIdx.x == 0) tokens[b] = best ? (int64_t)(0xFFFFFFFFu - (uint32_t)best) : 0;
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
