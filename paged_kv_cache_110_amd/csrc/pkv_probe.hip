// Measurement probes (include/pkv_probe.h): a load-only pass over the decode's
// paged K/V rows, a plain streaming read and copy, and a register-only MFMA
// loop.  Built into libpkv_probe.so, apart from the attention library.  The
// two reads take the load instruction's non-temporal hint as an option (the
// decode streams its K/V with it).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "pkv_probe.h"

namespace {

using pkv::bf16x8;
using pkv::f32x16;
using pkv::ld16;
using pkv::ld16_stream;
using pkv::u32x4;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr uint32_t kNever = 0x9e3779b9u;  // the fold practically never equals it

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

template <bool NT>
__device__ __forceinline__ u32x4 load16(const void* p) {
  if constexpr (NT) return ld16_stream(p);
  else return ld16(p);
}

// One wavefront per (page, KV head): the page's used rows of that head, K and
// V, two 16-token tiles per round.  A row of one head is d bf16 = d/8 lanes of
// 16 bytes, so one load instruction covers 64 / (d/8) rows.
template <int D, bool NT>
__global__ __launch_bounds__(1024) void paged_read_kernel(const uint16_t* __restrict__ k_cache,
                                                        const uint16_t* __restrict__ v_cache,
                                                        const int32_t* __restrict__ pages,
                                                        int32_t num_blocks, int32_t H_kv,
                                                        int32_t block_size,
                                                        uint32_t* __restrict__ sink) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  constexpr int kLoadsPerTile = 16 / kRowsPerLoad;
  // one wavefront per (page, head); a workgroup holds one of them, or all
  // H_kv heads of one page (then they read the page's rows together)
  const int unit = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int page = unit / H_kv;
  const int h = unit - page * H_kv;
  const int32_t block = pages[2 * page];
  const int32_t used = min(pages[2 * page + 1], block_size);
  if (block < 0 || block >= num_blocks) return;  // a bad entry reads nothing
  const int lane = threadIdx.x & 63;
  const int r0 = lane / kLanesPerRow;
  const int64_t row = (int64_t)H_kv * D;
  const int64_t base = (int64_t)block * block_size * row + h * D + (lane % kLanesPerRow) * 8;
  const uint16_t* kb = k_cache + base;
  const uint16_t* vb = v_cache + base;
  uint32_t acc = 0;
  int t = 0;
  for (; t + 32 <= used; t += 32) {  // whole rounds: no per-row test
    u32x4 kr[2 * kLoadsPerTile], vr[2 * kLoadsPerTile];
#pragma unroll
    for (int i = 0; i < 2 * kLoadsPerTile; ++i) {
      const int tok = t + i * kRowsPerLoad + r0;
      kr[i] = load16<NT>(kb + tok * row);
      vr[i] = load16<NT>(vb + tok * row);
    }
#pragma unroll
    for (int i = 0; i < 2 * kLoadsPerTile; ++i) acc ^= fold(kr[i]) ^ fold(vr[i]);
  }
  for (int tok = t + r0; tok < used; tok += kRowsPerLoad)  // the page's last rows
    acc ^= fold(load16<NT>(kb + tok * row)) ^ fold(load16<NT>(vb + tok * row));
  if (acc == kNever) sink[0] = acc;
}

// Each workgroup streams one contiguous 256 KiB chunk (the last one may be
// shorter), eight 16-byte loads per lane in flight: the fastest of the plain
// patterns measured on this device (grid-stride loops ran 3-10% slower).
constexpr int64_t kChunk16 = (256 << 10) / 16;  // 16-byte units per chunk

template <bool NT>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * kChunk16;
  const int64_t end = min(base + kChunk16, n16);
  uint32_t acc = 0;
  int64_t i = base + threadIdx.x;
  for (; i + 7 * 256 < end; i += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = load16<NT>(&src[i + k * 256]);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= fold(v[k]);
  }
  for (; i < end; i += 256) acc ^= fold(load16<NT>(&src[i]));
  if (acc == kNever) sink[0] = acc;
}

__global__ __launch_bounds__(256) void copy_kernel(u32x4* __restrict__ dst,
                                                   const u32x4* __restrict__ src, int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * kChunk16;
  const int64_t end = min(base + kChunk16, n16);
  int64_t i = base + threadIdx.x;
  for (; i + 7 * 256 < end; i += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = src[i + k * 256];
#pragma unroll
    for (int k = 0; k < 8; ++k) dst[i + k * 256] = v[k];
  }
  for (; i < end; i += 256) dst[i] = src[i];
}

// CH independent accumulator chains of 32x32x16 MFMAs on register operands.
template <int CH, bool F16>
__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ sink, int32_t iters) {
  const int lane = threadIdx.x & 63;
  u32x4 bits;
#pragma unroll
  for (int e = 0; e < 4; ++e) bits[e] = 0x3c003c00u ^ (uint32_t)((lane * 4 + e) & 0x3ff);
  f32x16 acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if constexpr (F16)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, bits),
                                                        __builtin_bit_cast(f16x8, bits), acc[c],
                                                        0, 0, 0);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bits),
                                                         __builtin_bit_cast(bf16x8, bits), acc[c],
                                                         0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if (lane == 0) sink[(int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int status(hipError_t e) { return e == hipSuccess ? 0 : 3; }

template <int CH>
void launch_mfma(dim3 grid, float* sink, int32_t iters, bool f16, hipStream_t stream) {
  if (f16)
    hipLaunchKernelGGL((mfma_kernel<CH, true>), grid, dim3(256), 0, stream, sink, iters);
  else
    hipLaunchKernelGGL((mfma_kernel<CH, false>), grid, dim3(256), 0, stream, sink, iters);
}

}  // namespace

extern "C" {

int pkv_probe_paged_read(const void* k_cache, const void* v_cache, const int32_t* pages,
                         int32_t num_pages, int32_t num_blocks, int32_t H_kv, int32_t d,
                         int32_t block_size, uint32_t* sink, int32_t nontemporal,
                         int32_t group_heads, hipStream_t stream) {
  if (!k_cache || !v_cache || !pages || !sink || num_pages < 1 || num_blocks < 1 || H_kv < 1)
    return 1;
  if (group_heads && H_kv > 16) return 1;
  if (d != 64 && d != 128) return 1;
  if (block_size < 16 || (block_size & (block_size - 1))) return 1;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return 1;
  if ((int64_t)num_pages * H_kv > INT32_MAX) return 1;
  const dim3 grid((unsigned)(group_heads ? num_pages : num_pages * H_kv));
  const dim3 block(group_heads ? 64 * H_kv : 64);
  const auto* kc = static_cast<const uint16_t*>(k_cache);
  const auto* vc = static_cast<const uint16_t*>(v_cache);
  const bool nt = nontemporal != 0;
  if (d == 128 && nt)
    hipLaunchKernelGGL((paged_read_kernel<128, true>), grid, block, 0, stream, kc, vc, pages,
                       num_blocks, H_kv, block_size, sink);
  else if (d == 128)
    hipLaunchKernelGGL((paged_read_kernel<128, false>), grid, block, 0, stream, kc, vc, pages,
                       num_blocks, H_kv, block_size, sink);
  else if (nt)
    hipLaunchKernelGGL((paged_read_kernel<64, true>), grid, block, 0, stream, kc, vc, pages,
                       num_blocks, H_kv, block_size, sink);
  else
    hipLaunchKernelGGL((paged_read_kernel<64, false>), grid, block, 0, stream, kc, vc, pages,
                       num_blocks, H_kv, block_size, sink);
  return status(hipGetLastError());
}

int pkv_probe_read(const void* src, int64_t bytes, uint32_t* sink, int32_t nontemporal,
                   hipStream_t stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 || !aligned16(src)) return 1;
  const int64_t chunks = (bytes / 16 + kChunk16 - 1) / kChunk16;
  if (chunks > INT32_MAX) return 1;
  if (nontemporal)
    hipLaunchKernelGGL(read_kernel<true>, dim3((unsigned)chunks), dim3(256), 0, stream,
                       static_cast<const u32x4*>(src), bytes / 16, sink);
  else
    hipLaunchKernelGGL(read_kernel<false>, dim3((unsigned)chunks), dim3(256), 0, stream,
                       static_cast<const u32x4*>(src), bytes / 16, sink);
  return status(hipGetLastError());
}

int pkv_probe_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  if (!src || !dst || bytes < 16 || bytes % 16 || !aligned16(src) || !aligned16(dst)) return 1;
  const int64_t chunks = (bytes / 16 + kChunk16 - 1) / kChunk16;
  if (chunks > INT32_MAX) return 1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)chunks), dim3(256), 0, stream,
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), bytes / 16);
  return status(hipGetLastError());
}

int pkv_probe_mfma(float* sink, int32_t num_cus, int32_t waves_per_simd, int32_t iters,
                   int32_t chains, int32_t use_f16, hipStream_t stream) {
  if (!sink || num_cus < 1 || waves_per_simd < 1 || waves_per_simd > 8 || iters < 1) return 1;
  const dim3 grid((unsigned)(num_cus * waves_per_simd));
  const bool f16 = use_f16 != 0;
  switch (chains) {
    case 1: launch_mfma<1>(grid, sink, iters, f16, stream); break;
    case 2: launch_mfma<2>(grid, sink, iters, f16, stream); break;
    case 4: launch_mfma<4>(grid, sink, iters, f16, stream); break;
    case 8: launch_mfma<8>(grid, sink, iters, f16, stream); break;
    default: return 1;
  }
  return status(hipGetLastError());
}

}  // extern "C"
