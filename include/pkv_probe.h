/*
 * libpkv_probe: measurement probes for MI355X (gfx950) that the benchmark
 * runs beside the attention kernels of libpkv.  They compute nothing of the
 * attention path; they measure what this device sustains with the same access
 * patterns and instructions, so the kernels' figures can be read against a
 * measured ceiling as well as against the published peaks.
 *
 * All pointers are device pointers the caller owns; every call is enqueued on
 * `stream` and returns at once.  Return codes are those of include/pkv.h
 * (0 = PKV_OK, 1 = PKV_EINVAL, 3 = PKV_ELAUNCH).
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Load-only pass over the K/V bytes a paged decode reads (devpress page,
 * "PagedAttention是如何实现的": the K/V rows of a sequence are found block by
 * block through its block table).  For every page p in [0, num_pages) and
 * every KV head h, rows 0 .. pages[2p+1]-1 of physical block pages[2p] are
 * read, head h only (d bf16 values of K and of V per row), in 16-token tiles
 * with 16-byte loads, exactly the bytes and the row pattern of the decode.
 * Nothing is computed from the data beyond an xor fold that decides whether
 * sink[0] is written (it practically never is), so no load can be dropped.
 *   k_cache, v_cache  [num_blocks, block_size, H_kv, d] bf16, 16-byte aligned
 *   pages             [num_pages][2] int32: physical block id, tokens used
 *                     (1 .. block_size); built on the host from the block
 *                     tables and context lengths.  An id outside
 *                     [0, num_blocks) reads nothing; token counts are clamped
 *                     to block_size
 *   sink              one uint32
 *   nontemporal       nonzero: the loads carry the non-temporal hint, as the
 *                     decode's K/V loads do
 *   group_heads       0: one workgroup of 64 lanes per (page, head), the
 *                     decode's pattern; nonzero: one workgroup of H_kv
 *                     wavefronts per page, one head each, so the heads of the
 *                     same token rows are read by one CU together
 * PKV_EINVAL: null pointers, num_pages < 1, num_blocks < 1, H_kv < 1, d not
 * 64 or 128, block_size not a power of two >= 16, misaligned caches,
 * group_heads with H_kv > 16.
 */
int pkv_probe_paged_read(const void* k_cache, const void* v_cache, const int32_t* pages,
                         int32_t num_pages, int32_t num_blocks, int32_t H_kv, int32_t d,
                         int32_t block_size, uint32_t* sink, int32_t nontemporal,
                         int32_t group_heads, hipStream_t stream);

/*
 * Plain streaming read of `bytes` bytes (a multiple of 16, 16-byte aligned
 * src) with 16-byte loads, xor-folded as above: one workgroup of 256 lanes
 * per contiguous 256 KiB chunk, eight loads per lane in flight; with the
 * non-temporal hint when `nontemporal` is nonzero.
 */
int pkv_probe_read(const void* src, int64_t bytes, uint32_t* sink, int32_t nontemporal,
                   hipStream_t stream);

/*
 * Plain device copy of `bytes` bytes (a multiple of 16; both pointers 16-byte
 * aligned) with 16-byte loads and stores, chunked as the read: the known-size
 * kernel that scales the FETCH_SIZE / WRITE_SIZE counters, and a copy ceiling.
 */
int pkv_probe_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);

/*
 * Dense bf16 MFMA issue rate: every wavefront runs `iters` rounds of
 * `chains` independent v_mfma_f32_32x32x16_bf16 (fp16 when use_f16 != 0)
 * on register operands (32*32*16*2 = 32768 flops each), with no memory
 * traffic but one fp32 per wavefront written to sink at the end.
 * waves_per_simd wavefronts per SIMD (1 .. 8), 4 SIMDs per compute unit,
 * one workgroup of 4 wavefronts per compute unit and unit of waves_per_simd.
 * Flops per call = num_cus * 4 * waves_per_simd * iters * chains * 32768.
 *   sink    [num_cus * 4 * waves_per_simd] fp32
 *   chains  1, 2, 4 or 8
 */
int pkv_probe_mfma(float* sink, int32_t num_cus, int32_t waves_per_simd, int32_t iters,
                   int32_t chains, int32_t use_f16, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
