// Varlen causal prefill over the paged KV cache on MFMA.
//
// What is computed (devpress "nano-vllm解读", "如何适配不同请求不同序列长度";
// AIInfraGuide 3.6, section 2): sequence b has nq new queries and nk keys,
// c = nk - nq of them cached; query i sits at position c + i and attends keys
// 0 .. c + i of the sequence, read through its block table.  Grouped-query:
// query head h reads KV head h / G.
//
// How (MI355X, gfx950): a dense contraction, so both products run on MFMA
// (v_mfma_f32_32x32x16_bf16, bf16 in, fp32 accumulate):
//  - a workgroup (4 wavefronts) owns one KV head, one sequence and a tile of
//    query positions; its M dimension packs (query position, head of the
//    group) pairs, 32 per wavefront, so all G heads share every K/V tile.
//    (8 wavefronts share each tile between twice the rows but run slower:
//    the per-tile barrier then keeps both wavefronts of a SIMD in the same
//    phase, while two 4-wavefront workgroups per CU drift apart and overlap
//    one's softmax with the other's MFMAs.  Two groups of 4 run half a tile
//    apart with a barrier per half tile ran slower still);
//  - K/V tiles of 64 keys are gathered through the block table (one look-up
//    per tile when a tile lies inside one block, per row otherwise, so any
//    power-of-two block size works) into LDS, double-buffered, the next tile's
//    global loads all in flight while the current tile computes.
//    Rows are stored with a 16-byte-chunk XOR swizzle chosen so that both
//    the K operand reads (one row per lane) and the V transpose reads (four
//    rows per 16 lanes) hit distinct banks;
//  - S^T = K Q^T puts keys on the MFMA M side and the packed query rows on N,
//    so every lane ends up owning scores of a single query row: the softmax
//    statistics are per lane (plus one exchange with lane l^32);
//  - O^T += V^T P^T: the P operand is the lane's own scores, rounded to fp16
//    (bf16 would leave outputs of magnitude 2..4 close to the 1e-2 error
//    bar), and the V^T operand comes straight from the row-major V tile, kept
//    in LDS as fp16 (exact for bf16 values of normal fp16 range), with
//    ds_read_b64_tr_b16, which transposes 4x16 blocks of 16-bit elements.
//    A workgroup whose rows show that V left fp16's range (a non-finite row,
//    or a row whose outputs are all tiny) runs its tiles again with V in bf16
//    and P as bf16 high and low parts, so every finite bf16 V is served;
//  - online softmax in the log2 domain with the same lazy rescale as decode;
//    only tiles that cross the diagonal are masked;
//  - grid (KV head, query tile, sequence), so the dispatch order is sequence
//    by sequence and, within one, the last (most expensive, causally longest)
//    query tile first.  Workgroups run on XCD (linear id mod 8), so with 8 KV
//    heads every XCD serves one head, and the workgroups it runs at a time
//    are the query tiles of a few sequences, which stream the same K/V tiles
//    at about the same time: those hit in the XCD's L2.  (Query tile
//    outermost spread each XCD over every sequence at once and fetched about
//    13 times the K/V bytes from HBM.)
#include <type_traits>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kPrefillBN = 64;     // keys per tile
constexpr int kPrefillWaves = 4;   // wavefronts per workgroup, 32 packed query rows each
constexpr float kPrefillLazy = 8.0f;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 8 bf16 -> 8 fp16 (round to nearest even).  V tiles are kept in LDS as fp16
// so that P can be rounded to fp16 (8x finer than bf16) for the PV product.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 w) {
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f16x2 h = {(_Float16)bf16_lo(w[k]), (_Float16)bf16_hi(w[k])};
    r[k] = __builtin_bit_cast(uint32_t, h);
  }
  return r;
}

__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}

// 16-byte chunk swizzle of the K/V tiles in LDS (a row is d bf16 = CPR chunks).
// gfx950 serves 16 lanes of 16-byte reads and 32 lanes of 8-byte reads per LDS
// cycle over 64 four-byte banks.  With these XOR patterns (checked with the
// SQ_LDS_BANK_CONFLICT counter) neither the K operand reads (one row per lane,
// 16 consecutive rows on one chunk) nor the V transpose reads (4 consecutive
// rows x 4 chunks per 32 lanes) nor the tile stores conflict.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CPR >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// PAGED: keys come from the paged cache through block_tables (k_cache/v_cache
// [num_blocks, block_size, H_kv, d]).  Otherwise (the no-prefix form of the
// devpress page's varlen call) keys of sequence b are the token rows
// cu_k[b] .. cu_k[b+1]-1 of packed K/V [total_k, H_kv, d]; num_blocks then
// carries total_k, and block_tables, bs_log2 and maxb are unused.  q, k and v
// rows are q_stride / k_stride / v_stride elements apart (views of a fused
// projection), heads and d contiguous.
template <int D, int G, int NWV, bool PAGED>
__global__ __launch_bounds__(64 * NWV, 8 / NWV) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, uint16_t* __restrict__ out,
    int32_t total_q, int32_t H_kv, int32_t num_blocks, int32_t bs_log2, int32_t maxb,
    int64_t q_stride, int64_t k_stride, int64_t v_stride, float scale_log2e) {
  constexpr int BN = kPrefillBN;
  constexpr int NT = 64 * NWV;         // threads per workgroup
  constexpr int QPW = 32 / G;          // query positions per wavefront
  constexpr int QPB = NWV * QPW;       // query positions per workgroup
  constexpr int KS = D / 16;           // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;           // 32-wide d blocks of O^T
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int RPP = NT / CPR;        // rows per load pass (a multiple of 16)
  constexpr int PASSES = BN / RPP;     // load passes per tile and tensor
  constexpr int TILE = BN * D;         // elements per K (or V) tile

  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * TILE];  // [buf][K|V][BN][D]

  const int h_kv = blockIdx.x;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int lane = tid & 63;
  const int H_q = H_kv * G;

  const int qs = cu_q[b];
  const int nq = cu_q[b + 1] - qs;
  const int cap = PAGED ? (maxb << bs_log2) : num_blocks;
  int nk = cu_k[b + 1] - cu_k[b];
  nk = nk > cap ? cap : nk;
  const int kb0 = PAGED ? 0 : cu_k[b];  // packed: first key row of the sequence
  if (nq <= 0 || nk < nq || qs < 0) return;
  const int c = nk - nq;
  const int nqt = (nq + QPB - 1) / QPB;
  const int qt = nqt - 1 - (int)blockIdx.y;
  if (qt < 0) return;
  const int q0 = qt * QPB;
  const int kend = min(nk, c + q0 + QPB);
  const int ntiles = (kend + BN - 1) / BN;

  // this lane's query row (one of the 32 packed rows of the wavefront)
  const int mrow = lane & 31;
  const int half = lane >> 5;
  const int qq = q0 + wave * QPW + mrow / G;
  const int head = h_kv * G + (mrow % G);
  const bool row_ok = qq < nq && (int64_t)qs + qq < total_q;
  const int qpos = c + qq;
  const int wave_first_pos = c + q0 + wave * QPW;
  const int wave_last_pos = wave_first_pos + QPW - 1;

  bf16x8 qf[KS];
  {
    const uint16_t* qp = q + ((int64_t)qs + qq) * q_stride + (int64_t)head * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = row_ok ? ld16(qp + 16 * ks) : u32x4{0, 0, 0, 0};
      // wait for q here, once: otherwise the wait-count pass cannot tell
      // inside the tile loop that these loads are done, and makes the first
      // score MFMA of every tile wait for the next tile's K/V loads as well
      asm volatile("" : "+v"(v));
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = kNegSentinel;
  float l = 0.f;

  // ---- per-lane offsets, computed once -------------------------------------
  // cooperative tile loader: thread -> (chunk ch, rows r0 + RPP * p)
  const int ch = tid % CPR;
  const int r0 = tid / CPR;
  const int64_t row_stride = k_stride;  // elements between K token rows (paged: == v_stride)
  const int64_t goff = r0 * row_stride + ch * 8;  // element offset of this thread's first row
  const int64_t goff_v = r0 * v_stride + ch * 8;
  // the same in bytes, and the bytes between load passes, for the buffer loads
  // of whole tiles (a tile spans less than 2^31 bytes from its first row)
  const int32_t goff_b = (int32_t)(goff * 2);
  const int32_t goff_vb = (int32_t)(goff_v * 2);
  const int32_t pass_kb = (int32_t)(RPP * row_stride * 2);
  const int32_t pass_vb = (int32_t)(RPP * v_stride * 2);
  // the LDS slot of this thread's chunk; rows r0 + RPP * p share their low four bits
  const int soff = r0 * D + ((ch ^ swz<CPR>(r0)) << 3);
  // K operand reads: row kb * 32 + mrow, logical chunk 2 * ks + half.  The row
  // base is a multiple of the row size, so the swizzled chunk is one XOR away:
  // element offset = kbase_lane ^ (16 * ks).
  const int kbase_lane = mrow * D + ((half ^ swz<CPR>(mrow)) << 3);
  // V^T operand reads: rows kb * 32 + 16 * s2 + rlo (+ 8), 4 columns at col
  const int i16 = lane & 15;
  const int grp16 = lane >> 4;
  // d block db's chunk is block 0's chunk XOR 4 * db (the swizzle changes
  // only a row's low chunk bits within each group of four), so its offset is
  // voff[hi] ^ (32 * db)
  int voff[2];
  {
    const int col = 16 * (grp16 & 1) + 4 * (i16 & 3);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int rlo = 4 * half + (i16 >> 2) + 8 * hi;
      voff[hi] = rlo * D + (((col >> 3) ^ swz<CPR>(rlo)) << 3) + (col & 7);
    }
  }
  const uint16_t* khead = k_cache + (int64_t)h_kv * D;
  const uint16_t* vhead = v_cache + (int64_t)h_kv * D;
  const int32_t* table = block_tables + (int64_t)b * maxb;
  const int bmask = (1 << bs_log2) - 1;

  u32x4 kr[PASSES], vr[PASSES];
  bool kok[PASSES];
  bool full_next = true;  // the tile in kr/vr needs no zeroing
  // Issues every global load of tile kt before any wait.  When a tile lies
  // inside one block (block size >= 64) its base is one scalar look-up and the
  // rows are fixed offsets from it; otherwise each row is looked up (all
  // look-ups first).  Rows past the keys this workgroup needs, or behind an
  // out-of-range block id, read valid memory and are zeroed when stashed.
  const bool tile_in_block = bs_log2 >= 6;
  // Whole tile from its first K and V rows: buffer loads whose base (a
  // scalar resource) moves per tile while the lane and pass offsets stay
  // fixed, so no 64-bit address is computed per load.
  auto load_rows = [&](const uint16_t* kb, const uint16_t* vb) {
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kb), (short)0,
                                                      0x7FFFFFFF, 0x00020000);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vb), (short)0,
                                                      0x7FFFFFFF, 0x00020000);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      kr[p] = __builtin_amdgcn_raw_buffer_load_b128(rk, goff_b, p * pass_kb, 0);
      vr[p] = __builtin_amdgcn_raw_buffer_load_b128(rv, goff_vb, p * pass_vb, 0);
    }
  };
  auto load_tile = [&](int kt) {
    if constexpr (!PAGED) {
      // consecutive token rows; rows past kend re-read the last key (zeroed when stashed)
      // (rows are also kept inside [0, total_k) whatever cu_k holds)
      const int j0 = kt * BN;
      if (j0 + BN <= kend && kb0 >= 0 && (int64_t)kb0 + j0 + BN <= num_blocks) {
        load_rows(khead + ((int64_t)kb0 + j0) * k_stride, vhead + ((int64_t)kb0 + j0) * v_stride);
#pragma unroll
        for (int p = 0; p < PASSES; ++p) kok[p] = true;
        full_next = true;
      } else {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
          const int j = j0 + r0 + RPP * p;
          kok[p] = j < kend;
          int64_t row = (int64_t)kb0 + (j < kend ? j : kend - 1);
          row = row < 0 ? 0 : (row >= num_blocks ? num_blocks - 1 : row);
          kr[p] = ld16(khead + row * k_stride + ch * 8);
          vr[p] = ld16(vhead + row * v_stride + ch * 8);
        }
        full_next = false;
      }
      return;
    }
    if (tile_in_block) {
      int blk = table[(kt * BN) >> bs_log2];  // kt * BN < kend: a valid entry
      const bool blk_ok = (unsigned)blk < (unsigned)num_blocks;
      blk = blk_ok ? blk : 0;
      const int64_t base = (((int64_t)blk << bs_log2) + ((kt * BN) & bmask)) * row_stride;
      load_rows(khead + base, vhead + base);
#pragma unroll
      for (int p = 0; p < PASSES; ++p) kok[p] = blk_ok && kt * BN + r0 + RPP * p < kend;
      full_next = blk_ok && kt * BN + BN <= kend;
    } else {
      int blk[PASSES];
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int j = kt * BN + r0 + RPP * p;
        blk[p] = j < kend ? table[j >> bs_log2] : 0;
      }
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int j = kt * BN + r0 + RPP * p;
        kok[p] = j < kend && (unsigned)blk[p] < (unsigned)num_blocks;
        const int64_t row = kok[p] ? (((int64_t)blk[p] << bs_log2) + (j & bmask)) : 0;
        kr[p] = ld16(khead + row * row_stride + ch * 8);
        vr[p] = ld16(vhead + row * v_stride + ch * 8);
      }
      full_next = false;
    }
  };
  // V goes to LDS as fp16 (the fast pass) or unchanged as bf16 (the exact pass).
  auto stash_tile = [&](uint16_t* kt_lds, uint16_t* vt_lds, auto exact_tag) {
    constexpr bool EXACT = decltype(exact_tag)::value;
    auto vconv = [](u32x4 w) { return EXACT ? w : bf16x8_to_f16x8(w); };
    if (full_next) {
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        *reinterpret_cast<u32x4*>(kt_lds + soff + RPP * p * D) = kr[p];
        *reinterpret_cast<u32x4*>(vt_lds + soff + RPP * p * D) = vconv(vr[p]);
      }
    } else {
      const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        *reinterpret_cast<u32x4*>(kt_lds + soff + RPP * p * D) = kok[p] ? kr[p] : zero;
        *reinterpret_cast<u32x4*>(vt_lds + soff + RPP * p * D) = kok[p] ? vconv(vr[p]) : zero;
      }
    }
  };

  // One 64-key tile in three parts: S^T = K Q^T (MFMA), the online softmax
  // (VALU; produces P in fp16), O^T += V^T P^T (MFMA).
  // The two 32-key halves are independent chains, interleaved.  The K reads
  // run up to four pairs ahead of their MFMAs (an LDS read takes longer than
  // the two MFMAs between a pair and the next): the first reads, then two
  // MFMAs and two reads at a time, then the remaining MFMAs.  Left to itself,
  // the compiler (at 254 registers) issued each read just one MFMA ahead.
  auto score_mfma = [&](const uint16_t* kt_lds, f32x16 (&sacc)[2]) {
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a =
            *reinterpret_cast<const u32x4*>(kt_lds + (kbase_lane ^ (16 * ks)) + kb * 32 * D);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[ks],
                                                           sacc[kb], 0, 0, 0);
      }
    constexpr int kReads = 2 * KS;                       // one per MFMA
    constexpr int kAhead = kReads < 8 ? kReads : 8;
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);  // DS reads
#pragma unroll
    for (int g = 0; g < (kReads - kAhead) / 2; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x8, 2, 0);    // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x8, kAhead, 0);
  };
  // Mask, running max and rescale of one tile's scores.  The fast pass
  // rescales lazily (P up to 2^8); the exact pass whenever the maximum grows
  // (P up to 1, so P * V stays within fp32 for every finite bf16 V).
  auto softmax_max = [&](int kt, f32x16 (&sacc)[2], float lazy) {
    // causal mask, only on tiles that reach past this wavefront's first position
    if (kt * BN + BN - 1 > wave_first_pos) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * BN + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key > qpos) sacc[kb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx *= scale_log2e;  // the scale is positive: max commutes with it
    mx = cross_reduce<32, true>(mx);  // with lane l ^ 32, on the VALU (v_permlane32_swap)
    if (__any(mx > m + lazy)) {
      const float mn = fmaxf(m, mx);
      const float alpha = fast_exp2(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
  };
  auto softmax = [&](int kt, f32x16 (&sacc)[2], f16x8 (&pf)[2][2]) {
    softmax_max(kt, sacc, kPrefillLazy);
    // P = 2^(s * scale * log2 e - m) (at most 2^8 with the lazy rescale),
    // rounded to fp16 for the PV product
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(__builtin_fmaf(sacc[kb][8 * s2 + e], scale_log2e, -m));
          l += p;
          pf[kb][s2][e] = (_Float16)p;
        }
  };
  auto softmax_exact = [&](int kt, f32x16 (&sacc)[2]) {
    softmax_max(kt, sacc, 0.0f);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(sacc[kb][r], scale_log2e, -m));
        l += p;
        sacc[kb][r] = p;  // kept in fp32 until the PV product splits it
      }
  };
  auto pv_mfma = [&](const uint16_t* vt_lds, const f16x8 (&pf)[2][2]) {
    // key slice outermost: the four d blocks' MFMAs of one slice are
    // independent, and each slice needs only its own 8 exponentials
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int rofs = (kb * 32 + 16 * s2) * D;
          const i16x4 va = lds_read_tr16(vt_lds + (voff[0] ^ (32 * db)) + rofs);
          const i16x4 vb = lds_read_tr16(vt_lds + (voff[1] ^ (32 * db)) + rofs);
          typedef short i16x8 __attribute__((ext_vector_type(8)));
          const i16x8 v8 = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, v8),
                                                         pf[kb][s2], o[db], 0, 0, 0);
        }
  };

  // The exact pass's PV product: V in bf16 as stored, P split into bf16 high
  // and low parts (P to about 2^-16 relative), two MFMAs per slice and block.
  auto pv_mfma_exact = [&](const uint16_t* vt_lds, const f32x16 (&pacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 ph, pl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = pacc[kb][8 * s2 + e];
          ph[e] = (__bf16)p;
          pl[e] = (__bf16)(p - (float)ph[e]);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int rofs = (kb * 32 + 16 * s2) * D;
          const i16x4 va = lds_read_tr16(vt_lds + (voff[0] ^ (32 * db)) + rofs);
          const i16x4 vb = lds_read_tr16(vt_lds + (voff[1] ^ (32 * db)) + rofs);
          typedef short i16x8 __attribute__((ext_vector_type(8)));
          const i16x8 v8 = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
          const bf16x8 vv = __builtin_bit_cast(bf16x8, v8);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, ph, o[db], 0, 0, 0);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pl, o[db], 0, 0, 0);
        }
      }
  };

  // Set when a fast pass produced a non-finite row of this workgroup.
  __shared__ int redo_exact;
  if (tid == 0) redo_exact = 0;  // ordered before the reads by the loop's barriers

  // Tile kt computes from LDS buffer kt & 1 and stages tile kt + 1 into the
  // other.  The loop runs two tiles per iteration so that each buffer's base
  // is a constant: the LDS operand addresses are then loop-invariant
  // registers plus immediate offsets.
  auto tile_step = [&](int kt, auto buf_tag, auto exact_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    constexpr bool EXACT = decltype(exact_tag)::value;
    uint16_t* cur = lds + BUF * 2 * TILE;
    uint16_t* nxt = lds + (1 - BUF) * 2 * TILE;
    const bool more = kt + 1 < ntiles;
    if (more) load_tile(kt + 1);
    // a tile wholly past this wavefront's last position is masked out for all
    // its rows: it would add nothing, so only the loading is shared
    if (kt * BN <= wave_last_pos) {
      f32x16 sacc[2];
      score_mfma(cur, sacc);
      if constexpr (EXACT) {
        softmax_exact(kt, sacc);
        pv_mfma_exact(cur + TILE, sacc);
      } else {
        f16x8 pf[2][2];
        softmax(kt, sacc, pf);
        pv_mfma(cur + TILE, pf);
      }
    }
    if (more) stash_tile(nxt, nxt + TILE, exact_tag);
    __syncthreads();
  };
  auto run_pass = [&](auto exact_tag) {
    load_tile(0);
    stash_tile(lds, lds + TILE, exact_tag);
    __syncthreads();
    for (int kt = 0; kt < ntiles; kt += 2) {
      tile_step(kt, std::integral_constant<int, 0>{}, exact_tag);
      if (kt + 1 < ntiles) tile_step(kt + 1, std::integral_constant<int, 1>{}, exact_tag);
    }
  };

  run_pass(std::false_type{});
  // The fast pass holds V in fp16.  Two cases need the exact pass instead:
  //  - a V value beyond fp16's range (|v| >= 2^16) becomes an fp16 infinity,
  //    and every row whose PV product met it ends non-finite (an infinity, or
  //    a NaN from an infinity times a zero weight);
  //  - V values below fp16's normal range (2^-14) keep an absolute error of
  //    up to 2^-25, which is below a bf16 output's rounding only while the
  //    row's largest output is at least about 2^-14.
  // If any row of the workgroup (which shares the tiles in LDS) has either,
  // the whole workgroup runs again exactly: V in bf16, P in two bf16 parts.
  // Checked once per row, after the tile loop.
  {
    float chk = l, amax = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        chk += o[db][r];
        amax = fmaxf(amax, fabsf(o[db][r]));
      }
    // the row's other half (d values and keys) sits in lane l ^ 32
    const float row_l = l + shfl_xor_f32(l, 32);
    const float row_amax = fmaxf(amax, shfl_xor_f32(amax, 32));
    const bool small = row_ok && !(row_amax >= 0x1p-14f * row_l);
    if (__any(!__builtin_isfinite(chk) || small) && lane == 0) redo_exact = 1;
    __syncthreads();
    if (redo_exact) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = f32x16{};
      m = kNegSentinel;
      l = 0.f;
      run_pass(std::true_type{});
    }
  }

  l += shfl_xor_f32(l, 32);
  if (!row_ok) return;
  const float inv = 1.0f / l;
  uint16_t* op = out + (((int64_t)qs + qq) * H_q + head) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = db * 32 + 8 * r4 + 4 * half;
      u32x2 w;
      w[0] = pack_bf16x2(o[db][4 * r4 + 0] * inv, o[db][4 * r4 + 1] * inv);
      w[1] = pack_bf16x2(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv);
      *reinterpret_cast<u32x2*>(op + d0) = w;
    }
  }
}

template <int D, int G, bool PAGED>
static void launch_pf(dim3 grid, hipStream_t st, const uint16_t* q, const uint16_t* kc,
                      const uint16_t* vc, const int32_t* bt, const int32_t* cq, const int32_t* ck,
                      uint16_t* out, int32_t total_q, int32_t H_kv, int32_t nb, int32_t bsl,
                      int32_t maxb, int64_t qs, int64_t ks, int64_t vs, float sl2e) {
  hipLaunchKernelGGL((prefill_kernel<D, G, kPrefillWaves, PAGED>), grid, dim3(64 * kPrefillWaves), 0,
                     st, q, kc, vc, bt, cq, ck, out, total_q, H_kv, nb, bsl, maxb, qs, ks, vs, sl2e);
}

template <bool PAGED>
static hipError_t launch_prefill_any(uint16_t* out, const uint16_t* q, const uint16_t* k,
                                     const uint16_t* v, const int32_t* block_tables,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     int32_t B, int32_t total_q, int32_t max_seqlen_q, int32_t H_q,
                                     int32_t H_kv, int32_t d, int32_t num_blocks, int32_t bsl,
                                     int32_t maxb, int64_t qs, int64_t ks, int64_t vs,
                                     float softmax_scale, hipStream_t stream) {
  const int G = H_q / H_kv;
  const unsigned zt = (unsigned)prefill_query_tiles(max_seqlen_q, G);
  dim3 grid((unsigned)H_kv, zt, (unsigned)B);
  const float sl2e = softmax_scale * 1.4426950408889634f;
#define PKV_PF(DD, GG)                                                                        \
  launch_pf<DD, GG, PAGED>(grid, stream, q, k, v, block_tables, cu_seqlens_q, cu_seqlens_k, out, \
                           total_q, H_kv, num_blocks, bsl, maxb, qs, ks, vs, sl2e)
  if (d == 128) {
    switch (G) {
      case 1: PKV_PF(128, 1); break;
      case 2: PKV_PF(128, 2); break;
      case 4: PKV_PF(128, 4); break;
      case 8: PKV_PF(128, 8); break;
    }
  } else {
    switch (G) {
      case 1: PKV_PF(64, 1); break;
      case 2: PKV_PF(64, 2); break;
      case 4: PKV_PF(64, 4); break;
      case 8: PKV_PF(64, 8); break;
    }
  }
#undef PKV_PF
  return hipGetLastError();
}

int64_t prefill_query_tiles(int32_t max_seqlen_q, int32_t G) {
  const int64_t qpb = kPrefillWaves * (32 / G);
  return ((int64_t)max_seqlen_q + qpb - 1) / qpb;
}

static int ilog2p(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

hipError_t launch_prefill(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                          const uint16_t* v_cache, const int32_t* block_tables,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t B,
                          int32_t total_q, int32_t max_seqlen_q, int32_t H_q, int32_t H_kv,
                          int32_t d, int32_t num_blocks, int32_t block_size,
                          int32_t max_blocks_per_seq, float softmax_scale, hipStream_t stream) {
  const int64_t row = (int64_t)H_kv * d;
  return launch_prefill_any<true>(out, q, k_cache, v_cache, block_tables, cu_seqlens_q,
                                  cu_seqlens_k, B, total_q, max_seqlen_q, H_q, H_kv, d,
                                  num_blocks, ilog2p(block_size), max_blocks_per_seq,
                                  (int64_t)H_q * d, row, row, softmax_scale, stream);
}

hipError_t launch_prefill_packed(uint16_t* out, const uint16_t* q, int64_t q_stride,
                                 const uint16_t* k, int64_t k_stride, const uint16_t* v,
                                 int64_t v_stride, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int32_t B, int32_t total_q,
                                 int32_t total_k, int32_t max_seqlen_q, int32_t H_q, int32_t H_kv,
                                 int32_t d, float softmax_scale, hipStream_t stream) {
  return launch_prefill_any<false>(out, q, k, v, nullptr, cu_seqlens_q, cu_seqlens_k, B, total_q,
                                   max_seqlen_q, H_q, H_kv, d, total_k, 0, 0, q_stride, k_stride,
                                   v_stride, softmax_scale, stream);
}

}  // namespace pkv
