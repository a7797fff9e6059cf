// Paged GQA decode attention: a persistent, load-balanced split over the KV
// sequence, then a log-sum-exp merge of the pieces.
//
// What is computed (devpress "nano-vllm解读", "PagedAttention是如何实现的";
// AIInfraGuide 3.6, section 2): for each sequence b and query head h,
//   out[b,h] = softmax_j(q[b,h] . K_b[j] * scale) V_b[j],  j < context_lens[b],
// with key j read from row j % block_size of physical block
// block_tables[b][j / block_size], KV head h / G.
//
// How (MI355X).  Decode is HBM-bound (about G flop per byte of K/V), so the
// kernel is organised around streaming K/V at full bandwidth until the very
// end of the call, not around MFMA:
//  - work is the flattened list of 16-token tiles of every (sequence, KV head)
//    segment.  Exactly one wavefront is launched per resident slot of the GPU,
//    and each takes an equal contiguous share of that list, so every slot
//    streams for the same time and the call ends sharply (with one wavefront
//    per fixed-size split instead, the last round of wavefronts runs on a
//    partly empty GPU);
//  - 16 divides every supported block size and tiles start at multiples of 16,
//    so a tile never crosses a page (the devpress page's point about read
//    lengths dividing the block size): its physical block id is one scalar load
//    and its rows are 16 contiguous token rows of one block;
//  - each token's head vector (d bf16) is spread over LPT = d / EPL lanes, as
//    128-bit words interleaved across the lanes so every load instruction
//    covers whole 128-byte lines; loads go straight to registers (nothing is
//    shared between lanes, so LDS staging would only add a round trip);
//  - a ring of NBUF register buffers keeps NBUF - 1 tiles in flight, also
//    across segment boundaries.  The ring loop is straight-line (every step
//    issues its loads; steps past the end re-read the last tile with zero
//    weight), so the compiler's wait counts track the ring exactly;
//  - q.k uses v_dot2_f32_bf16 on packed bf16 pairs (exact products, fp32
//    sums), reduced across the LPT lanes of a token with DPP;
//  - online softmax (ascendai overview, "FlashAttention 集成": running max and
//    sum, rescaled output) per lane group, in the log2 domain with
//    scale*log2(e) folded in; the rescale is lazy (only when some lane's tile
//    maximum exceeds its running maximum by more than 2^8), exact math;
//  - a segment that lies inside one wavefront's share is finished in place and
//    written as bf16.  Only a wavefront's first and last segment can straddle
//    wavefronts: those write an fp32 partial (m, l, acc[d]) to one of the
//    wavefront's two partial slots, and decode_merge_kernel combines them.
#include <stdlib.h>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kDecodeTile = 16;       // tokens per tile; divides every supported block size
constexpr float kLazyRescale = 8.0f;  // log2 headroom before the running max is updated
constexpr int kMinTilesPerWave = 32;  // a wavefront streams at least 512 tokens of one head

// Where the partials of one (sequence, KV head) segment live: the wavefronts
// w_first .. w_first + nparts - 1 hold one piece each, in partial slot
// `slot_first` for the first of them and slot 0 for the others.
struct SegInfo {
  int32_t nparts;
  int32_t w_first;
  int32_t slot_first;
  int32_t pad;
};

__device__ __forceinline__ int64_t wave_sum_i64(int64_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ int64_t wave_incl_scan_i64(int64_t x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

template <int D, int G, int EPL, int NBUF>
__global__ __launch_bounds__(64) void decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, uint16_t* __restrict__ out,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, SegInfo* __restrict__ ws_seg,
    int32_t B, int32_t H_kv, int32_t num_blocks, int32_t bs_log2, int32_t maxb,
    float scale_log2e) {
  constexpr int LPT = D / EPL;           // lanes per token
  constexpr int TPI = 64 / LPT;          // tokens side by side in a wave
  constexpr int TPL = kDecodeTile / TPI; // tokens per lane per tile
  constexpr int NW = EPL / 8;            // 128-bit words per lane per row
  static_assert(TPI * TPL == kDecodeTile, "tile shape");

  const int lane = threadIdx.x;
  const int grp = lane / LPT;
  const int sub = lane % LPT;
  // Lane `sub` of a token holds the 8-element words w = 0..NW-1 at d offsets
  // w * 8 * LPT + 8 * sub: one 128-bit load instruction of the LPT lanes then
  // covers 8 * LPT contiguous elements (a whole 128-byte line for LPT = 8).
  auto dofs = [&](int w) { return w * 8 * LPT + 8 * sub; };
  const int H_q = H_kv * G;
  const int cap = maxb << bs_log2;
  const int bmask = (1 << bs_log2) - 1;
  const int rs = H_kv * D;  // elements between consecutive token rows
  const int64_t W = gridDim.x;
  const int64_t wv = blockIdx.x;

  auto clamp_len = [&](int len) { return len < 0 ? 0 : (len > cap ? cap : len); };

  // ---- this wavefront's share of the flattened tile list -----------------
  // Units are (sequence, KV head, 16-token tile); sequence b owns
  // H_kv * ceil(len_b / 16) consecutive units, KV heads in order.
  constexpr int kCachedChunks = 8;  // tile counts of the first 512 sequences stay in registers
  int cnt[kCachedChunks];
  int64_t part = 0;
#pragma unroll
  for (int c = 0; c < kCachedChunks; ++c) {
    const int b = c * 64 + lane;
    cnt[c] = b < B ? (clamp_len(context_lens[b]) + kDecodeTile - 1) / kDecodeTile : 0;
    part += cnt[c];
  }
  for (int b0 = kCachedChunks * 64; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    if (b < B) part += (clamp_len(context_lens[b]) + kDecodeTile - 1) / kDecodeTile;
  }
  const int64_t total = wave_sum_i64(part) * H_kv;
  int64_t U = (total + W - 1) / W;
  U = U < kMinTilesPerWave ? kMinTilesPerWave : U;
  const int64_t start = wv * U;
  if (start >= total) return;
  const int64_t end = start + U < total ? start + U : total;

  // sequence holding `start`, and the units before it
  int sb = 0;
  int64_t sb_base = 0;
  {
    int64_t run = 0;
    for (int b0 = 0, c = 0; b0 < B; b0 += 64, ++c) {
      const int b = b0 + lane;
      int nt = 0;
      if (c < kCachedChunks) {
#pragma unroll
        for (int k = 0; k < kCachedChunks; ++k)
          if (k == c) nt = cnt[k];
      } else if (b < B) {
        nt = (clamp_len(context_lens[b]) + kDecodeTile - 1) / kDecodeTile;
      }
      const int64_t n = (int64_t)nt * H_kv;
      const int64_t incl = wave_incl_scan_i64(n, lane) + run;
      const int64_t excl = incl - n;
      const unsigned long long hit = __ballot(n > 0 && excl <= start && start < incl);
      if (hit) {
        const int idx = __ffsll((long long)hit) - 1;
        sb = b0 + idx;
        sb_base = __shfl(excl, idx, 64);
        break;
      }
      run = __shfl(incl, 63, 64);
    }
  }

  // A cursor walks the units in order: sequence b (length len, nt tiles),
  // KV head h, tile j; base = units before sequence b.  All wave-uniform.
  struct Cursor {
    int b, h, j, nt, len;
    int64_t base;
  };
  auto make_cursor = [&]() {
    Cursor c;
    c.b = sb;
    c.len = clamp_len(context_lens[sb]);
    c.nt = (c.len + kDecodeTile - 1) / kDecodeTile;
    c.base = sb_base;
    const int64_t off = start - sb_base;
    c.h = (int)(off / c.nt);
    c.j = (int)(off - (int64_t)c.h * c.nt);
    return c;
  };
  auto advance = [&](Cursor& c) {
    if (++c.j < c.nt) return;
    c.j = 0;
    if (++c.h < H_kv) return;
    c.h = 0;
    c.base += (int64_t)c.nt * H_kv;
    do {  // skip empty sequences; never runs past the last unit of the call
      ++c.b;
      c.len = clamp_len(context_lens[c.b]);
      c.nt = (c.len + kDecodeTile - 1) / kDecodeTile;
    } while (c.nt == 0 && c.b + 1 < B);
  };

  // ---- the tile ring -------------------------------------------------------
  const int64_t R = end - start;  // tiles this wavefront computes
  Cursor L = make_cursor();       // load cursor, NBUF - 1 tiles ahead
  Cursor C = L;                   // compute cursor
  int64_t lstep = 0;

  // q of the next segment is loaded by the load cursor when it enters that
  // segment, so starting the segment does not drain the tile ring.  One
  // buffer: if it is still taken when another segment starts (segments of
  // fewer than NBUF - 1 tiles), that segment loads its q when it starts.
  uint32_t qn[G][EPL / 2];
  int64_t qn_seg = -1;  // flattened (sequence, KV head) index held in qn, -1 = free
  auto load_q = [&](int b, int h, uint32_t (&dst)[G][EPL / 2]) {
    const int64_t head0 = (int64_t)b * H_q + (int64_t)h * G;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const u32x4 v = ld16(q + (head0 + g) * D + dofs(w));
        dst[g][4 * w + 0] = v[0];
        dst[g][4 * w + 1] = v[1];
        dst[g][4 * w + 2] = v[2];
        dst[g][4 * w + 3] = v[3];
      }
    }
  };

  // Loads the tile under the load cursor, then moves the cursor on (while it
  // has tiles left; past the end it stays on the last tile, whose re-read is
  // an L2 hit, and the tile is marked empty).
  auto load_tile = [&](u32x4 (&kx)[TPL][NW], u32x4 (&vx)[TPL][NW], bool (&ok)[TPL]) {
    const bool real = lstep < R;
    if (real && lstep > 0 && L.j == 0 && qn_seg < 0) {
      load_q(L.b, L.h, qn);
      qn_seg = (int64_t)L.b * H_kv + L.h;
    }
    const int t = L.j * kDecodeTile;
    int blk = block_tables[(int64_t)L.b * maxb + (t >> bs_log2)];
    const bool blk_ok = real && (unsigned)blk < (unsigned)num_blocks;
    blk = (unsigned)blk < (unsigned)num_blocks ? blk : 0;
    const int64_t row0 = ((int64_t)blk << bs_log2) + (t & bmask);
    const uint16_t* kt = k_cache + row0 * rs + (int64_t)L.h * D;
    const uint16_t* vt = v_cache + row0 * rs + (int64_t)L.h * D;
    const int last = L.len - 1 - t;
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const int r = grp + i * TPI;
      ok[i] = blk_ok && r <= last;
      const int off = (r <= last ? r : last) * rs;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        kx[i][w] = ld16(kt + off + dofs(w));
        vx[i][w] = ld16(vt + off + dofs(w));
      }
    }
    if (lstep + 1 < R) advance(L);
    ++lstep;
  };

  uint32_t qw[G][EPL / 2];
  float acc[G][EPL];
  float m[G], l[G];

  auto begin_segment = [&]() {
    if (qn_seg == (int64_t)C.b * H_kv + C.h) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < EPL / 2; ++k) qw[g][k] = qn[g][k];
      qn_seg = -1;
    } else {
      load_q(C.b, C.h, qw);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = kNegSentinel;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }
  };

  auto compute_tile = [&](const u32x4 (&kx)[TPL][NW], const u32x4 (&vx)[TPL][NW],
                          const bool (&ok)[TPL]) {
    // scores in the log2 domain
    float sc[TPL][G];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float dsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          dsum = dot2_bf16(qw[g][4 * w + 0], kx[i][w][0], dsum);
          dsum = dot2_bf16(qw[g][4 * w + 1], kx[i][w][1], dsum);
          dsum = dot2_bf16(qw[g][4 * w + 2], kx[i][w][2], dsum);
          dsum = dot2_bf16(qw[g][4 * w + 3], kx[i][w][3], dsum);
        }
        dsum = group_sum<LPT>(dsum);
        sc[i][g] = ok[i] ? dsum * scale_log2e : -INFINITY;
      }
    }
    // lazy running-max update
    bool need = false;
    float mt[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      mt[g] = sc[0][g];
#pragma unroll
      for (int i = 1; i < TPL; ++i) mt[g] = fmaxf(mt[g], sc[i][g]);
      need |= mt[g] > m[g] + kLazyRescale;
    }
    if (__any(need)) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mn = fmaxf(m[g], mt[g]);
        const float alpha = fast_exp2(m[g] - mn);
        m[g] = mn;
        l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
      }
    }
    // weights and weighted V
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      float p[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        p[g] = fast_exp2(sc[i][g] - m[g]);
        l[g] += p[g];
      }
#pragma unroll
      for (int w = 0; w < NW; ++w) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float v0 = bf16_lo(vx[i][w][k]);
          const float v1 = bf16_hi(vx[i][w][k]);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            acc[g][8 * w + 2 * k] += p[g] * v0;
            acc[g][8 * w + 2 * k + 1] += p[g] * v1;
          }
        }
      }
    }
  };

  bool first_segment = true;
  auto end_segment = [&]() {
    // merge the TPI lane groups (log-sum-exp); group 0 holds the result
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float M = m[g];
#pragma unroll
      for (int off = LPT; off < 64; off <<= 1) M = fmaxf(M, shfl_xor_f32(M, off));
      const float alpha = fast_exp2(m[g] - M);
      float lg = l[g] * alpha;
#pragma unroll
      for (int off = LPT; off < 64; off <<= 1) lg += shfl_xor_f32(lg, off);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float a = acc[g][e] * alpha;
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) a += shfl_xor_f32(a, off);
        acc[g][e] = a;
      }
      m[g] = M;
      l[g] = lg;
    }
    const int64_t seg_start = C.base + (int64_t)C.h * C.nt;
    const int64_t w_first = seg_start / U;
    const int nparts = (int)((seg_start + C.nt - 1) / U - w_first + 1);
    const int slot = first_segment ? 0 : 1;
    if (wv == w_first && lane == 0)
      ws_seg[(int64_t)C.b * H_kv + C.h] = SegInfo{nparts, (int32_t)w_first, slot, 0};
    first_segment = false;
    if (grp != 0) return;
    const int64_t head0 = (int64_t)C.b * H_q + (int64_t)C.h * G;
    if (nparts == 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float inv = 1.0f / l[g];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          u32x4 o;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            o[k] = pack_bf16x2(acc[g][8 * w + 2 * k] * inv, acc[g][8 * w + 2 * k + 1] * inv);
          st16(out + (head0 + g) * D + dofs(w), o);
        }
      }
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int64_t row = (wv * 2 + slot) * G + g;
        float* ap = ws_acc + row * D;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          *reinterpret_cast<f32x4*>(ap + dofs(w)) =
              f32x4{acc[g][8 * w], acc[g][8 * w + 1], acc[g][8 * w + 2], acc[g][8 * w + 3]};
          *reinterpret_cast<f32x4*>(ap + dofs(w) + 4) =
              f32x4{acc[g][8 * w + 4], acc[g][8 * w + 5], acc[g][8 * w + 6], acc[g][8 * w + 7]};
        }
        if (sub == 0) *reinterpret_cast<float2*>(ws_ml + row * 2) = make_float2(m[g], l[g]);
      }
    }
  };

  // Ring of NBUF register buffers; the loop is unrolled NBUF times so every
  // buffer index is a compile-time constant (no register copies).
  u32x4 kbuf[NBUF][TPL][NW], vbuf[NBUF][TPL][NW];
  bool okbuf[NBUF][TPL];
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i) load_tile(kbuf[i], vbuf[i], okbuf[i]);
  int64_t cstep = 0;
  const int64_t niter = (R + NBUF - 1) / NBUF;
  for (int64_t it = 0; it < niter; ++it) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int nxt = (u + NBUF - 1) % NBUF;
      load_tile(kbuf[nxt], vbuf[nxt], okbuf[nxt]);
      if (cstep < R) {
        if (cstep == 0 || C.j == 0) begin_segment();
        compute_tile(kbuf[u], vbuf[u], okbuf[u]);
        if (cstep + 1 == R || C.j + 1 == C.nt) end_segment();
        if (cstep + 1 < R) advance(C);
      }
      ++cstep;
    }
  }
}

// Combine the pieces of one (sequence, query head) whose segment straddled
// wavefronts: M = max_p m_p, L = sum_p l_p 2^(m_p - M),
// out = sum_p acc_p 2^(m_p - M) / L, pieces in wavefront order (deterministic).
// Rows of empty sequences are written as zeros here.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
    const SegInfo* __restrict__ ws_seg, const int32_t* __restrict__ context_lens,
    uint16_t* __restrict__ out, int32_t B, int32_t H_q, int32_t G) {
  constexpr int EPT = D / 64;
  const int lane = threadIdx.x % 64;
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;  // b * H_q + h
  if (row >= (int64_t)B * H_q) return;
  const int b = (int)(row / H_q);
  const int hq = (int)(row - (int64_t)b * H_q);
  uint16_t* op = out + row * D + lane * EPT;
  if (context_lens[b] <= 0) {
    if constexpr (EPT == 2) *reinterpret_cast<uint32_t*>(op) = 0u;
    else *op = 0;
    return;
  }
  const int H_kv = H_q / G;
  const SegInfo info = ws_seg[(int64_t)b * H_kv + hq / G];
  if (info.nparts <= 1) return;  // written directly by the decode kernel
  const int g = hq % G;
  auto piece = [&](int p) -> int64_t {
    const int64_t wave = (int64_t)info.w_first + p;
    const int slot = p == 0 ? info.slot_first : 0;
    return (wave * 2 + slot) * G + g;
  };

  float M = -INFINITY;
  for (int p0 = 0; p0 < info.nparts; p0 += 64)
    if (p0 + lane < info.nparts) M = fmaxf(M, ws_ml[2 * piece(p0 + lane)]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, shfl_xor_f32(M, off));

  float L = 0.f;
  float o[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) o[e] = 0.f;
  for (int p0 = 0; p0 < info.nparts; p0 += 64) {
    float w = 0.f;
    if (p0 + lane < info.nparts) {
      const float2 st = *reinterpret_cast<const float2*>(ws_ml + 2 * piece(p0 + lane));
      w = fast_exp2(st.x - M);
      L += st.y * w;
    }
    const int cnt = min(64, info.nparts - p0);
#pragma unroll 8
    for (int j = 0; j < cnt; ++j) {
      const float wj =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
      const float* src = ws_acc + piece(p0 + j) * D + lane * EPT;
#pragma unroll
      for (int e = 0; e < EPT; ++e) o[e] += src[e] * wj;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) L += shfl_xor_f32(L, off);
  const float inv = 1.0f / L;
  if constexpr (EPT == 2) {
    *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(o[0] * inv, o[1] * inv);
  } else {
    const uint32_t pk = pack_bf16x2(o[0] * inv, 0.f);
    *op = (uint16_t)(pk & 0xffffu);
  }
}

// ----------------------------------------------------------------- host side

static int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

// One wavefront per resident slot of the current device (cached per device
// and kernel variant).
template <int D, int G, int EPL, int NBUF>
static int resident_waves() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<D, G, EPL, NBUF>, 64,
                                                     0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 8;
    cached[dev] = cus * per_cu;
  }
  return cached[dev];
}

// Kernel variant per (d, G): elements per lane and ring depth.
template <typename F>
static bool dispatch(int d, int G, F& f) {
  if (d == 128) {
    switch (G) {
      case 1: f.template run<128, 1, 16, 3>(); return true;
      case 2: f.template run<128, 2, 16, 3>(); return true;
      case 4: f.template run<128, 4, 8, 3>(); return true;
      case 8: f.template run<128, 8, 8, 2>(); return true;
    }
  } else if (d == 64) {
    switch (G) {
      case 1: f.template run<64, 1, 8, 3>(); return true;
      case 2: f.template run<64, 2, 8, 3>(); return true;
      case 4: f.template run<64, 4, 8, 3>(); return true;
      case 8: f.template run<64, 8, 8, 2>(); return true;
    }
  }
  return false;
}

struct WaveQuery {
  int waves = 0;
  template <int D, int G, int EPL, int NBUF>
  void run() { waves = resident_waves<D, G, EPL, NBUF>(); }
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

DecodePlan decode_plan(int32_t B, int32_t H_q, int32_t H_kv, int32_t d, int32_t block_size,
                       int32_t max_blocks_per_seq) {
  (void)block_size;
  (void)max_blocks_per_seq;
  DecodePlan p{0, 0};
  const int G = H_q / H_kv;
  WaveQuery wq;
  if (!dispatch(d, G, wq)) return p;
  p.num_waves = wq.waves;
  const size_t rows = (size_t)wq.waves * 2 * G;  // two partial slots per wavefront
  p.workspace_bytes = align256(rows * d * sizeof(float)) + align256(rows * 2 * sizeof(float)) +
                      (size_t)B * H_kv * sizeof(SegInfo);
  return p;
}

struct DecodeLaunch {
  dim3 grid;
  hipStream_t st;
  const uint16_t *q, *kc, *vc;
  const int32_t *bt, *cl;
  uint16_t* out;
  float *wa, *wm;
  SegInfo* wseg;
  int32_t B, H_kv, nb, bsl, maxb;
  float sl2e;
  template <int D, int G, int EPL, int NBUF>
  void run() {
    hipLaunchKernelGGL((decode_kernel<D, G, EPL, NBUF>), grid, dim3(64), 0, st, q, kc, vc, bt, cl,
                       out, wa, wm, wseg, B, H_kv, nb, bsl, maxb, sl2e);
  }
};

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int32_t B, int32_t H_q, int32_t H_kv,
                         int32_t d, int32_t num_blocks, int32_t block_size,
                         int32_t max_blocks_per_seq, float softmax_scale, void* workspace,
                         const DecodePlan& plan, hipStream_t stream) {
  const int G = H_q / H_kv;
  const size_t rows = (size_t)plan.num_waves * 2 * G;
  char* ws = static_cast<char*>(workspace);
  float* wa = reinterpret_cast<float*>(ws);
  float* wm = reinterpret_cast<float*>(ws + align256(rows * d * sizeof(float)));
  SegInfo* wseg = reinterpret_cast<SegInfo*>(ws + align256(rows * d * sizeof(float)) +
                                             align256(rows * 2 * sizeof(float)));
  DecodeLaunch lf{dim3((unsigned)plan.num_waves), stream, q, k_cache, v_cache, block_tables,
                  context_lens, out, wa, wm, wseg, B, H_kv, num_blocks, ilog2(block_size),
                  max_blocks_per_seq, softmax_scale * 1.4426950408889634f};
  if (!dispatch(d, G, lf)) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nrows = (int64_t)B * H_q;
  dim3 mgrid((unsigned)((nrows + 3) / 4));
  if (d == 128)
    hipLaunchKernelGGL(decode_merge_kernel<128>, mgrid, dim3(256), 0, stream, wa, wm, wseg,
                       context_lens, out, B, H_q, G);
  else
    hipLaunchKernelGGL(decode_merge_kernel<64>, mgrid, dim3(256), 0, stream, wa, wm, wseg,
                       context_lens, out, B, H_q, G);
  return hipGetLastError();
}

}  // namespace pkv
