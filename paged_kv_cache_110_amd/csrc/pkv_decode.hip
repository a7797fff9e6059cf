// Paged GQA decode attention with split-K over the KV sequence.
//
// What is computed (devpress "nano-vllm解读", "PagedAttention是如何实现的";
// AIInfraGuide 3.6, section 2): for each sequence b and query head h,
//   out[b,h] = softmax_j(q[b,h] . K_b[j] * scale) V_b[j],  j < context_lens[b],
// with key j read from row j % block_size of physical block
// block_tables[b][j / block_size], KV head h / G.
//
// How (MI355X): decode is HBM-bound (about G flop per byte of K/V), so the
// kernel is built around keeping enough bytes in flight, not around MFMA:
//  - one wavefront per (sequence, KV head, split); the G query heads that
//    share the KV head are processed together so every K/V byte is read once;
//  - a tile is 16 tokens.  16 divides every supported block size, and tiles
//    start at multiples of 16, so a tile never crosses a page (the devpress
//    page's observation about read lengths that divide the block size): the
//    tile's physical block id is one scalar load and its rows are 16
//    contiguous token rows of one block;
//  - each token's head vector (d bf16) is spread over LPT = d / EPL lanes,
//    each lane loading EPL contiguous elements with 128-bit loads straight into
//    registers (no LDS round trip: nothing is shared between lanes).  The next
//    tile's loads are issued before the current tile is computed;
//  - q.k uses v_dot2_f32_bf16 on packed bf16 pairs (exact products, fp32
//    sums), reduced across the LPT lanes of a token with DPP;
//  - online softmax (ascendai overview, "FlashAttention 集成": running max and
//    sum, rescaled output) is kept per lane group, in the log2 domain with
//    scale*log2(e) folded into the score; the rescale is lazy: it runs only
//    when some lane's tile maximum exceeds its running maximum by more than
//    2^8, which keeps every weight <= 256 and leaves the math exact;
//  - at the end of the split the lane groups are merged with the same
//    log-sum-exp rule, and the split either writes the bf16 output (one split)
//    or an fp32 partial (m, l, acc[d]) that decode_merge_kernel combines.
#include <stdlib.h>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kDecodeTile = 16;  // tokens per tile; divides every supported block size
constexpr float kLazyRescale = 8.0f;  // log2 headroom before the running max is updated

template <int D, int G, int EPL>
__global__ __launch_bounds__(64) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, uint16_t* __restrict__ out,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, int32_t H_kv, int32_t num_blocks,
    int32_t bs_log2, int32_t maxb, int32_t split_tokens, int32_t num_splits, float scale_log2e) {
  constexpr int LPT = D / EPL;           // lanes per token
  constexpr int TPI = 64 / LPT;          // tokens side by side in a wave
  constexpr int TPL = kDecodeTile / TPI; // tokens per lane per tile
  constexpr int NW = EPL / 8;            // 128-bit words per lane per row
  static_assert(TPI * TPL == kDecodeTile, "tile shape");

  const int lane = threadIdx.x;
  const int grp = lane / LPT;
  const int sub = lane % LPT;
  const int h = blockIdx.x % H_kv;
  const int b = blockIdx.x / H_kv;
  const int s = blockIdx.y;
  const int H_q = H_kv * G;
  const int cap = maxb << bs_log2;
  int len = context_lens[b];
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int64_t head0 = (int64_t)b * H_q + (int64_t)h * G;  // first query head row

  if (len == 0) {  // nothing to attend to: the defined output is zero
    if (s == 0 && grp == 0) {
      for (int g = 0; g < G; ++g)
        for (int w = 0; w < NW; ++w) st16(out + (head0 + g) * D + sub * EPL + 8 * w, u32x4{0, 0, 0, 0});
    }
    return;
  }
  const int t0 = s * split_tokens;
  if (t0 >= len) return;
  const int t1 = min(t0 + split_tokens, len);
  const int nsplit = (len + split_tokens - 1) / split_tokens;

  // query heads of this KV group, EPL elements each, as packed bf16 pairs
  uint32_t qw[G][EPL / 2];
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      u32x4 v = ld16(q + (head0 + g) * D + sub * EPL + 8 * w);
      qw[g][4 * w + 0] = v[0];
      qw[g][4 * w + 1] = v[1];
      qw[g][4 * w + 2] = v[2];
      qw[g][4 * w + 3] = v[3];
    }
  }

  float acc[G][EPL];
  float m[G], l[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegSentinel;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  const int rs = H_kv * D;  // elements between consecutive token rows
  const uint16_t* kbase = k_cache + (int64_t)h * D;  // wave-uniform bases
  const uint16_t* vbase = v_cache + (int64_t)h * D;
  const int32_t* table = block_tables + (int64_t)b * maxb;
  const int bmask = (1 << bs_log2) - 1;

  // Loads one tile.  Every load is unconditional: in the last, partial tile the
  // rows past the end re-read the last valid row (finite data) and get weight 0
  // through ok[] = false, so no lane ever touches a row outside the sequence.
  auto load_tile = [&](int t, u32x4 (&kx)[TPL][NW], u32x4 (&vx)[TPL][NW], bool (&ok)[TPL]) {
    int blk = table[t >> bs_log2];
    const bool blk_ok = (unsigned)blk < (unsigned)num_blocks;
    blk = blk_ok ? blk : 0;
    const int64_t row0 = ((int64_t)blk << bs_log2) + (t & bmask);
    const uint16_t* kt = kbase + row0 * rs;
    const uint16_t* vt = vbase + row0 * rs;
    const int last = t1 - 1 - t;
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const int r = grp + i * TPI;
      ok[i] = blk_ok && r <= last;
      const int off = (r <= last ? r : last) * rs + sub * EPL;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        kx[i][w] = ld16(kt + off + 8 * w);
        vx[i][w] = ld16(vt + off + 8 * w);
      }
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

  // two register buffers in ping-pong: the next tile's loads are in flight
  // while the current tile is computed, with no register copies
  u32x4 ka[TPL][NW], va[TPL][NW], kb2[TPL][NW], vb2[TPL][NW];
  bool oka[TPL], okb[TPL];
  load_tile(t0, ka, va, oka);
  for (int t = t0; t < t1; t += 2 * kDecodeTile) {
    const bool has_b = t + kDecodeTile < t1;
    if (has_b) load_tile(t + kDecodeTile, kb2, vb2, okb);
    compute_tile(ka, va, oka);
    if (!has_b) break;
    if (t + 2 * kDecodeTile < t1) load_tile(t + 2 * kDecodeTile, ka, va, oka);
    compute_tile(kb2, vb2, okb);
  }

  // merge the TPI lane groups (log-sum-exp), result in group 0
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

  if (grp != 0) return;
  if (nsplit == 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float inv = 1.0f / l[g];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          o[k] = pack_bf16x2(acc[g][8 * w + 2 * k] * inv, acc[g][8 * w + 2 * k + 1] * inv);
        st16(out + (head0 + g) * D + sub * EPL + 8 * w, o);
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t row = (head0 + g) * num_splits + s;
      float* ap = ws_acc + row * D + sub * EPL;
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<f32x4*>(ap + e) = f32x4{acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]};
      if (sub == 0) *reinterpret_cast<float2*>(ws_ml + row * 2) = make_float2(m[g], l[g]);
    }
  }
}

// Combine the split partials of one (sequence, query head) per wavefront:
// M = max_s m_s, L = sum_s l_s 2^(m_s - M), out = sum_s acc_s 2^(m_s - M) / L.
// Splits are visited in ascending order, so results are deterministic.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ context_lens, uint16_t* __restrict__ out, int32_t B, int32_t H_q,
    int32_t cap, int32_t split_tokens, int32_t num_splits) {
  constexpr int EPT = D / 64;
  const int lane = threadIdx.x % 64;
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;  // b * H_q + h
  if (row >= (int64_t)B * H_q) return;
  const int b = (int)(row / H_q);
  int len = context_lens[b];
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int nsplit = (len + split_tokens - 1) / split_tokens;
  if (nsplit <= 1) return;  // written directly by the split kernel
  const float* ml = ws_ml + row * num_splits * 2;
  const float* ap = ws_acc + row * num_splits * D + lane * EPT;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f;
  float o[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) o[e] = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float w = fast_exp2(ml[2 * s] - M);
    L += ml[2 * s + 1] * w;
#pragma unroll
    for (int e = 0; e < EPT; ++e) o[e] += ap[(int64_t)s * D + e] * w;
  }
  const float inv = 1.0f / L;
  uint16_t* op = out + row * D + lane * EPT;
  if constexpr (EPT == 2) {
    *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(o[0] * inv, o[1] * inv);
  } else {
    const uint32_t pk = pack_bf16x2(o[0] * inv, 0.f);
    *op = (uint16_t)(pk & 0xffffu);
  }
}

static int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

DecodePlan decode_plan(int32_t B, int32_t H_q, int32_t H_kv, int32_t d, int32_t block_size,
                       int32_t max_blocks_per_seq) {
  DecodePlan p{kDecodeTile, 0, 0};
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  int64_t split = cap <= 4096 ? 256 : 512;
  if (const char* env = getenv("PKV_DECODE_SPLIT")) {  // tuning override, tokens
    const long v = strtol(env, nullptr, 10);
    if (v > 0) split = v;
  }
  split = (split + kDecodeTile - 1) / kDecodeTile * kDecodeTile;
  if (cap > 0 && split > cap) split = (cap + kDecodeTile - 1) / kDecodeTile * kDecodeTile;
  p.split_tokens = (int32_t)split;
  p.num_splits = cap > 0 ? (int32_t)((cap + split - 1) / split) : 0;
  if (p.num_splits > 1) {
    const size_t rows = (size_t)B * H_q * p.num_splits;
    const size_t acc = (rows * d * sizeof(float) + 255) / 256 * 256;
    p.workspace_bytes = acc + rows * 2 * sizeof(float);
  }
  return p;
}

template <int D, int G, int EPL>
static void launch_split(dim3 grid, hipStream_t stream, const uint16_t* q, const uint16_t* kc,
                         const uint16_t* vc, const int32_t* bt, const int32_t* cl, uint16_t* out,
                         float* wa, float* wm, int32_t H_kv, int32_t nb, int32_t bsl, int32_t maxb,
                         int32_t split, int32_t ns, float sl2e) {
  hipLaunchKernelGGL((decode_split_kernel<D, G, EPL>), grid, dim3(64), 0, stream, q, kc, vc, bt,
                     cl, out, wa, wm, H_kv, nb, bsl, maxb, split, ns, sl2e);
}

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int32_t B, int32_t H_q, int32_t H_kv,
                         int32_t d, int32_t num_blocks, int32_t block_size,
                         int32_t max_blocks_per_seq, float softmax_scale, void* workspace,
                         const DecodePlan& plan, hipStream_t stream) {
  const int G = H_q / H_kv;
  const int bsl = ilog2(block_size);
  const float sl2e = softmax_scale * 1.4426950408889634f;
  float* wa = nullptr;
  float* wm = nullptr;
  if (plan.num_splits > 1) {
    const size_t rows = (size_t)B * H_q * plan.num_splits;
    wa = static_cast<float*>(workspace);
    wm = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                  (rows * d * sizeof(float) + 255) / 256 * 256);
  }
  const int ns = plan.num_splits > 0 ? plan.num_splits : 1;
  dim3 grid((unsigned)(B * H_kv), (unsigned)ns);
#define PKV_SPLIT(DD, GG, EE)                                                                   \
  launch_split<DD, GG, EE>(grid, stream, q, k_cache, v_cache, block_tables, context_lens, out, \
                           wa, wm, H_kv, num_blocks, bsl, max_blocks_per_seq, plan.split_tokens, \
                           ns, sl2e)
  if (d == 128) {
    switch (G) {
      case 1: PKV_SPLIT(128, 1, 16); break;
      case 2: PKV_SPLIT(128, 2, 16); break;
      case 4: PKV_SPLIT(128, 4, 16); break;
      case 8: PKV_SPLIT(128, 8, 8); break;
    }
  } else {
    switch (G) {
      case 1: PKV_SPLIT(64, 1, 8); break;
      case 2: PKV_SPLIT(64, 2, 8); break;
      case 4: PKV_SPLIT(64, 4, 8); break;
      case 8: PKV_SPLIT(64, 8, 8); break;
    }
  }
#undef PKV_SPLIT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (plan.num_splits > 1) {
    const int64_t rows = (int64_t)B * H_q;
    dim3 mgrid((unsigned)((rows + 3) / 4));
    const int32_t cap = max_blocks_per_seq * block_size;
    if (d == 128)
      hipLaunchKernelGGL(decode_merge_kernel<128>, mgrid, dim3(256), 0, stream, wa, wm,
                         context_lens, out, B, H_q, cap, plan.split_tokens, plan.num_splits);
    else
      hipLaunchKernelGGL(decode_merge_kernel<64>, mgrid, dim3(256), 0, stream, wa, wm,
                         context_lens, out, B, H_q, cap, plan.split_tokens, plan.num_splits);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace pkv
