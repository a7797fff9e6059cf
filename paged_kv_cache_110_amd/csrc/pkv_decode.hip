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
//    segment.  Exactly one wavefront is launched per resident slot of the GPU.
//    Each first streams a static share of the list, then takes shrinking
//    shares from an atomic counter (decode_schedule.h): the two wavefronts of
//    a SIMD progress at very different rates, so equal static shares would
//    leave the call waiting for the slowest.  A small call (a few tiles per
//    wavefront) is one static pass spread over as many wavefronts as it fills;
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
//  - wide groups (G >= 4) take the MFMA form instead (MF): the VALU's q.k and
//    p.v work per byte of K/V grows with G (about 80 instructions per tile
//    and query head) and at G = 8 would outrun the HBM stream.  Each tile is
//    staged in LDS (swizzled 16-byte chunks), S^T = K Q^T runs on
//    v_mfma_f32_16x16x32_bf16 (16 keys x the G heads padded to 16 columns),
//    the online softmax on the four scores a lane holds, and O^T += V^T P^T
//    on v_mfma_f32_16x16x16_bf16 with V^T read transposed from LDS
//    (ds_read_b64_tr_b16) and P as bf16 high and low parts;
//  - online softmax (ascendai overview, "FlashAttention 集成": running max and
//    sum, rescaled output) per lane group, in the log2 domain with
//    scale*log2(e) folded in; the rescale is lazy (only when some lane's tile
//    maximum exceeds its running maximum by more than 2^8), exact math;
//  - a segment that lies inside one share is finished in place and written as
//    bf16.  A segment cut by share boundaries writes an fp32 partial
//    (m, l, acc[d]) per piece into its share's partial slots, and
//    decode_merge_kernel combines the pieces in share order;
//  - with the step's store fused in (FUSE, pkv_store_decode), the wavefront
//    that loads a segment's last tile takes the new token's row (and the
//    masked rows after it) from the new K/V input rather than the cache, and
//    writes that row into the cache before computing the tile.  No other tile
//    holds the row, so nothing else reads it, and the kernel never reads a
//    cache row it writes.
#include <limits.h>
#include <stdlib.h>

#include <type_traits>

#include "decode_schedule.h"
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kDecodeTile = 16;       // tokens per tile; divides every supported block size
constexpr float kLazyRescale = 8.0f;  // log2 headroom before the running max is updated
constexpr int kSeqCache = 512;        // sequences whose unit offsets are kept in LDS

// Where the partial results of one (sequence, KV head) segment live: it was
// cut into the shares k_first .. k_last, one piece each (k_first == k_last:
// one piece, written directly).
struct SegInfo {
  int32_t k_first;
  int32_t k_last;
  int32_t pad0, pad1;
};


// Inclusive prefix sum over the 64 lanes on DPP: shifts by 1, 2, 4 and 8
// within each row of 16 lanes, then each row adds the last lane of the rows
// before it (row_bcast:15, then row_bcast:31).  Lanes a shift would read from
// outside their row add 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Unit counts fit in int32: the host rejects shapes where
// B * H_kv * ceil(max_blocks_per_seq * block_size / 16) could exceed INT32_MAX.
template <int D, int G, int EPL, int NBUF, int WPE, bool MF, bool FUSE>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(WPE))) void decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, uint16_t* __restrict__ out,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, SegInfo* __restrict__ ws_seg,
    int32_t* __restrict__ queue, int32_t B, int32_t H_kv, int32_t num_blocks, int32_t bs_log2,
    int32_t maxb, float scale_log2e, NewToken nt_in) {
  constexpr int LPT = D / EPL;           // lanes per token
  constexpr int TPI = 64 / LPT;          // tokens side by side in a wave
  constexpr int TPL = kDecodeTile / TPI; // tokens per lane per tile
  constexpr int NW = EPL / 8;            // 128-bit words per lane per row
  static_assert(TPI * TPL == kDecodeTile, "tile shape");
  static_assert(!MF || (NW == 1 && G <= 16), "MFMA form: one 128-bit word per lane and row");

  __shared__ int pre[kSeqCache + 1];  // units of the sequences before b
  __shared__ int lenc[kSeqCache];     // clamped context length of b
  // fused store: whether sequence b's new token lies inside its table
  // (context_lens[b] <= the table's capacity); a clamped length stores nothing
  __shared__ int8_t newok[FUSE ? kSeqCache : 1];
  // MFMA form: the tile being computed, K then V, 16 rows of D bf16 each with
  // swizzled 16-byte chunks (mf_off)
  __shared__ __attribute__((aligned(16))) uint16_t kv_lds[MF ? 2 * kDecodeTile * D : 8];

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
  const int W = gridDim.x;
  const int wv = blockIdx.x;

  auto clamp_len = [&](int len) { return len < 0 ? 0 : (len > cap ? cap : len); };
  auto tiles_of = [&](int len) { return (clamp_len(len) + kDecodeTile - 1) / kDecodeTile; };

  // ---- unit offsets of the sequences -----------------------------------
  // Units are (sequence, KV head, 16-token tile); sequence b owns
  // H_kv * ceil(len_b / 16) consecutive units, KV heads in order.
  const int nb_cached = B < kSeqCache ? B : kSeqCache;
  int T = 0;
  {
    constexpr int kChunks = kSeqCache / 64;
    int cnt[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int b = c * 64 + lane;
      int len;
      if constexpr (FUSE) {
        const int raw = b < B ? context_lens[b] : 0;
        len = clamp_len(raw);
        newok[c * 64 + lane] = raw <= cap;
      } else {
        len = b < B ? clamp_len(context_lens[b]) : 0;
      }
      lenc[c * 64 + lane] = len;
      cnt[c] = (len + kDecodeTile - 1) / kDecodeTile;
    }
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      if (c * 64 < B) {
        const int n = cnt[c] * H_kv;
        const int incl = wave_incl_scan(n) + T;
        pre[c * 64 + lane] = incl - n;
        T = uniform(__shfl(incl, 63, 64));
      } else {
        pre[c * 64 + lane] = T;  // no sequences here: the offsets stay at T
      }
    }
    if (lane == 0) pre[kSeqCache] = T;
    for (int b0 = kSeqCache; b0 < B; b0 += 64) {
      const int b = b0 + lane;
      const int n = b < B ? tiles_of(context_lens[b]) * H_kv : 0;
      T += uniform(__shfl(wave_incl_scan(n), 63, 64));
    }
  }

  __syncthreads();
  // pre[] is read back with relaxed atomic loads: they stay LDS reads and are
  // not hoisted into registers that would stay live across the tile loop.
  auto pre_at = [&](int i) {
    return __hip_atomic_load(&pre[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  // clamped length of sequence b (from LDS for the first kSeqCache sequences)
  auto len_of = [&](int b) {
    return b < kSeqCache
               ? uniform(__hip_atomic_load(&lenc[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))
               : clamp_len(context_lens[b]);
  };
  const int T_cached = uniform(pre_at(nb_cached));

  // ---- share layout (see decode_schedule.h) ---------------------------------
  // Divisions run on the vector ALU: pin every result that addresses memory
  // to scalar registers, so block-table reads stay scalar loads instead of
  // vector loads whose wait would drain the tile ring.
  ShareSchedule sch = ShareSchedule::make(T, W, MF);
  sch.S0 = uniform(sch.S0);
  sch.P1 = uniform(sch.P1);
  sch.S1 = uniform(sch.S1);
  const bool dynamic = sch.dynamic();
  const int num_shares = sch.num_shares();

  // A cursor walks units in order: sequence b (length len, nt tiles), KV head
  // h, tile j; base = units before sequence b; u = the unit; [us, ue) = the
  // share being walked, k its index.  All wave-uniform.
  struct Cursor {
    int b, h, j, nt, len, base, u, us, ue, k;
  };
  // Position a cursor on unit u (< T): the last sequence whose offset is <= u.
  auto locate = [&](Cursor& c, int u) {
    int b = 0, base = 0;
    if (u < T_cached) {
      constexpr int kStride = kSeqCache / 64;
      const int i0 = lane * kStride;
      const bool hit0 = i0 < nb_cached && pre_at(i0 < nb_cached ? i0 : 0) <= u;
      const int c0 = 63 - __clzll(__ballot(hit0));
      const int i1 = c0 * kStride + lane;
      const bool hit1 = lane < kStride && i1 < nb_cached && pre_at(i1 < nb_cached ? i1 : 0) <= u;
      b = c0 * kStride + (63 - __clzll(__ballot(hit1)));
      base = uniform(pre_at(b));
    } else {
      int run = T_cached;
      for (int b0 = kSeqCache; b0 < B; b0 += 64) {
        const int bb = b0 + lane;
        const int n = bb < B ? tiles_of(context_lens[bb]) * H_kv : 0;
        const int incl = wave_incl_scan(n) + run;
        const int excl = incl - n;
        const unsigned long long hit = __ballot(n > 0 && excl <= u && u < incl);
        if (hit) {
          const int idx = __ffsll((long long)hit) - 1;
          b = b0 + idx;
          base = uniform(__shfl(excl, idx, 64));
          break;
        }
        run = uniform(__shfl(incl, 63, 64));
      }
    }
    c.b = uniform(b);
    c.len = len_of(c.b);
    c.nt = (c.len + kDecodeTile - 1) / kDecodeTile;
    c.base = base;
    const int off = u - base;
    c.h = uniform(off / c.nt);
    c.j = off - c.h * c.nt;
    c.u = u;
  };
  auto pin = [&](Cursor& c) {  // keep the cursor in scalar registers
    c.b = uniform(c.b);
    c.h = uniform(c.h);
    c.j = uniform(c.j);
    c.nt = uniform(c.nt);
    c.len = uniform(c.len);
    c.base = uniform(c.base);
    c.u = uniform(c.u);
    c.us = uniform(c.us);
    c.ue = uniform(c.ue);
    c.k = uniform(c.k);
  };
  auto step_unit = [&](Cursor& c) {  // next unit inside the share
    ++c.u;
    if (++c.j < c.nt) return;
    c.j = 0;
    if (++c.h < H_kv) return;
    c.h = 0;
    c.base += c.nt * H_kv;
    do {  // skip empty sequences; never runs past the last unit of the call
      ++c.b;
      c.len = len_of(c.b);
      c.nt = (c.len + kDecodeTile - 1) / kDecodeTile;
    } while (c.nt == 0 && c.b + 1 < B);
  };

  // The next dynamic share is requested in the step that loads the second-to-
  // last tile of the current one, before that step's tile loads, and read
  // after the computation of the following step: by then every load issued
  // before the request has been waited for anyway, so reading the counter
  // costs no extra wait.
  // Lane 0 of grab[i]: value the counter returned for a request made while
  // loading ring slot i (one register per slot, so the read one step later is
  // known not to race a request of its own step).
  int grab[NBUF];
#pragma unroll
  for (int i = 0; i < NBUF; ++i) grab[i] = 0;
  bool switch_pending = false;

  Cursor L;  // load cursor, NBUF - 1 tiles ahead of the computation
  sch.range(wv, L.us, L.ue);
  L.us = uniform(L.us);
  L.ue = uniform(L.ue);
  if (L.us >= T) return;
  bool l_active = true;
  L.k = wv;
  locate(L, L.us);
  pin(L);

  // Per ring slot: what the tile is, for the compute side (wave-uniform).
  // A piece is the part of one (sequence, KV head) segment inside one share.
  enum : int {
    kValid = 1,        // a real tile
    kBegin = 2,        // first tile of a piece
    kEnd = 4,          // last tile of a piece
    kBeganBefore = 8,  // the piece's segment started in an earlier share
    kSegEnd = 16,      // the piece holds the segment's last tile
    kLast = 32,        // the wavefront's last tile
    kNewRow = 64       // the segment's last tile of a call with the store fused in
  };
  struct Meta {
    int b, h, flags, k;
    int rows;  // valid key rows of the tile (0 for an empty tile)
    int new_row;  // kNewRow: the new token's row (slot) in the caches
  };

  // q of the next pieces is loaded by the load cursor when it reaches their
  // first tiles, so starting a piece does not drain the tile ring.  Two
  // buffers cover the NBUF - 1 tiles between the cursors even for one-tile
  // pieces; if both are taken the piece loads its q when it starts.
  constexpr int kQBufs = NBUF > 2 ? 2 : 1;
  // VALU form: lane-group layout, q[g] words of this lane's d chunk.  MFMA
  // form (QM): the B operand of the score MFMA, column mcol = head mcol of
  // the group (zero past G), d chunk KSM * mq + ks (8 elements) for k-step ks.
  constexpr int KSM = D / 32;  // k-steps of the score MFMA
  constexpr int DBM = D / 16;  // 16-row d blocks of O^T
  const int mcol = lane & 15;
  const int mq = lane >> 4;
  struct QV { uint32_t w[G][EPL / 2]; };
  struct QM { u32x4 k[KSM]; };
  using QBuf = typename std::conditional<MF, QM, QV>::type;
  QBuf qn0, qn1;
  int qn_seg0 = -1, qn_seg1 = -1;  // (sequence, KV head) index held, -1 = free
  auto load_q = [&](int b, int h, QBuf& dst) {
    const int64_t head0 = (int64_t)b * H_q + (int64_t)h * G;
    if constexpr (MF) {
#pragma unroll
      for (int ks = 0; ks < KSM; ++ks)
        dst.k[ks] = mcol < G ? ld16(q + (head0 + mcol) * D + 8 * (KSM * mq + ks)) : u32x4{0, 0, 0, 0};
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const u32x4 v = ld16(q + (head0 + g) * D + dofs(w));
          dst.w[g][4 * w + 0] = v[0];
          dst.w[g][4 * w + 1] = v[1];
          dst.w[g][4 * w + 2] = v[2];
          dst.w[g][4 * w + 3] = v[3];
        }
      }
    }
  };

  // Loads the tile under the load cursor and moves the cursor on.  Once the
  // wavefront has no work left the cursor stays on its last tile, whose
  // re-read is an L2 hit, and the tile is marked empty.
  auto load_tile = [&](u32x4 (&kx)[TPL][NW], u32x4 (&vx)[TPL][NW], Meta& mt, int& grab_slot) {
    pin(L);
    const bool real = uniform(l_active ? 1 : 0) != 0;
    mt.flags = 0;
    // Ask for the next share when loading the current one's second-to-last
    // tile (its only tile for one-tile shares); switch after the last.
    // (A one-tile share has no earlier tile: it asks when it ends.)
    if (real && L.u + 2 == L.ue && dynamic && lane == 0) grab_slot = atomicAdd(queue, 1);
    if (real && L.u + 1 == L.ue) switch_pending = true;
    if (real) {
      const bool begin = L.j == 0 || L.u == L.us;
      const bool end = L.j + 1 == L.nt || L.u + 1 == L.ue;
      const int seg0 = L.base + L.h * L.nt;  // unit of the segment's tile 0
      mt.b = L.b;
      mt.h = L.h;
      mt.k = L.k;
      mt.flags = uniform(kValid | (begin ? kBegin : 0) | (end ? kEnd : 0) |
                         (seg0 < L.us ? kBeganBefore : 0) | (L.j + 1 == L.nt ? kSegEnd : 0));
      if (begin) {
        if (qn_seg0 < 0) {
          load_q(L.b, L.h, qn0);
          qn_seg0 = uniform(L.b * H_kv + L.h);
        } else if (kQBufs > 1 && qn_seg1 < 0) {
          load_q(L.b, L.h, qn1);
          qn_seg1 = uniform(L.b * H_kv + L.h);
        }
      }
    }
    const int t = L.j * kDecodeTile;
    int blk = block_tables[(int64_t)L.b * maxb + (t >> bs_log2)];
    const bool blk_ok = real && (unsigned)blk < (unsigned)num_blocks;
    blk = (unsigned)blk < (unsigned)num_blocks ? blk : 0;
    const int64_t row0 = ((int64_t)blk << bs_log2) + (t & bmask);
    const uint16_t* kt = k_cache + row0 * rs + (int64_t)L.h * D;
    const uint16_t* vt = v_cache + row0 * rs + (int64_t)L.h * D;
    const int last = L.len - 1 - t;
    mt.rows = uniform(blk_ok ? last + 1 : 0);
    // With the store fused in, the segment's last tile (also when re-read as
    // an empty step) takes its last row from the new token, so the kernel
    // never reads the cache row it writes.
    bool from_new = false;
    if constexpr (FUSE) {
      if (L.j + 1 == L.nt)
        from_new = L.b < kSeqCache ? uniform(newok[L.b]) != 0 : context_lens[L.b] <= cap;
    }
    if (from_new && real && blk_ok) {
      mt.flags |= kNewRow;
      mt.new_row = (int)(row0 + last);  // a slot: below num_blocks * block_size <= INT32_MAX
    }
    const uint16_t* kn = from_new ? nt_in.key + (int64_t)L.b * nt_in.key_stride + (int64_t)L.h * D : kt;
    const uint16_t* vn = from_new ? nt_in.value + (int64_t)L.b * nt_in.value_stride + (int64_t)L.h * D : vt;
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const int r = grp + i * TPI;
      // rows past the last one re-read it (weight 0): from the new token too,
      // since its cache row is not written yet
      const bool nr = from_new && r >= last;
      const int off = (r <= last ? r : last) * rs;
      const uint16_t* kp = nr ? kn : kt + off;
      const uint16_t* vp = nr ? vn : vt + off;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        kx[i][w] = ld16_stream(kp + dofs(w));
        vx[i][w] = ld16_stream(vp + dofs(w));
      }
    }
    if (real && !switch_pending) step_unit(L);
    pin(L);
  };

  // After the step that loaded a share's last tile: move the load cursor to
  // the share the counter handed out, or end the wavefront's work (a counter
  // value outside [0, dynamic shares) also ends it).
  auto finish_share = [&](Meta& mt, const int& grab_prev) {
    if (!switch_pending) return;
    switch_pending = false;
    int gv = -1;
    if (dynamic) {
      if (L.ue - L.us == 1) {
        // one-tile share: ask now and wait (rare: only at the end of a level)
        int g1 = 0;
        if (lane == 0) g1 = atomicAdd(queue, 1);
        gv = uniform(g1);
      } else {
        gv = uniform(grab_prev);
      }
    }
    const int kn = gv >= 0 && gv < num_shares - W ? W + gv : num_shares;
    int ns = T, ne = T;
    if (kn < num_shares) sch.range(kn, ns, ne);
    ns = uniform(ns);
    ne = uniform(ne);
    if (ns < T) {
      L.k = kn;
      L.us = ns;
      L.ue = ne;
      locate(L, ns);
    } else {
      l_active = false;
      mt.flags |= kLast;
    }
    pin(L);
  };

  QBuf qw;
  // VALU form: per lane group, G running (m, l) and acc[g][EPL] of this
  // lane's d chunk.  MFMA form: O^T in d blocks (lane: rows d = 16 * db +
  // 4 * mq .. + 3 of column mcol), one (m, l) per lane for column mcol
  // (m common to the column's four lanes, l a partial sum over its keys).
  float acc[MF ? 1 : G][EPL];
  float m[MF ? 1 : G], l[MF ? 1 : G];
  f32x4 om[MF ? DBM : 1];

  auto pin_q = [&](QBuf& x) {
    if constexpr (MF) {
#pragma unroll
      for (int ks = 0; ks < KSM; ++ks) asm volatile("" : "+v"(x.k[ks]));
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < EPL / 2; ++k) asm volatile("" : "+v"(x.w[g][k]));
    }
  };

  auto begin_segment = [&](const Meta& mt) {
    const int id = mt.b * H_kv + mt.h;
    if (qn_seg0 == id) {
      qw = qn0;
      qn_seg0 = -1;
    } else if (kQBufs > 1 && qn_seg1 == id) {
      qw = qn1;
      qn_seg1 = -1;
    } else {
      // Rare (both prefetch buffers taken): load q now and wait for it here,
      // so that qw carries no pending load out of this branch (otherwise the
      // first use of qw on every path would wait for this step's tile loads).
      load_q(mt.b, mt.h, qw);
      pin_q(qw);
    }
    if constexpr (MF) {
      m[0] = kNegSentinel;
      l[0] = 0.f;
#pragma unroll
      for (int db = 0; db < DBM; ++db) om[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        m[g] = kNegSentinel;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
      }
    }
  };

  // MFMA form: element offset of 16-byte chunk c of row r (0..15) of a staged
  // K or V tile, chunks XOR-swizzled by row.  With this swizzle the chunk
  // stores (16 lanes per row), the transposing V reads and the K operand reads
  // (quarter mq of k-step ks reads chunk KSM * mq + ks of row mcol) measure
  // free of LDS bank conflicts (SQ_LDS_BANK_CONFLICT).  The order of the d
  // chunks over the k-steps is free, since q is laid out the same way; the
  // order 4 * ks + mq conflicted (about 4 stall cycles per K read).
  auto mf_off = [&](int r, int c) {
    const int sw = D == 128 ? 2 * (r & 7) + (r >> 3) : 2 * ((r >> 1) & 3) + ((r >> 3) & 1);
    return r * D + ((c ^ sw) << 3);
  };

  // MFMA form of one tile: stage K and V in LDS, S^T = K Q^T (16 keys x 16
  // columns, one v_mfma_f32_16x16x32_bf16 per 32 d), the online softmax on
  // the four scores each lane holds (keys 4 * mq .. + 3 of column mcol), then
  // O^T += V^T P^T per 16-row d block with V^T read transposed from LDS
  // (ds_read_b64_tr_b16) and P split into bf16 high and low parts (two
  // v_mfma_f32_16x16x16_bf16), which keeps P to about 2^-16.
  auto compute_tile_mf = [&](const u32x4 (&kx)[TPL][NW], const u32x4 (&vx)[TPL][NW], int rows) {
    if constexpr (MF) {
      uint16_t* kl = kv_lds;
      uint16_t* vl = kv_lds + kDecodeTile * D;
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        const int r = grp + i * TPI;
        *reinterpret_cast<u32x4*>(kl + mf_off(r, sub)) = kx[i][0];
        *reinterpret_cast<u32x4*>(vl + mf_off(r, sub)) = vx[i][0];
      }
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSM; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kl + mf_off(mcol, KSM * mq + ks));
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                     __builtin_bit_cast(bf16x8, qw.k[ks]), st, 0, 0, 0);
      }
      float sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = 4 * mq + r < rows ? st[r] * scale_log2e : -INFINITY;
      float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mx = cross_reduce<16, true>(mx);
      if (__any(mx > m[0] + kLazyRescale)) {
        const float mn = fmaxf(m[0], mx);
        const float alpha = fast_exp2(m[0] - mn);
        m[0] = mn;
        l[0] *= alpha;
#pragma unroll
        for (int db = 0; db < DBM; ++db) om[db] *= alpha;
      }
      i16x4 ph, pl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(sc[r] - m[0]);
        l[0] += p;
        const __bf16 hi = (__bf16)p;
        const __bf16 lo = (__bf16)(p - (float)hi);
        ph[r] = __builtin_bit_cast(short, hi);
        pl[r] = __builtin_bit_cast(short, lo);
      }
#pragma unroll
      for (int db = 0; db < DBM; ++db) {
        // lane mcol of quarter mq gets V[4 * mq + e][16 * db + mcol], e = 0..3
        const int col = 16 * db + 4 * (mcol & 3);
        const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vl + mf_off(4 * mq + (mcol >> 2), col >> 3) +
                                                       (col & 7)));
        om[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, ph, om[db], 0, 0, 0);
        om[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pl, om[db], 0, 0, 0);
      }
    }
  };

  auto compute_tile = [&](const u32x4 (&kx)[TPL][NW], const u32x4 (&vx)[TPL][NW], int rows) {
    if constexpr (MF) {
      compute_tile_mf(kx, vx, rows);
      return;
    } else {
      // scores in the log2 domain
      float sc[TPL][G];
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float dsum = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            dsum = dot2_bf16(qw.w[g][4 * w + 0], kx[i][w][0], dsum);
            dsum = dot2_bf16(qw.w[g][4 * w + 1], kx[i][w][1], dsum);
            dsum = dot2_bf16(qw.w[g][4 * w + 2], kx[i][w][2], dsum);
            dsum = dot2_bf16(qw.w[g][4 * w + 3], kx[i][w][3], dsum);
          }
          dsum = group_sum<LPT>(dsum);
          sc[i][g] = grp + i * TPI < rows ? dsum * scale_log2e : -INFINITY;
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

    }
  };

  // MFMA form of the end of a piece: the column's l summed over its four
  // lanes (m is already common to them); lanes of columns below G hold d rows
  // 16 * db + 4 * mq .. + 3 of head mcol, written as bf16 (a segment in one
  // piece) or as an fp32 partial with (m, l) (a piece of a cut segment).
  auto end_segment_mf = [&](const Meta& mt) {
    if constexpr (MF) {
      const float lt = cross_reduce<16, false>(l[0]);
      const bool first_piece = !(mt.flags & kBeganBefore);
      const bool last_piece = (mt.flags & kSegEnd) != 0;
      if (lane == 0) {
        int32_t* rec = reinterpret_cast<int32_t*>(ws_seg + ((int64_t)mt.b * H_kv + mt.h));
        if (first_piece) rec[0] = mt.k;
        if (last_piece) rec[1] = mt.k;
      }
      if (mcol >= G) return;
      const int64_t head0 = (int64_t)mt.b * H_q + (int64_t)mt.h * G;
      if (first_piece && last_piece) {
        const float inv = 1.0f / lt;
        uint16_t* op = out + (head0 + mcol) * D + 4 * mq;
#pragma unroll
        for (int db = 0; db < DBM; ++db)
          *reinterpret_cast<u32x2*>(op + 16 * db) =
              u32x2{pack_bf16x2(om[db][0] * inv, om[db][1] * inv),
                    pack_bf16x2(om[db][2] * inv, om[db][3] * inv)};
      } else {
        const int slot = first_piece ? 1 : 0;
        const int64_t row = ((int64_t)mt.k * 2 + slot) * G + mcol;
        float* ap = ws_acc + row * D + 4 * mq;
#pragma unroll
        for (int db = 0; db < DBM; ++db) *reinterpret_cast<f32x4*>(ap + 16 * db) = om[db];
        if (mq == 0) *reinterpret_cast<float2*>(ws_ml + row * 2) = make_float2(m[0], lt);
      }
    }
  };

  auto end_segment = [&](const Meta& mt) {
    if constexpr (MF) {
      end_segment_mf(mt);
      return;
    } else {
      // merge the TPI lane groups (log-sum-exp); group 0 holds the result
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float M = cross_reduce<LPT, true>(m[g]);
        const float alpha = fast_exp2(m[g] - M);
        l[g] = cross_reduce<LPT, false>(l[g] * alpha);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = cross_reduce<LPT, false>(acc[g][e] * alpha);
        m[g] = M;
      }
      // A segment in one piece is written directly.  Otherwise its first
      // piece records its share in k_first and its last piece in k_last; the
      // merge combines shares k_first .. k_last.
      const bool first_piece = !(mt.flags & kBeganBefore);
      const bool last_piece = (mt.flags & kSegEnd) != 0;
      if (lane == 0) {
        int32_t* rec = reinterpret_cast<int32_t*>(ws_seg + ((int64_t)mt.b * H_kv + mt.h));
        if (first_piece) rec[0] = mt.k;
        if (last_piece) rec[1] = mt.k;
      }
      const int64_t head0 = (int64_t)mt.b * H_q + (int64_t)mt.h * G;
      if (first_piece && last_piece) {
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
        // partial slot 0: the share's piece that began in an earlier share;
        // slot 1: a piece that begins in this share and goes on past it
        const int slot = first_piece ? 1 : 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int64_t row = ((int64_t)mt.k * 2 + slot) * G + g;
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

    }
  };

  // The fused store: the lanes holding the tile's last row (the new token,
  // read from the new K/V input) write it into the caches.
  // (The caches are written through the kernel's own cache pointers: the
  // call's caches are not const, and this row is read by no one in the call.)
  auto store_new_row = [&](const u32x4 (&kx)[TPL][NW], const u32x4 (&vx)[TPL][NW], const Meta& mt) {
    const int64_t at = (int64_t)mt.new_row * rs + (int64_t)mt.h * D;
    uint16_t* kd = const_cast<uint16_t*>(k_cache) + at;
    uint16_t* vd = const_cast<uint16_t*>(v_cache) + at;
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      if (grp + i * TPI != mt.rows - 1) continue;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        st16(kd + dofs(w), kx[i][w]);
        st16(vd + dofs(w), vx[i][w]);
      }
    }
  };

  // Ring of NBUF register buffers; the loop is unrolled NBUF times so every
  // buffer index is a compile-time constant (no register copies).
  u32x4 kbuf[NBUF][TPL][NW], vbuf[NBUF][TPL][NW];
  Meta meta[NBUF];
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i) {
    load_tile(kbuf[i], vbuf[i], meta[i], grab[i]);
    finish_share(meta[i], grab[(i + NBUF - 1) % NBUF]);
  }
  bool done = false;
  while (!done) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int nxt = (u + NBUF - 1) % NBUF;
      const Meta mt = meta[u];
      // take the piece's q before this step's loads may refill a q buffer
      if ((mt.flags & (kValid | kBegin)) == (kValid | kBegin)) begin_segment(mt);
      load_tile(kbuf[nxt], vbuf[nxt], meta[nxt], grab[nxt]);
      if (mt.flags & kValid) {
        if (FUSE && (mt.flags & kNewRow)) store_new_row(kbuf[u], vbuf[u], mt);
        compute_tile(kbuf[u], vbuf[u], mt.rows);
        if (mt.flags & kEnd) end_segment(mt);
        if (mt.flags & kLast) done = true;
      }
      finish_share(meta[nxt], grab[(nxt + NBUF - 1) % NBUF]);
    }
  }
}

// Combine the pieces of one (sequence, query head) whose segment was cut
// into several shares: M = max_p m_p, L = sum_p l_p 2^(m_p - M),
// out = sum_p acc_p 2^(m_p - M) / L.  The first piece sits in partial slot 1
// of its share, the others in slot 0.  One wavefront per output row; its 64
// lanes take 8 pieces at a time (8 lanes of D / 8 elements per piece), and
// the 8 piece groups are summed at the end in a fixed order, so the result is
// deterministic.  Rows of empty sequences are written as zeros here, and the
// share counter is reset for the next call (this kernel runs after the
// decode kernel).
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
    const SegInfo* __restrict__ ws_seg, int32_t* __restrict__ queue,
    const int32_t* __restrict__ context_lens, uint16_t* __restrict__ out, int32_t B,
    int32_t H_q, int32_t G, int32_t max_shares) {
  constexpr int EPL = D / 8;  // elements per lane of a piece group
  if (blockIdx.x == 0 && threadIdx.x == 0) *queue = 0;
  const int lane = threadIdx.x % 64;
  const int pg = lane / 8;   // piece group
  const int sub = lane % 8;  // d chunk
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;  // b * H_q + h
  if (row >= (int64_t)B * H_q) return;
  // row / H_q in 32 bits when every row index fits (a uniform branch)
  const int b = (int64_t)B * H_q <= INT32_MAX ? (int)((uint32_t)row / (uint32_t)H_q)
                                              : (int)(row / H_q);
  const int hq = (int)(row - (int64_t)b * H_q);
  uint16_t* op = out + row * D + sub * EPL;
  // the length and the segment record are independent: both loads in flight
  const int H_kv = H_q / G;
  const int32_t len = context_lens[b];
  const SegInfo info = ws_seg[(int64_t)b * H_kv + hq / G];
  // used here, so the compiler cannot sink the record's load below the branch
  asm volatile("" ::"v"(info.k_first), "v"(info.k_last));
  if (len <= 0) {
    if (pg == 0) {
#pragma unroll
      for (int w = 0; w < EPL / 8; ++w) st16(op + 8 * w, u32x4{0u, 0u, 0u, 0u});
    }
    return;
  }
  if (info.k_last <= info.k_first) return;  // one piece: written by the decode kernel
  if (info.k_first < 0 || info.k_last >= max_shares) return;  // not from this call's layout
  const int nparts = info.k_last - info.k_first + 1;
  const int g = hq % G;
  auto prow = [&](int p) -> int64_t {
    const int64_t k = (int64_t)info.k_first + p;
    return (k * 2 + (p == 0 ? 1 : 0)) * G + g;
  };

  // One pass: each piece group keeps a running (max, sum, acc) over its
  // pieces, so all of a row's loads can be in flight together; the 8 groups
  // are then rescaled to the common max and summed.  (A piece's max is
  // finite: every piece holds at least one tile of keys.)
  float mg = -INFINITY, lg = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  if (nparts <= 8) {  // at most one piece per group: one round of loads
    if (pg < nparts) {
      const int64_t r = prow(pg);
      const float2 st = *reinterpret_cast<const float2*>(ws_ml + 2 * r);
      const float* src = ws_acc + r * D + sub * EPL;
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + e);
        o[e] = v[0];
        o[e + 1] = v[1];
        o[e + 2] = v[2];
        o[e + 3] = v[3];
      }
      mg = st.x;
      lg = st.y;
    }
  }
  // More pieces: each group fetches KB of them before combining any, so a
  // row's loads overlap.
  auto batched = [&](auto kb_tag) {
    constexpr int KB = decltype(kb_tag)::value;
    for (int p0 = pg; p0 < nparts; p0 += 8 * KB) {
      float2 st[KB];
      f32x4 v[KB][EPL / 4];
#pragma unroll
      for (int j = 0; j < KB; ++j) {  // unconditional loads (a piece past the end reads piece pg)
        const int p = p0 + 8 * j;
        const int64_t r = prow(p < nparts ? p : pg);
        st[j] = *reinterpret_cast<const float2*>(ws_ml + 2 * r);
        const float* src = ws_acc + r * D + sub * EPL;
#pragma unroll
        for (int e = 0; e < EPL / 4; ++e) v[j][e] = *reinterpret_cast<const f32x4*>(src + 4 * e);
      }
      __builtin_amdgcn_sched_barrier(0);  // every load of the batch is issued before any use
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        // a piece past the end weighs 0 (max -inf); piece j = 0 always exists,
        // so mg is finite before any such piece and its a is 1
        const bool in = p0 + 8 * j < nparts;
        const float mj = in ? st[j].x : -INFINITY;
        const float mn = fmaxf(mg, mj);
        const float a = fast_exp2(mg - mn);  // 0 for the group's first piece
        const float w = fast_exp2(mj - mn);
        lg = lg * a + (in ? st[j].y : 0.f) * w;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = o[e] * a + v[j][e / 4][e % 4] * w;
        mg = mn;
      }
    }
  };
  if (nparts > 8) batched(std::integral_constant<int, 2>{});
  const float M = cross_reduce<8, true>(mg);
  const float sg = fast_exp2(mg - M);  // 0 for a group without pieces
  const float L = cross_reduce<8, false>(lg * sg);
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = cross_reduce<8, false>(o[e] * sg);
  if (pg != 0) return;
  const float inv = 1.0f / L;
#pragma unroll
  for (int w = 0; w < EPL / 8; ++w) {
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v[k] = pack_bf16x2(o[8 * w + 2 * k] * inv, o[8 * w + 2 * k + 1] * inv);
    st16(op + 8 * w, v);
  }
}

// The merge for wide groups, one wavefront per (sequence, KV head) segment
// instead of one per output row: the segment's record and the sequence's
// length are read once for its G rows, lane group g (64 / G lanes, G * D / 64
// elements each) combines query head g, and every lane keeps four pieces'
// loads in flight.  Pieces are combined in share order, as in
// decode_merge_kernel, so the result is deterministic.  Used at G = 8 (at
// G = 4 it measured the same as one wavefront per row, at G = 2 slower).
template <int D, int G>
__global__ __launch_bounds__(256) void decode_merge_seg_kernel(
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
    const SegInfo* __restrict__ ws_seg, int32_t* __restrict__ queue,
    const int32_t* __restrict__ context_lens, uint16_t* __restrict__ out, int32_t B, int32_t H_kv,
    int32_t max_shares) {
  constexpr int LPR = 64 / G;   // lanes per query head
  constexpr int EPL = D / LPR;  // elements per lane
  constexpr int KB = 4;         // pieces in flight
  static_assert(EPL % 8 == 0, "whole 16-byte stores per lane");
  if (blockIdx.x == 0 && threadIdx.x == 0) *queue = 0;
  const int lane = threadIdx.x % 64;
  const int g = lane / LPR;
  const int sub = lane % LPR;
  const int64_t seg = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;  // b * H_kv + h
  if (seg >= (int64_t)B * H_kv) return;
  const int b = (int)(seg / H_kv);
  const int32_t len = context_lens[b];
  const SegInfo info = ws_seg[seg];
  asm volatile("" ::"v"(info.k_first), "v"(info.k_last));
  uint16_t* op = out + (seg * G + g) * D + sub * EPL;  // row b * H_q + h * G + g
  if (len <= 0) {
#pragma unroll
    for (int w = 0; w < EPL / 8; ++w) st16(op + 8 * w, u32x4{0u, 0u, 0u, 0u});
    return;
  }
  if (info.k_last <= info.k_first) return;  // one piece: written by the decode kernel
  if (info.k_first < 0 || info.k_last >= max_shares) return;  // not from this call's layout
  const int nparts = info.k_last - info.k_first + 1;
  auto prow = [&](int p) -> int64_t {
    const int64_t k = (int64_t)info.k_first + p;
    return (k * 2 + (p == 0 ? 1 : 0)) * G + g;
  };
  float mg = -INFINITY, lg = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  for (int p0 = 0; p0 < nparts; p0 += KB) {
    float2 st[KB];
    f32x4 v[KB][EPL / 4];
#pragma unroll
    for (int j = 0; j < KB; ++j) {  // unconditional loads (a piece past the end reads piece 0)
      const int p = p0 + j;
      const int64_t r = prow(p < nparts ? p : 0);
      st[j] = *reinterpret_cast<const float2*>(ws_ml + 2 * r);
      const float* src = ws_acc + r * D + sub * EPL;
#pragma unroll
      for (int e = 0; e < EPL / 4; ++e) v[j][e] = *reinterpret_cast<const f32x4*>(src + 4 * e);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the batch is issued before any use
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      // piece 0 always exists and its max is finite, so mg is finite before
      // any piece past the end, which weighs 0
      const bool in = p0 + j < nparts;
      const float mj = in ? st[j].x : -INFINITY;
      const float mn = fmaxf(mg, mj);
      const float a = fast_exp2(mg - mn);  // 0 for the first piece
      const float w = fast_exp2(mj - mn);
      lg = lg * a + (in ? st[j].y : 0.f) * w;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = o[e] * a + v[j][e / 4][e % 4] * w;
      mg = mn;
    }
  }
  const float inv = 1.0f / lg;
#pragma unroll
  for (int w = 0; w < EPL / 8; ++w) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      r[k] = pack_bf16x2(o[8 * w + 2 * k] * inv, o[8 * w + 2 * k + 1] * inv);
    st16(op + 8 * w, r);
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
template <int D, int G, int EPL, int NBUF, int WPE, bool MF>
static int resident_waves() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<D, G, EPL, NBUF, WPE, MF, false>,
                                                     64, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 8;
    cached[dev] = cus * per_cu;
  }
  return cached[dev];
}

// Kernel variant per (d, G): elements per lane, ring depth, wavefronts per
// SIMD, and the MFMA form for wide groups (G >= 4), where the VALU's q.k and
// p.v work per byte of K/V would outrun the HBM stream.
template <typename F>
static bool dispatch(int d, int G, F& f) {
  if (d == 128) {
    switch (G) {
      case 1: f.template run<128, 1, 16, 3, 2, false>(); return true;
      case 2: f.template run<128, 2, 16, 3, 2, false>(); return true;
      case 4: f.template run<128, 4, 8, 3, 2, true>(); return true;
      case 8: f.template run<128, 8, 8, 3, 2, true>(); return true;
    }
  } else if (d == 64) {
    switch (G) {
      case 1: f.template run<64, 1, 8, 3, 2, false>(); return true;
      case 2: f.template run<64, 2, 8, 3, 2, false>(); return true;
      case 4: f.template run<64, 4, 8, 3, 2, true>(); return true;
      case 8: f.template run<64, 8, 8, 3, 2, true>(); return true;
    }
  }
  return false;
}

struct WaveQuery {
  int waves = 0;
  template <int D, int G, int EPL, int NBUF, int WPE, bool MF>
  void run() { waves = resident_waves<D, G, EPL, NBUF, WPE, MF>(); }
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace: two fp32 partial slots (acc[d], then (m, l)) per query head of
// a group for every share the schedule can hold (ShareSchedule::max_shares), one SegInfo
// per (sequence, KV head), and the share counter in its own 256-byte line.
struct WorkspaceLayout {
  size_t acc, ml, seg, queue, total;
};
static WorkspaceLayout workspace_layout(int32_t B, int32_t H_kv, int32_t G, int32_t d,
                                        int32_t waves) {
  WorkspaceLayout w;
  const size_t rows = (size_t)ShareSchedule::max_shares(waves) * 2 * G;
  w.acc = 0;
  w.ml = align256(rows * d * sizeof(float));
  w.seg = w.ml + align256(rows * 2 * sizeof(float));
  w.queue = w.seg + align256((size_t)B * H_kv * sizeof(SegInfo));
  w.total = w.queue + 256;
  return w;
}

DecodePlan decode_plan(int32_t B, int32_t H_q, int32_t H_kv, int32_t d, int32_t block_size,
                       int32_t max_blocks_per_seq) {
  (void)block_size;
  (void)max_blocks_per_seq;
  DecodePlan p{0, 0};
  const int G = H_q / H_kv;
  WaveQuery wq;
  if (!dispatch(d, G, wq)) return p;
  p.num_waves = wq.waves;
  p.workspace_bytes = workspace_layout(B, H_kv, G, d, wq.waves).total;
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
  int32_t* queue;
  int32_t B, H_kv, nb, bsl, maxb;
  float sl2e;
  NewToken nt;
  template <int D, int G, int EPL, int NBUF, int WPE, bool MF>
  void run() {
    // the fused store is its own instantiation, so the plain decode keeps its
    // registers; both have the same occupancy (two wavefronts per SIMD)
    if (nt.key)
      hipLaunchKernelGGL((decode_kernel<D, G, EPL, NBUF, WPE, MF, true>), grid, dim3(64), 0, st, q, kc, vc,
                         bt, cl, out, wa, wm, wseg, queue, B, H_kv, nb, bsl, maxb, sl2e, nt);
    else
      hipLaunchKernelGGL((decode_kernel<D, G, EPL, NBUF, WPE, MF, false>), grid, dim3(64), 0, st, q, kc, vc,
                         bt, cl, out, wa, wm, wseg, queue, B, H_kv, nb, bsl, maxb, sl2e, nt);
  }
};

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int32_t B, int32_t H_q, int32_t H_kv,
                         int32_t d, int32_t num_blocks, int32_t block_size,
                         int32_t max_blocks_per_seq, float softmax_scale, void* workspace,
                         const DecodePlan& plan, const NewToken& new_token, hipStream_t stream) {
  const int G = H_q / H_kv;
  const WorkspaceLayout wl = workspace_layout(B, H_kv, G, d, plan.num_waves);
  char* ws = static_cast<char*>(workspace);
  float* wa = reinterpret_cast<float*>(ws + wl.acc);
  float* wm = reinterpret_cast<float*>(ws + wl.ml);
  SegInfo* wseg = reinterpret_cast<SegInfo*>(ws + wl.seg);
  int32_t* queue = reinterpret_cast<int32_t*>(ws + wl.queue);
  DecodeLaunch lf{dim3((unsigned)plan.num_waves), stream, q, k_cache, v_cache, block_tables,
                  context_lens, out, wa, wm, wseg, queue, B, H_kv, num_blocks, ilog2(block_size),
                  max_blocks_per_seq, softmax_scale * 1.4426950408889634f, new_token};
  if (!dispatch(d, G, lf)) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nrows = (int64_t)B * H_q;
  const int32_t max_shares = (int32_t)ShareSchedule::max_shares(plan.num_waves);
  if (G == 8) {
    const dim3 sgrid((unsigned)(((int64_t)B * H_kv + 3) / 4));
    if (d == 128)
      hipLaunchKernelGGL((decode_merge_seg_kernel<128, 8>), sgrid, dim3(256), 0, stream, wa, wm, wseg,
                         queue, context_lens, out, B, H_kv, max_shares);
    else
      hipLaunchKernelGGL((decode_merge_seg_kernel<64, 8>), sgrid, dim3(256), 0, stream, wa, wm, wseg,
                         queue, context_lens, out, B, H_kv, max_shares);
    return hipGetLastError();
  }
  dim3 mgrid((unsigned)((nrows + 3) / 4));
  if (d == 128)
    hipLaunchKernelGGL(decode_merge_kernel<128>, mgrid, dim3(256), 0, stream, wa, wm, wseg,
                       queue, context_lens, out, B, H_q, G, max_shares);
  else
    hipLaunchKernelGGL(decode_merge_kernel<64>, mgrid, dim3(256), 0, stream, wa, wm, wseg,
                       queue, context_lens, out, B, H_q, G, max_shares);
  return hipGetLastError();
}

}  // namespace pkv
