// Share schedule of the persistent decode kernel: how the flattened list of
// T units ((sequence, KV head, 16-token tile) triples) is cut into shares
// for W wavefronts.  Plain C++ usable on the host and the device, so the
// layout can be checked on the CPU.
//
// A call of at most kOnePassUnits units per wavefront is one static pass
// of ceil(T / W) units per wavefront, but at least PKV_SCHED_SMALL_MIN, so
// that more wavefronts start at once (small batches are latency-bound) while
// segments are not cut into more pieces than the merge gathers quickly.
// Larger calls:
// Level 0: one static share of S0 units per wavefront, ending at unit P1:
// for calls of at most kMidStaticUnits units per wavefront 70% of the work
// (80% for the decode's MFMA form, whose wavefronts run at more even rates),
// 40% for larger ones (a small call loses more to share changes and split
// pieces, a large one more to wavefronts drifting apart).  Levels 1..kLevels-2 hold N = ceil(W / 2) shares
// each and are handed out in order through an atomic counter: level 1's
// shares hold S1 units (what is left, spread over 2W), each further level
// three quarters as many (at least kDynMinUnits).  The last level has W
// shares that split whatever remains.  Shares shrink towards the end of the
// call, so a slow wavefront that takes one late cannot hold the call up for
// long, and every wavefront stops within a few tiles of the others.  Share k
// covers [start, end); only the last non-empty level can hold empty shares
// (start == T), so the pieces of any run of consecutive units lie in
// consecutive non-empty shares.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define PKV_HD __attribute__((host, device, always_inline)) inline
#else
#define PKV_HD inline
#endif

namespace pkv {

struct ShareSchedule {
#ifndef PKV_SCHED_STATIC_NUM
#define PKV_SCHED_STATIC_NUM 2  // static part of large calls: 2/5 of the work
#define PKV_SCHED_STATIC_DEN 5
#endif
#ifndef PKV_SCHED_MID_STATIC_NUM
#define PKV_SCHED_MID_STATIC_NUM 7  // static part of calls up to kMidStaticUnits per wavefront: 7/10
#define PKV_SCHED_MID_STATIC_DEN 10
#endif
#ifndef PKV_SCHED_MID_STATIC_MF_NUM
#define PKV_SCHED_MID_STATIC_MF_NUM 4  // the same for the MFMA form: 4/5
#define PKV_SCHED_MID_STATIC_MF_DEN 5
#endif
#ifndef PKV_SCHED_DYN_MIN
#define PKV_SCHED_DYN_MIN 16
#endif
#ifndef PKV_SCHED_SMALL_MIN
#define PKV_SCHED_SMALL_MIN 4  // least units per wavefront in a one-pass call
#endif
#ifndef PKV_SCHED_SHRINK
#define PKV_SCHED_SHRINK 2  // each level keeps 1 - 2^-SHRINK of the previous size
#endif
  static constexpr int kLevels = 16;
  static constexpr int kMinStaticUnits = 8;
  // Up to this many units per wavefront, one even static pass beats dynamic
  // shares, whose 16-unit minimum would leave most wavefronts idle.
  static constexpr int kOnePassUnits = 64;
  static constexpr int kMidStaticUnits = 128;
  static constexpr int kDynMinUnits = PKV_SCHED_DYN_MIN;

  int T, W, S0, P1, S1, N;

  // 0 < W; 0 <= T.  mfma_form: the schedule of the decode's MFMA form.
  static PKV_HD ShareSchedule make(int T, int W, bool mfma_form = false) {
    ShareSchedule s;
    s.T = T;
    s.W = W;
    const int64_t per_wave = ((int64_t)T + W - 1) / W;
    if (per_wave <= kOnePassUnits) {
      s.S0 = per_wave < PKV_SCHED_SMALL_MIN ? PKV_SCHED_SMALL_MIN : (int)per_wave;
    } else {
      const bool mid = per_wave <= kMidStaticUnits;
      const int64_t num = !mid ? PKV_SCHED_STATIC_NUM
                               : (mfma_form ? PKV_SCHED_MID_STATIC_MF_NUM : PKV_SCHED_MID_STATIC_NUM);
      const int64_t den = !mid ? PKV_SCHED_STATIC_DEN
                               : (mfma_form ? PKV_SCHED_MID_STATIC_MF_DEN : PKV_SCHED_MID_STATIC_DEN);
      const int s0 = (int)(((int64_t)T * num / den) / W);
      s.S0 = s0 < kMinStaticUnits ? kMinStaticUnits : s0;
    }
    s.P1 = (int64_t)s.S0 * W < T ? s.S0 * W : T;
    s.N = (W + 1) / 2;
    const int s1 = (int)(((int64_t)(T - s.P1) + 2 * (int64_t)W - 1) / (2 * (int64_t)W));
    s.S1 = s1 < kDynMinUnits ? kDynMinUnits : s1;
    return s;
  }

  PKV_HD bool dynamic() const { return P1 < T; }
  // Shares that can exist (the workspace holds partial slots for this many).
  static PKV_HD int64_t max_shares(int W) {
    return 2 * (int64_t)W + (int64_t)(kLevels - 2) * ((W + 1) / 2);
  }
  PKV_HD int num_shares() const { return dynamic() ? (int)max_shares(W) : W; }

  // [st, en) of share k, 0 <= k < num_shares(); st == T for an empty share.
  PKV_HD void range(int k, int& st, int& en) const {
    if (k < W) {
      st = (int64_t)k * S0 < P1 ? k * S0 : T;
      en = st < T ? (P1 - st > S0 ? st + S0 : P1) : T;
      return;
    }
    int i = k - W, lo = P1, s = S1;
    for (int l = 1; l < kLevels - 1; ++l) {
      const int sz = s < kDynMinUnits ? kDynMinUnits : s;
      const int64_t len64 = (int64_t)N * sz;
      const int len = len64 < (int64_t)T - lo ? (int)len64 : T - lo;
      if (i < N) {
        piece(lo, len, sz, i, st, en);
        return;
      }
      i -= N;
      lo += len;
      s -= s >> PKV_SCHED_SHRINK;
    }
    const int sz = (int)(((int64_t)T - lo + W - 1) / W);
    piece(lo, T - lo, sz < 1 ? 1 : sz, i, st, en);
  }

  // Index of the share holding unit u, 0 <= u < T.
  PKV_HD int share_of(int u) const {
    if (u < P1) return u / S0;
    int base = W, lo = P1, s = S1;
    for (int l = 1; l < kLevels - 1; ++l) {
      const int sz = s < kDynMinUnits ? kDynMinUnits : s;
      const int64_t len64 = (int64_t)N * sz;
      const int len = len64 < (int64_t)T - lo ? (int)len64 : T - lo;
      if (u - lo < len) return base + (u - lo) / sz;
      base += N;
      lo += len;
      s -= s >> PKV_SCHED_SHRINK;
    }
    const int sz = (int)(((int64_t)T - lo + W - 1) / W);
    return base + (u - lo) / (sz < 1 ? 1 : sz);
  }

 private:
  // share i of a level that starts at lo and holds len units in shares of sz
  PKV_HD void piece(int lo, int len, int sz, int i, int& st, int& en) const {
    const int64_t off = (int64_t)i * sz;
    if (off >= len) {
      st = en = T;  // empty
      return;
    }
    st = lo + (int)off;
    en = len - (int)off > sz ? st + sz : lo + len;
  }
};

}  // namespace pkv
