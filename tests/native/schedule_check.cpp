// Checks the decode share schedule (paged_kv_cache_110_amd/csrc/decode_schedule.h)
// on the host, for both forms of the decode (VALU and MFMA, whose static
// fractions differ).  Reads "T W" pairs from stdin; prints the first violated
// property and exits non-zero, or "ok" and the case count.
//   1. the non-empty shares, in index order, tile [0, T) contiguously;
//   2. empty shares only follow the last non-empty one;
//   3. share_of(u) names the share whose range holds u;
//   4. static shares (k < W) hold S0 units except the last non-empty one,
//      and when dynamic shares exist every static share is non-empty;
//   5. no more than max_shares(W) shares; dynamic shares shrink (never grow)
//      from one level to the next, except for the last level (W shares that
//      split whatever remains);
//   6. a call of at most kOnePassUnits units per wavefront is static and
//      gives no wavefront more than max(ceil(T / W), PKV_SCHED_SMALL_MIN) units.
#include <cstdio>
#include <cstdint>

#include "decode_schedule.h"

static int fail(const char* what, long long T, long long W, long long a, long long b) {
  std::printf("FAIL %s T=%lld W=%lld (%lld, %lld)\n", what, T, W, a, b);
  return 1;
}

static int check(int T, int W, bool mfma_form) {
  const pkv::ShareSchedule s = pkv::ShareSchedule::make(T, W, mfma_form);
  const int n = s.num_shares();
  if (n > pkv::ShareSchedule::max_shares(W)) return fail("share count", T, W, n, 0);
  long long next = 0;  // first unit not yet covered
  bool seen_empty = false;
  int last_dyn_size = -1, last_level = 0;
  for (int k = 0; k < n; ++k) {
    int st = 0, en = 0;
    s.range(k, st, en);
    if (st >= T) {
      seen_empty = true;
      continue;
    }
    if (seen_empty) return fail("non-empty share after an empty one", T, W, k, st);
    if (st != next || en <= st || en > T) return fail("not contiguous", T, W, k, st);
    if (k < W && en - st != s.S0 && en != T && en != s.P1) return fail("static size", T, W, k, en - st);
    // levels: k < W static; then kLevels - 2 levels of ceil(W / 2) shares; then W shares
    const int N = (W + 1) / 2;
    const int level = k < W ? 0 : 1 + (k - W) / N;
    if (level >= 1 && level < pkv::ShareSchedule::kLevels - 1) {
      if (level > last_level && last_dyn_size >= 0 && (en - st) > last_dyn_size)
        return fail("dynamic share grew", T, W, k, en - st);
      last_dyn_size = en - st;
      last_level = level;
    }
    // 3: exhaustive for small ranges, ends and a midpoint otherwise
    if (en - st <= 64) {
      for (int u = st; u < en; ++u)
        if (s.share_of(u) != k) return fail("share_of", T, W, u, s.share_of(u));
    } else {
      const int probe[3] = {st, st + (en - st) / 2, en - 1};
      for (int u : probe)
        if (s.share_of(u) != k) return fail("share_of", T, W, u, s.share_of(u));
    }
    next = en;
  }
  if (next != T) return fail("coverage", T, W, next, 0);
  const long long per_wave = ((long long)T + W - 1) / W;
  if (per_wave <= pkv::ShareSchedule::kOnePassUnits) {
    if (s.dynamic()) return fail("small call not static", T, W, per_wave, 0);
    for (int k = 0; k < W; ++k) {
      int st = 0, en = 0;
      s.range(k, st, en);
      const long long cap = per_wave > PKV_SCHED_SMALL_MIN ? per_wave : PKV_SCHED_SMALL_MIN;
      if (en - st > cap) return fail("small call share size", T, W, k, en - st);
    }
  }
  if (s.dynamic()) {
    for (int k = 0; k < W; ++k) {
      int st = 0, en = 0;
      s.range(k, st, en);
      if (st >= T) return fail("empty static share with dynamic work", T, W, k, 0);
    }
  }
  return 0;
}

int main() {
  long long T = 0, W = 0;
  int cases = 0;
  while (std::scanf("%lld %lld", &T, &W) == 2) {
    if (check((int)T, (int)W, false) || check((int)T, (int)W, true)) return 1;
    ++cases;
  }
  std::printf("ok %d cases\n", cases);
  return 0;
}
