// Per-row top-k of the block selection, written once for the device wave and
// for a host emulation of it.
//
// A CSR row keeps the `keep` best of its window's pooled scores, ties going
// to the lower key-block index, and emits them in ascending block order (the
// mask selection and CSR construction of the FlashVSR Hopper PR page, "What
// Was Actually Slow" and "Rebuild sparse attention for Hopper").  One wave of
// 64 lanes holds the row: candidate e = lane + 64 j sits in slot j < M of
// lane e % 64, and candidates run in ascending block order.
//
// The functions take a Wave object for the two cross-lane operations they
// need: ballot (a 64-bit mask of a predicate over the lanes) and or_and (the
// wave-wide OR and AND of a 64-bit value).  The device passes the hardware
// ballot and lane shuffles; a host test passes 64 threads that meet at a
// barrier for each operation, so the same code runs under the host's
// undefined-behaviour checks.
#pragma once

#include <cstdint>

#if defined(__HIPCC__)
#define LCSA_HD __host__ __device__
#else
#define LCSA_HD
#endif

namespace lcsa {

// Order-preserving key of a double: a larger score gives a larger key, and
// -0 and +0 give the same key.
LCSA_HD inline uint64_t order_key(double s) {
  const uint64_t u = __builtin_bit_cast(uint64_t, s + 0.0);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// The keep-th largest key of a row, decided bit by bit from the top: the
// largest T with #{valid keys >= T} >= keep.  Bits that every valid key
// shares (above the highest bit where two of them differ) are taken from
// the wave-wide AND and need no count.  Returns T; *exact is set when the
// count at T is exactly keep, so {key >= T} is the kept set with no tie to
// break.  Needs 1 <= keep <= the number of valid keys; invalid slots hold
// key 0, which never reaches a trial value (every trial has a bit set).
template <int M, class Wave>
LCSA_HD inline uint64_t kth_key(Wave& w, const uint64_t (&key)[M], const bool (&valid)[M],
                                int keep, bool* exact) {
  uint64_t kor = 0ull, kand = ~0ull;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    kor |= valid[j] ? key[j] : 0ull;
    kand &= valid[j] ? key[j] : ~0ull;
  }
  w.or_and(kor, kand);
  const uint64_t diff = kor ^ kand;
  // No differing bit: every valid key equals kand, which is then the
  // keep-th largest (shifting by hb + 1 would be a shift by 0 .. 64).
  if (diff == 0ull) {
    *exact = false;
    return kand;
  }
  const int hb = 63 - __builtin_clzll(diff);
  uint64_t t = hb == 63 ? 0ull : kand & ~((2ull << hb) - 1ull);
  *exact = false;
  for (int bit = hb; bit >= 0; --bit) {
    const uint64_t trial = t | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < M; ++j) cnt += __builtin_popcountll(w.ballot(key[j] >= trial));
    if (cnt >= keep) t = trial;
    if (cnt == keep) {  // {key >= trial} is exactly the top keep
      *exact = true;
      break;
    }
  }
  return t;
}

// Selection of the `keep` best valid candidates (1 <= keep < valid count):
// keys above the keep-th are kept; keys equal to it are kept in ascending
// candidate order until keep are kept.
template <int M, class Wave>
LCSA_HD inline void topk_select(Wave& w, int lane, const uint64_t (&key)[M],
                                const bool (&valid)[M], int keep, bool (&sel)[M]) {
  bool exact = false;
  const uint64_t t = kth_key<M>(w, key, valid, keep, &exact);
  if (exact) {
#pragma unroll
    for (int j = 0; j < M; ++j) sel[j] = valid[j] && key[j] >= t;
    return;
  }
  const uint64_t below = (1ull << lane) - 1ull;
  int need = keep;
#pragma unroll
  for (int j = 0; j < M; ++j) need -= __builtin_popcountll(w.ballot(valid[j] && key[j] > t));
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const bool tie = valid[j] && key[j] == t;
    const uint64_t tm = w.ballot(tie);
    const int rank = __builtin_popcountll(tm & below);
    sel[j] = (valid[j] && key[j] > t) || (tie && rank < need);
    need -= __builtin_popcountll(tm);
    need = need < 0 ? 0 : need;
  }
}

// Output position (0 .. keep-1, ascending candidate order) of every
// selected candidate, or -1.  A selected candidate beyond the first `keep`
// gets -1 as well, so a row never writes past its own `keep` entries.
template <int M, class Wave>
LCSA_HD inline void kept_positions(Wave& w, int lane, const bool (&sel)[M], int keep,
                                   int (&pos)[M]) {
  const uint64_t below = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const uint64_t m = w.ballot(sel[j]);
    const int at = base + __builtin_popcountll(m & below);
    pos[j] = sel[j] && at < keep ? at : -1;
    base += __builtin_popcountll(m);
  }
}

}  // namespace lcsa
