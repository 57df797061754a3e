// Host check of the select kernel's per-row top-k (csrc/topk_wave.h).
//
// A wave is emulated by 64 threads, one per lane, that meet at a barrier for
// every cross-lane operation, so the exact device code of the selection runs
// on the CPU under the undefined-behaviour and address checks.  Each case
// mirrors the kernel's row: keep = min(k, n); a window no longer than keep is
// kept whole, otherwise topk_select picks the keep best and kept_positions
// places them.  The result must equal a brute-force stable sort by (score
// descending, candidate index ascending) and fill exactly positions
// 0 .. keep-1, each once.  Prints one line per failure and exits non-zero on
// any.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>
#include <thread>
#include <vector>

#include "topk_wave.h"

namespace {

constexpr int kLanes = 64;

// Sense-reversing barrier; waiting threads yield, since the 64 lanes share
// a few cores.
class Barrier {
 public:
  void arrive_and_wait() {
    const bool sense = !sense_.load(std::memory_order_relaxed);
    if (count_.fetch_add(1, std::memory_order_acq_rel) == kLanes - 1) {
      count_.store(0, std::memory_order_relaxed);
      sense_.store(sense, std::memory_order_release);
    } else {
      while (sense_.load(std::memory_order_acquire) != sense) std::this_thread::yield();
    }
  }

 private:
  std::atomic<int> count_{0};
  std::atomic<bool> sense_{false};
};

struct Shared {
  Barrier bar;
  uint64_t v0[kLanes];
  uint64_t v1[kLanes];
};

// One lane's view of the emulated wave: every operation writes the lane's
// value, waits for all lanes, combines, and waits again so that the next
// operation cannot overwrite a value another lane is still reading.
struct HostWave {
  Shared* sh;
  int lane;
  uint64_t ballot(bool pred) {
    sh->v0[lane] = pred ? 1u : 0u;
    sh->bar.arrive_and_wait();
    uint64_t m = 0;
    for (int i = 0; i < kLanes; ++i) m |= (sh->v0[i] & 1ull) << i;
    sh->bar.arrive_and_wait();
    return m;
  }
  void or_and(uint64_t& o, uint64_t& a) {
    sh->v0[lane] = o;
    sh->v1[lane] = a;
    sh->bar.arrive_and_wait();
    uint64_t ro = 0, ra = ~0ull;
    for (int i = 0; i < kLanes; ++i) {
      ro |= sh->v0[i];
      ra &= sh->v1[i];
    }
    sh->bar.arrive_and_wait();
    o = ro;
    a = ra;
  }
};

struct Case {
  const char* what;
  std::vector<double> s;   // window scores, candidate order
  int k;
};

template <int M>
void lane_row(Shared* sh, int lane, const Case& c, std::vector<std::atomic<int>>* out,
              std::atomic<int>* bad_pos) {
  HostWave w{sh, lane};
  const int n = static_cast<int>(c.s.size());
  const int keep = std::min(c.k, n);
  bool valid[M], sel[M];
  uint64_t key[M];
  for (int j = 0; j < M; ++j) {
    const int e = lane + kLanes * j;
    valid[j] = e < n;
    key[j] = valid[j] ? lcsa::order_key(c.s[e]) : 0ull;
  }
  if (keep >= n) {
    for (int j = 0; j < M; ++j) sel[j] = valid[j];
  } else {
    lcsa::topk_select<M>(w, lane, key, valid, keep, sel);
  }
  int pos[M];
  lcsa::kept_positions<M>(w, lane, sel, keep, pos);
  for (int j = 0; j < M; ++j) {
    if (pos[j] < 0) continue;
    if (pos[j] >= keep) {
      bad_pos->fetch_add(1);
      continue;
    }
    int expect = -1;
    if (!(*out)[pos[j]].compare_exchange_strong(expect, lane + kLanes * j)) bad_pos->fetch_add(1);
  }
}

template <int M>
bool run_case(const Case& c) {
  const int n = static_cast<int>(c.s.size());
  const int keep = std::min(c.k, n);
  Shared sh;
  std::vector<std::atomic<int>> out(keep > 0 ? keep : 1);
  for (auto& x : out) x = -1;
  std::atomic<int> bad_pos{0};
  std::vector<std::thread> th;
  for (int l = 0; l < kLanes; ++l) th.emplace_back(lane_row<M>, &sh, l, std::cref(c), &out, &bad_pos);
  for (auto& t : th) t.join();

  std::vector<int> idx(n);
  for (int i = 0; i < n; ++i) idx[i] = i;
  std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return c.s[a] > c.s[b]; });
  std::vector<int> want(idx.begin(), idx.begin() + keep);
  std::sort(want.begin(), want.end());
  bool ok = bad_pos.load() == 0;
  for (int i = 0; i < keep && ok; ++i) ok = out[i].load() == want[i];
  if (!ok) {
    std::printf("FAIL %s: n=%d k=%d M=%d bad_pos=%d got", c.what, n, c.k, M, bad_pos.load());
    for (int i = 0; i < keep && i < 12; ++i) std::printf(" %d", out[i].load());
    std::printf(" want");
    for (int i = 0; i < keep && i < 12; ++i) std::printf(" %d", want[i]);
    std::printf("\n");
  }
  return ok;
}

// The compiled candidate widths of the select kernel.
bool run(const Case& c) {
  const int m = (static_cast<int>(c.s.size()) + kLanes - 1) / kLanes;
  if (m <= 1) return run_case<1>(c);
  if (m <= 2) return run_case<2>(c);
  if (m <= 3) return run_case<3>(c);
  if (m <= 4) return run_case<4>(c);
  if (m <= 6) return run_case<6>(c);
  if (m <= 8) return run_case<8>(c);
  if (m <= 12) return run_case<12>(c);
  return run_case<16>(c);
}

}  // namespace

int main() {
  std::vector<Case> cases;
  const double inf = std::numeric_limits<double>::infinity();
  // Every score equal (a query block whose pooled query is zero, or a window
  // of identical pooled keys): no bit differs between the keys.
  for (int n : {2, 5, 63, 64, 65, 130, 180, 726, 1024})
    for (double v : {0.0, -0.0, 1.5, -3.25, 1e-300, -inf})
      for (int k : {1, n / 2, n - 1, n, n + 7})
        cases.push_back({"all equal", std::vector<double>(n, v), std::max(k, 1)});
  // Zeros of both signs: the same score.
  {
    std::vector<double> s(180);
    for (int i = 0; i < 180; ++i) s[i] = (i % 3) ? 0.0 : -0.0;
    for (int k : {1, 45, 60, 179}) cases.push_back({"signed zeros", s, k});
  }
  // One candidate; two equal candidates.
  cases.push_back({"single candidate", {0.75}, 1});
  cases.push_back({"single candidate, k past it", {-2.0}, 4});
  cases.push_back({"two equal", {4.0, 4.0}, 1});
  std::mt19937_64 rng(12345);
  // Ties at the k-th score: few distinct values, so the k-th and (k+1)-th
  // (and many around them) coincide.
  for (int n : {3, 64, 90, 180, 242, 726, 968}) {
    for (int levels : {2, 3, 7}) {
      std::vector<double> s(n);
      std::uniform_int_distribution<int> d(0, levels - 1);
      for (auto& x : s) x = 0.5 * d(rng) - 1.0;
      for (int k : {1, 2, n / 3, n / 2, n - 2, n - 1})
        if (k >= 1) cases.push_back({"ties at the k-th score", s, k});
    }
  }
  // The k-th and (k+1)-th scores one ulp apart, the rest spread out.
  for (int n : {60, 180, 726}) {
    std::vector<double> s(n);
    std::normal_distribution<double> d(0.0, 10.0);
    for (auto& x : s) x = d(rng);
    std::vector<double> sorted = s;
    std::sort(sorted.rbegin(), sorted.rend());
    const int k = n / 3;
    const double kth = sorted[k - 1];
    for (auto& x : s)
      if (x == sorted[k]) x = std::nextafter(kth, -inf);
    cases.push_back({"one ulp at the k-th score", s, k});
  }
  // Distinct random scores of mixed sign and magnitude, and denormals.
  for (int n : {1, 17, 64, 100, 180, 600, 1024}) {
    std::vector<double> s(n);
    std::normal_distribution<double> d(0.0, 1.0);
    for (auto& x : s) x = d(rng) * std::ldexp(1.0, static_cast<int>(rng() % 40) - 20);
    for (int k : {1, 45, 60, n / 2 + 1}) cases.push_back({"random", s, k});
    std::vector<double> t(n);
    for (int i = 0; i < n; ++i) t[i] = (i % 2 ? -1 : 1) * 4.9e-324 * static_cast<double>(rng() % 4);
    cases.push_back({"denormals", t, std::max(1, n / 4)});
  }
  int fails = 0;
  for (const Case& c : cases) fails += run(c) ? 0 : 1;
  std::printf("%zu cases, %d failed\n", cases.size(), fails);
  return fails ? 1 : 0;
}
