// Host check of the decode's partial-slot bookkeeping (csrc/slots.hpp)
// against brute-force ownership.  Built with g++ with the device qualifiers
// defined away; prints "ok" and exits 0 when every check holds.
//
// Balanced split: W units (every segment's cost units, then its real units)
// over N workgroups, workgroup w owning [w W / N, (w+1) W / N).  A workgroup
// visits the segments its range meets in order, starting with the one that
// holds its first unit; a piece is the part of a segment's real units in its
// range, stored at slot 2 w for the first segment visited and 2 w + 1 after.
// Persistent split-K: I items over N workgroups, each storing one partial
// per segment at the slot of its first item there.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "slots.hpp"

using pkv::BalancedSlots;
using pkv::RunSlots;
using pkv::SplitSlots;

static int failures = 0;
#define EXPECT(c, ...)                      \
  do {                                      \
    if (!(c)) {                             \
      if (failures < 10) {                  \
        std::printf("FAIL %s: ", #c);       \
        std::printf(__VA_ARGS__);           \
        std::printf("\n");                  \
      }                                     \
      ++failures;                           \
    }                                       \
  } while (0)

struct Seg {
  long long Sv, S, E;  // cost units from Sv, real units [S, E)
};

// Every segment with at least one real unit gets C cost units in front.
static std::vector<Seg> layout(const std::vector<int>& nb, int C, long long& W) {
  std::vector<Seg> segs;
  W = 0;
  for (int n : nb) {
    if (n == 0) continue;
    segs.push_back({W, W + C, W + C + n});
    W += C + n;
  }
  return segs;
}

// brute force: per segment, the (workgroup, slot) of every piece that is not
// the whole segment, in workgroup order
static std::vector<std::vector<std::pair<int, int>>> balanced_pieces(const std::vector<Seg>& segs,
                                                                     long long W, int N) {
  std::vector<std::vector<std::pair<int, int>>> out(segs.size());
  for (int w = 0; w < N; ++w) {
    const long long a0 = (long long)w * W / N, a1 = (long long)(w + 1) * W / N;
    if (a0 >= a1) continue;
    bool first = true;
    for (size_t i = 0; i < segs.size(); ++i) {
      const Seg& s = segs[i];
      if (s.E <= a0) continue;
      if (s.Sv >= a1) break;
      const long long lo = a0 > s.S ? a0 : s.S, hi = a1 < s.E ? a1 : s.E;
      if (lo < hi && !(lo == s.S && hi == s.E)) out[i].push_back({w, first ? 2 * w : 2 * w + 1});
      first = false;
    }
  }
  return out;
}

static void check_balanced(const std::vector<int>& nb, int C, int N) {
  long long W;
  const std::vector<Seg> segs = layout(nb, C, W);
  if (W == 0) return;
  const auto pieces = balanced_pieces(segs, W, N);
  std::set<int> used;
  for (size_t i = 0; i < segs.size(); ++i) {
    const auto& pc = pieces[i];
    if (pc.empty()) continue;  // one workgroup holds the whole segment: no slots
    EXPECT(pc.size() >= 2, "a split segment with one piece (W %lld N %d seg %zu)", W, N, i);
    const BalancedSlots sl(W, segs[i].S, segs[i].E, segs[i].Sv, N);
    EXPECT(sl.count() == (int)pc.size(), "count %d, brute force %zu (W %lld N %d seg %zu)",
           sl.count(), pc.size(), W, N, i);
    for (int k = 0; k < sl.count() && k < (int)pc.size(); ++k) {
      int s = -1;
      sl.slot(k, s);
      EXPECT(s == pc[k].second, "slot %d of seg %zu: %d, brute force %d (W %lld N %d)", k, i, s,
             pc[k].second, W, N);
      EXPECT(s >= 0 && s < 2 * N, "slot %d out of [0, 2N)", s);
      EXPECT(used.insert(s).second, "slot %d used twice (W %lld N %d)", s, W, N);
    }
  }
}

static void check_runs(const std::vector<int>& nparts, int NP, int N, std::mt19937& rng) {
  long long I = 0;
  std::vector<long long> S;
  for (int n : nparts) {
    S.push_back(I);
    I += n;
  }
  if (I == 0) return;
  for (size_t seg = 0; seg < nparts.size(); ++seg) {
    const int n = nparts[seg];
    if (n == 0) continue;
    const int p_lo = (int)(rng() % (unsigned)(NP - n + 1));
    const int base = (int)seg * NP + p_lo;
    const long long s0 = S[seg], e0 = s0 + n;
    std::vector<int> want;
    for (int w = 0; w < N; ++w) {
      const long long i0 = (long long)w * I / N, i1 = (long long)(w + 1) * I / N;
      const long long lo = i0 > s0 ? i0 : s0, hi = i1 < e0 ? i1 : e0;
      if (lo < hi) want.push_back(base + (int)(lo - s0));
    }
    const RunSlots sl(I, s0, e0, N, base);
    EXPECT(sl.count() == (int)want.size(), "run count %d, brute force %zu (I %lld N %d)", sl.count(),
           want.size(), I, N);
    std::set<int> used;
    for (int k = 0; k < sl.count() && k < (int)want.size(); ++k) {
      int s = -1;
      sl.slot(k, s);
      EXPECT(s == want[k], "run slot %d: %d, brute force %d", k, s, want[k]);
      EXPECT(s >= (int)seg * NP + p_lo && s < (int)seg * NP + p_lo + n, "run slot %d outside its segment", s);
      EXPECT(used.insert(s).second, "run slot %d used twice", s);
    }
  }
}

int main() {
  std::mt19937 rng(20240611u);
  auto pick = [&](int lo, int hi) { return lo + (int)(rng() % (unsigned)(hi - lo + 1)); };
  long long trials = 0;
  // balanced: ragged batches with empty segments, cost units 0 .. 12,
  // workgroup counts from 1 to past the unit total
  for (int t = 0; t < 4000; ++t) {
    const int nseg = pick(1, 40);
    std::vector<int> nb(nseg);
    for (int& n : nb) n = rng() % 5 == 0 ? 0 : pick(1, t % 3 == 0 ? 3 : 60);
    const int C = pick(0, 12);
    const int N = t % 4 == 0 ? pick(1, 8) : pick(1, 600);
    check_balanced(nb, C, N);
    ++trials;
  }
  // the exact boundary W == N and W == N +- 1
  for (int n = 1; n <= 64; ++n)
    for (int dn = -1; dn <= 1; ++dn) {
      std::vector<int> nb(n, 1);
      if (n + dn >= 1) check_balanced(nb, 0, n + dn);
      ++trials;
    }
  // persistent split-K runs
  for (int t = 0; t < 4000; ++t) {
    const int nseg = pick(1, 30), NP = pick(1, 70);
    std::vector<int> np(nseg);
    for (int& n : np) n = rng() % 6 == 0 ? 0 : pick(1, NP);
    check_runs(np, NP, t % 3 == 0 ? pick(1, 8) : pick(1, 800), rng);
    ++trials;
  }
  // fixed partitions
  for (int p_lo = 0; p_lo < 8; ++p_lo)
    for (int p_hi = p_lo; p_hi < 12; ++p_hi) {
      const SplitSlots sl{100, p_lo, p_hi};
      EXPECT(sl.count() == p_hi - p_lo + 1, "split count");
      for (int k = 0; k < sl.count(); ++k) {
        int s = -1;
        sl.slot(k, s);
        EXPECT(s == 100 + p_lo + k, "split slot");
      }
    }
  if (failures) {
    std::printf("%d failures in %lld trials\n", failures, trials);
    return 1;
  }
  std::printf("ok %lld trials\n", trials);
  return 0;
}
