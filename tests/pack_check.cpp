// Host check of the backward's tile packing (lce::pack_tiles), built with g++
// against lce_contract.cpp by tests/test_host_planner.py.
//
// For each case it replays the walk a packed launch makes on the device --
// slot b = 8 s + x of XCD x runs c[b][j] tiles of product j, starting after
// the tiles of product j that the XCD's earlier slots run, inside the XCD's
// contiguous range of that product's logical tiles -- and checks that every
// logical tile of every product runs exactly once, that no count overflows,
// and that the reported makespan is the busiest slot's modelled load and
// lies between the lower bound and the target at which best fit cannot fail.
// A packing that needs more than 255 tiles of one product on a slot is
// refused (the launch then keeps hardware dispatch).
// Prints "ok <cases> <packed> <refused>" or the first failing case.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "lce_internal.h"

namespace {

constexpr int kXcds = 8, kSlots = 256, kPerXcd = kSlots / kXcds;

// first logical tile of XCD x when n tiles are dealt to 8 XCDs in contiguous
// ranges, the larger ranges first (the device kernel's rule)
int64_t range_lo(int64_t n, int x) {
  const int64_t q = n / kXcds, r = n % kXcds;
  return x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
}

bool check(const int64_t n[3], const double dur[3], int *packed, int *refused) {
  lce::PackCounts pc;
  int slots = -1;
  double ms = -1.0;
  if (!lce::pack_tiles(n, dur, &pc, &slots, &ms)) {   // hardware dispatch instead
    ++*refused;
    return true;
  }
  ++*packed;
  for (int j = 0; j < 3; ++j) {
    std::vector<int> hits(size_t(n[j]), 0);
    for (int b = 0; b < kSlots; ++b) {
      const int x = b % kXcds, s = b / kXcds;
      int64_t off = 0;
      for (int t = 0; t < s; ++t) off += pc.c[kXcds * t + x][j];
      const int64_t lo = range_lo(n[j], x), hi = range_lo(n[j], x + 1);
      for (int i = 0; i < pc.c[b][j]; ++i) {
        const int64_t ls = lo + off + i;
        if (ls >= hi) {
          std::printf("FAIL n=%lld,%lld,%lld product %d slot %d runs past its XCD range\n",
                      (long long)n[0], (long long)n[1], (long long)n[2], j, b);
          return false;
        }
        ++hits[size_t(ls)];
      }
    }
    for (int64_t t = 0; t < n[j]; ++t)
      if (hits[size_t(t)] != 1) {
        std::printf("FAIL n=%lld,%lld,%lld product %d tile %lld runs %d times\n",
                    (long long)n[0], (long long)n[1], (long long)n[2], j, (long long)t,
                    hits[size_t(t)]);
        return false;
      }
  }
  // the makespan is the busiest slot's load (a tile costs dur + 1), at least
  // the lower bound, and at most the target at which best fit cannot fail
  // (an XCD's load / 32 + its longest tile) within the 0.5% to which the
  // target is bisected
  double worst = 0.0, lb = 0.0, ub = 0.0;
  int most = 0;
  for (int x = 0; x < kXcds; ++x) {
    double total = 0.0, longest = 0.0;
    int used = 0;
    for (int s = 0; s < kPerXcd; ++s) {
      const int b = kXcds * s + x;
      double load = 0.0;
      for (int j = 0; j < 3; ++j) load += double(pc.c[b][j]) * (dur[j] + 1.0);
      if (load > worst) worst = load;
      if (load > 0.0) ++used;
      total += load;
    }
    if (used > most) most = used;
    if (total / kPerXcd > lb) lb = total / kPerXcd;
    for (int j = 0; j < 3; ++j)
      if (range_lo(n[j], x + 1) > range_lo(n[j], x) && dur[j] + 1.0 > longest)
        longest = dur[j] + 1.0;
    if (longest > lb) lb = longest;
    if (total / kPerXcd + longest > ub) ub = total / kPerXcd + longest;
  }
  if (std::fabs(worst - ms) > 1e-9 * (1.0 + ms) || ms < lb * (1.0 - 1e-12) ||
      ms > ub * 1.005 * (1.0 + 1e-12) || slots != most || slots > kPerXcd) {
    std::printf("FAIL n=%lld,%lld,%lld dur=%g,%g,%g makespan %g (busiest %g, bounds %g..%g) "
                "slots %d (used %d)\n",
                (long long)n[0], (long long)n[1], (long long)n[2], dur[0], dur[1], dur[2], ms,
                worst, lb, ub, slots, most);
    return false;
  }
  return true;
}

}  // namespace

int main() {
  // tile counts of the headline launches and of edge shapes: empty products,
  // fewer tiles than XCDs, ragged XCD ranges, more tiles than slots
  const int64_t counts[] = {0, 1, 7, 8, 9, 31, 32, 33, 100, 128, 144, 255, 256, 257, 288, 513,
                            1000, 2047, 4097};
  const double durs[][3] = {{71.9, 52.7, 33.5}, {33.5, 52.7, 71.9}, {10.0, 10.0, 10.0},
                            {120.0, 3.0, 40.0}, {0.5, 200.0, 7.0}};
  int cases = 0, packed = 0, refused = 0;
  for (const auto &d : durs)
    for (int64_t a : counts)
      for (int64_t b : counts)
        for (int64_t c : counts) {
          const int64_t n[3] = {a, b, c};
          ++cases;
          if (!check(n, d, &packed, &refused)) return 1;
        }
  // seeded random shapes and durations
  std::srand(12345);
  for (int i = 0; i < 3000; ++i) {
    int64_t n[3];
    double d[3];
    for (int j = 0; j < 3; ++j) {
      n[j] = std::rand() % 1200;
      d[j] = 1.0 + double(std::rand() % 20000) / 100.0;
    }
    ++cases;
    if (!check(n, d, &packed, &refused)) return 1;
  }
  // the 255-tile limit of a slot's count: 255 per slot packs, one more
  // tile of a product on every XCD's busiest slot does not
  const double d3[3] = {10.0, 10.0, 10.0};
  const int64_t limits[][3] = {{65280, 0, 0}, {65288, 0, 0}, {0, 65280, 8}};
  for (const auto &n : limits) {
    ++cases;
    if (!check(n, d3, &packed, &refused)) return 1;
  }
  std::printf("ok %d %d %d\n", cases, packed, refused);
  return 0;
}
