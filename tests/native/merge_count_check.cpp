// Host check of the in-launch decode merge counter (merge_count.h): the
// packing never carries between fields up to 127 splits, the last arriver is
// found exactly once, the one-XCD test accepts equal offsets and rejects any
// mix, and no value reachable from a zeroed counter is taken for stale.
// Prints "ok" and exits 0 on success.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "merge_count.h"

using namespace qa;

static int fails = 0;
#define CHECK(c, ...)                \
  do {                               \
    if (!(c)) {                      \
      if (fails < 20) {              \
        std::printf("FAIL %s: ", #c); \
        std::printf(__VA_ARGS__);    \
        std::printf("\n");           \
      }                              \
      ++fails;                       \
    }                                \
  } while (0)

// Arrivals with offsets ds (in arrival order) on a zeroed counter.  Returns
// whether the last arriver's one-XCD test passed; checks every step.
static bool run(const std::vector<unsigned>& ds) {
  const unsigned ns = (unsigned)ds.size();
  unsigned w = 0;
  int n_last = 0;
  bool one = false;
  unsigned sum = 0, sum2 = 0;
  for (unsigned i = 0; i < ns; ++i) {
    const unsigned old = w;
    w += merge_count_add(ds[i]);
    sum += ds[i];
    sum2 += ds[i] * ds[i];
    CHECK(merge_count_valid(old, ns), "ns=%u i=%u old=%08x", ns, i, old);
    CHECK(merge_count_n(w) == i + 1 && merge_count_dsum(w) == sum &&
              merge_count_d2sum(w) == sum2,
          "fields ns=%u i=%u w=%08x", ns, i, w);
    if (merge_count_last(old, ns)) {
      ++n_last;
      one = merge_count_one_xcd(w, ns, ds[i]);
    }
  }
  CHECK(n_last == 1, "ns=%u: %d last arrivers", ns, n_last);
  return one;
}

int main() {
  // equal offsets: every split count, every offset (d = 7, ns = 127: the
  // largest field values, 889 and 6223)
  for (unsigned ns = 1; ns <= (unsigned)kInlineMaxSplits; ++ns)
    for (unsigned d = 0; d < 8; ++d)
      CHECK(run(std::vector<unsigned>(ns, d)), "equal offsets rejected ns=%u d=%u", ns, d);
  {
    unsigned w = 0;
    for (int i = 0; i < kInlineMaxSplits; ++i) w += merge_count_add(7);
    CHECK(merge_count_n(w) == 127 && merge_count_dsum(w) == 889 &&
              merge_count_d2sum(w) == 6223 && (w >> 30) == 0,
          "field bounds w=%08x", w);
  }
  // every mix of offsets for up to 4 splits, in every arrival order
  for (unsigned ns = 2; ns <= 4; ++ns) {
    unsigned total = 1;
    for (unsigned i = 0; i < ns; ++i) total *= 8;
    for (unsigned code = 0; code < total; ++code) {
      std::vector<unsigned> ds(ns);
      unsigned c = code;
      bool mixed = false;
      for (unsigned i = 0; i < ns; ++i) {
        ds[i] = c & 7u;
        c >>= 3;
        mixed |= ds[i] != ds[0];
      }
      CHECK(run(ds) == !mixed, "ns=%u code=%u", ns, code);
    }
  }
  // random mixes, including a single odd one out, up to 127 splits
  std::mt19937 g(12345);
  for (int it = 0; it < 200000; ++it) {
    const unsigned ns = 2 + g() % (kInlineMaxSplits - 1);
    std::vector<unsigned> ds(ns);
    const unsigned base = g() % 8;
    for (auto& d : ds) d = base;
    if (it & 1) {
      ds[g() % ns] = (base + 1 + g() % 7) % 8;  // exactly one differs
    } else {
      for (auto& d : ds) d = g() % 8;
    }
    bool mixed = false;
    for (auto d : ds) mixed |= d != ds[0];
    CHECK(run(ds) == !mixed, "random ns=%u", ns);
  }
  // stale words: a count at or past n_split, or sums no zeroed counter
  // reaches, e.g. the bits of a float in [-1, 1] (a cos/sin table entry)
  for (unsigned ns = 1; ns <= (unsigned)kInlineMaxSplits; ++ns) {
    CHECK(!merge_count_valid(ns, ns), "count == ns accepted");
    CHECK(!merge_count_valid(0x7fu, ns), "count 127 accepted");
  }
  std::uniform_real_distribution<float> u(-1.f, 1.f);
  for (int it = 0; it < 100000; ++it) {
    const float f = u(g);
    unsigned w;
    std::memcpy(&w, &f, 4);
    if (w == 0u || w == 0x80000000u) continue;  // +-0 read as a zeroed counter
    CHECK(!merge_count_valid(w, 18), "float bits %08x accepted", w);
  }
  CHECK(!merge_count_valid(0x3f800000u, 18), "1.0f accepted");
  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
