// pkv_sched.h - tile counts of the multi-token step's work items, shared by
// its balanced (tile-stream) kernel and its merge.  Plain C++ (constexpr
// functions are usable from device code), so host tests compile it too.
//
// A sequence with L context positions and n new query rows (its last n
// positions, base = L - n) is cut into groups of tpg consecutive query rows.
// Group g reads the blocks up to its last row's position: with
// e = min(n, (g + 1) * tpg), that is ceil((base + e) / 16) blocks of 16
// positions (causal attention: a row sees the positions up to its own).
#pragma once
#include <stdint.h>

namespace pkv {

// Sum over i = 0 .. n - 1 of floor((a * i + b) / m), for n >= 0, m >= 1,
// a >= 0, b >= 0, by the Euclid-like reduction: split off the integer parts
// of a / m and b / m (closed-form sums), then count the lattice points under
// the remaining line with the roles of the axes swapped, which replaces
// (m, a) by (a, m mod a) as in Euclid's algorithm, so the loop runs
// O(log m) times.
constexpr int64_t floor_sum(int64_t n, int64_t m, int64_t a, int64_t b) {
  int64_t total = 0;
  while (n > 0) {
    if (a >= m) {
      total += (a / m) * (n * (n - 1) / 2);
      a %= m;
    }
    if (b >= m) {
      total += (b / m) * n;
      b %= m;
    }
    // Now a, b < m.  The terms are the numbers of integers k >= 1 with
    // k * m <= a * i + b, i < n; the largest value a * (n - 1) + b < m * n.
    const int64_t top = a * n + b;   // floor(top / m) lattice rows are crossed
    if (top < m) break;
    // Counting by rows: row k (k = 1 .. floor(top / m)) holds the i with
    // a * i >= k * m - b, i.e. n - ceil((k * m - b) / a) of them; that sum
    // is again of this form, with the axes swapped.
    n = top / m;
    b = top % m;
    const int64_t t = m;
    m = a;
    a = t;
  }
  return total;
}

// Blocks group g reads (0 <= g < groups; tpg >= 1, 0 <= n <= L).
constexpr int group_tiles(int L, int n, int tpg, int g) {
  const int e = (n < (g + 1) * tpg) ? n : (g + 1) * tpg;
  return (L - n + e + 15) / 16;
}

// Blocks read by groups 0 .. g - 1 (g <= number of groups).  The full groups
// (g' < n / tpg) read floor((tpg * g' + base + tpg + 15) / 16) blocks, a
// floor-sum; a last, partial group reads ceil(L / 16).
constexpr int64_t group_prefix(int L, int n, int tpg, int g) {
  const int full = n / tpg;
  const int k = g < full ? g : full;
  int64_t s = floor_sum(k, 16, tpg, static_cast<int64_t>(L - n) + tpg + 15);
  if (g > full) s += (L + 15) / 16;
  return s;
}

// Number of groups of n rows.
constexpr int num_groups(int n, int tpg) { return (n + tpg - 1) / tpg; }

}  // namespace pkv
