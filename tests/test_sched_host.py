"""Host check of the multi-token step's tile arithmetic (csrc/pkv_sched.h):
the floor-sum and the per-group block prefix sums against brute force,
compiled with the host C++ compiler (no GPU)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "paged_kv_gqa_cache_amd", "csrc")

CHECK = r"""
#include "pkv_sched.h"
#include <cstdio>
int main() {
  long bad = 0, checks = 0;
  for (int64_t n = 0; n <= 40; ++n)
    for (int64_t m = 1; m <= 40; ++m)
      for (int64_t a = 0; a <= 45; ++a)
        for (int64_t b = 0; b <= 45; b += 3) {
          int64_t want = 0;
          for (int64_t i = 0; i < n; ++i) want += (a * i + b) / m;
          ++checks;
          if (pkv::floor_sum(n, m, a, b) != want) ++bad;
        }
  // large operands (block counts of 32768-token contexts)
  for (int64_t n = 1000; n <= 1010; ++n) {
    int64_t want = 0;
    for (int64_t i = 0; i < n; ++i) want += (37 * i + 5000) / 16;
    ++checks;
    if (pkv::floor_sum(n, 16, 37, 5000) != want) ++bad;
  }
  for (int L = 1; L <= 300; ++L)
    for (int n = 0; n <= L; n += (n < 40 ? 1 : 7))
      for (int tpg = 1; tpg <= 34; ++tpg) {
        const int groups = pkv::num_groups(n, tpg);
        int64_t acc = 0;
        for (int g = 0; g <= groups; ++g) {
          // group g reads the blocks up to its last row's position
          if (g < groups) {
            const int last = (L - n) + ((g + 1) * tpg < n ? (g + 1) * tpg : n) - 1;
            ++checks;
            if (pkv::group_tiles(L, n, tpg, g) != last / 16 + 1) ++bad;
          }
          ++checks;
          if (pkv::group_prefix(L, n, tpg, g) != acc) ++bad;
          if (g < groups) acc += pkv::group_tiles(L, n, tpg, g);
        }
      }
  printf("%ld checks, %ld wrong\n", checks, bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_group_tiles_and_prefix_sums_match_brute_force(tmp_path):
    src = tmp_path / "check.cpp"
    src.write_text(CHECK)
    exe = tmp_path / "check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert ", 0 wrong" in r.stdout
