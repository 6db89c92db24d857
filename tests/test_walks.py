"""Host check of the persistent grids' work walks (csrc/lora_plan.h): for
every grid size and item totals tried, the waves' walks take every shrink and
expand item exactly once, the launch grid never exceeds the resident
work-groups it is given, and the item decoder's divider is exact.  The single-launch apply kernel relies on this: a
wave finishes all of its shrink items before it arrives at the phase
barrier, so once every work-group of the grid has arrived, every shrink item
(every partial sum of v) has been written.  Compiled with the host compiler
from the same header the kernels use; no GPU needed."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SRC = r"""
#include <cstdio>
#include <vector>
#include "lora_plan.h"
using namespace lora;
static int bad = 0;
static void expect_once(const std::vector<int>& hits, const char* what, int grid, int tm, int tv) {
  for (size_t i = 0; i < hits.size(); ++i)
    if (hits[i] != 1) {
      if (bad < 10) printf("FAIL %s item %zu taken %d times (grid %d, mfma %d, valu %d)\n", what, i, hits[i], grid, tm, tv);
      ++bad;
      return;
    }
}
static void shrink(int grid, int tm, int tv) {
  std::vector<int> hm(tm, 0), hv(tv, 0);
  for (int b = 0; b < grid; ++b)
    for (int w = 0; w < kWaves; ++w) {
      int Wm, R;
      shrink_walk_split(tm, tv, w, grid, b, Wm, R);
      for (WaveWalk it(tm, w, kWaves, grid, b); it.i < it.end; it.i += it.stride) hm[it.i]++;
      TwoClassWalk iv(tv, Wm, R, w, grid, b);
      for (int i = iv.i; i < iv.end; i = iv.next()) { hv[i]++; iv.i = i; }
    }
  expect_once(hm, "shrink mbgmm", grid, tm, tv);
  expect_once(hv, "shrink mbgmv", grid, tm, tv);
}
static void expand(int grid, int tm, int tv) {
  std::vector<int> hm(tm, 0), hv(tv, 0);
  for (int b = 0; b < grid; ++b) {
    const ExpandSplit es = expand_walk_split(tm, tv, grid, b);
    for (int i = es.first; i < es.end_m; i += es.step) hm[i]++;
    for (int w = 0; w < kWaves; ++w) {
      TwoClassWalk it(tv, es.Gm * kWaves, es.R, w, grid, b);
      for (int i = it.i; i < it.end; i = it.next()) { hv[i]++; it.i = i; }
    }
  }
  expect_once(hm, "expand mbgmm", grid, tm, tv);
  expect_once(hv, "expand mbgmv", grid, tm, tv);
}
static void grid(int resident, long long bound) {
  const int g = launch_grid(resident, bound);
  const int res = resident < 1 ? 1 : resident;
  const long long want = bound < 1 ? 1 : bound;
  const long long need = want < res ? want : res;
  // resident, a multiple of 8 whenever 8 fit, and short of the items' bound
  // (or of the resident count) by less than 8
  const bool ok = g >= 1 && g <= res && (res < 8 || g % 8 == 0) && g > need - 8;
  if (!ok) {
    if (bad < 10) printf("FAIL launch_grid(%d, %lld) = %d\n", resident, bound, g);
    ++bad;
  }
}
static void fastdiv(int d, int n) {
  const FastDiv f(d);
  if (f.div(n) != n / d) {
    if (bad < 10) printf("FAIL FastDiv %d / %d = %d, want %d\n", n, d, f.div(n), n / d);
    ++bad;
  }
}
int main() {
  for (int d = 1; d <= 3000; ++d) {
    for (int n = 0; n <= 3 * d + 5; ++n) fastdiv(d, n);
    for (int n : {1 << 20, (1 << 30) - 1, 1 << 30, 2147483647, 2147483647 - d, 2147483646}) fastdiv(d, n);
  }
  unsigned long long x = 88172645463325252ull;
  for (int k = 0; k < 2000000; ++k) {  // xorshift draws of large divisors and dividends
    x ^= x << 13; x ^= x >> 7; x ^= x << 17;
    const int d = 1 + (int)((x >> 5) % 2147483647u), n = (int)((x >> 33) & 0x7fffffff);
    fastdiv(d, n);
    fastdiv(1 + (int)(x % 100000), n);
  }
  for (int d : {1, 2, 3, 7, 1 << 30, 2147483647}) fastdiv(d, 2147483647);
  for (int r = 0; r <= 2100; ++r)
    for (long long b : {-1LL, 0LL, 1LL, 5LL, 7LL, 8LL, 9LL, 100LL, 767LL, 768LL, 769LL, 2047LL, 5000LL, 1LL << 40})
      grid(r, b);
  const int grids[] = {1, 3, 8, 16, 24, 40, 64, 96, 256, 768, 1280, 2048};
  const int totals[] = {0, 1, 5, 7, 8, 9, 63, 64, 100, 777, 4096, 20000, 150000};
  for (int g : grids)
    for (int tm : totals)
      for (int tv : totals) {
        shrink(g, tm, tv);
        expand(g, tm, tv);
      }
  printf(bad ? "FAILED\n" : "OK\n");
  return bad != 0;
}
"""


def test_walks_take_every_item_exactly_once(tmp_path):
    src = tmp_path / "walks.cpp"
    src.write_text(SRC)
    exe = tmp_path / "walks"
    inc = os.path.join(ROOT, "heterogeneous_adapters_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O2", f"-I{inc}", str(src), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout[-2000:]
