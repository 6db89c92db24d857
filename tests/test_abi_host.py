"""Host-side tests of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status codes
before touching the device (these run without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from heterogeneous_adapters_amd import lora
from heterogeneous_adapters_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("lora.h", "lora_pool.h")]


def header_functions():
    txt = "\n".join(open(h).read() for h in HEADERS)
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(lora_[a-z_]+)\s*\(", txt, flags=re.M)))


def test_library_exports_every_declared_function():
    assert os.path.exists(LIB_PATH), "run __graft_entry__.build() first"
    L = ctypes.CDLL(LIB_PATH)
    fns = header_functions()
    assert set(fns) >= {"lora_build_segments", "lora_shrink", "lora_expand", "lora_apply",
                        "lora_workspace_size", "lora_status_string"}
    assert set(fns) == set(lora.EXPORTS)
    for f in fns:
        assert hasattr(L, f), f


def test_binding_constants_match_header():
    txt = open(HEADERS[0]).read()
    defs = dict(re.findall(r"^#define (LORA_[A-Z_0-9]+) \(?([^/\n]*?)\)?\s*(?:/\*.*)?$", txt, flags=re.M))
    for name in ("LORA_MAX_RANK", "LORA_MAX_ADAPTERS", "LORA_KSLICE", "LORA_DTYPE_F32", "LORA_DTYPE_BF16",
                 "LORA_MAX_TOKENS", "LORA_MAX_LAUNCH_ITEMS"):
        assert eval(defs[name].strip()) == getattr(lora, name), name
    # an adapter count past the limit is refused before any device work
    b = _Buf()
    s = lora.lora_segments_t()
    L = lora.lib()
    assert L.lora_segments_size(8, lora.LORA_MAX_ADAPTERS) > 0
    assert L.lora_segments_init(ctypes.c_void_p(b.p()), 1 << 14, 8, lora.LORA_MAX_ADAPTERS + 1, ctypes.byref(s)) == -1


def test_status_strings():
    L = lora.lib()
    for code in range(-8, 1):
        assert lora.lora_status_string(code) not in ("", "unknown status")
    assert lora.lora_status_string(-99) == "unknown status"
    ks = lora.LORA_KSLICE
    assert L.lora_v_slices(1) == 1 and L.lora_v_slices(ks) == 1 and L.lora_v_slices(ks + 1) == 2
    assert L.lora_v_slices(11008) == -(-11008 // ks) and L.lora_v_slices(0) == 0


def test_sizes():
    L = lora.lib()
    assert L.lora_segments_size(-1, 4) == 0 and L.lora_segments_size(4, 0) == 0
    s = L.lora_segments_size(1024, 1000)
    assert s >= 4 * (1024 + 4 * 1001 + 1000 + 8)
    w = L.lora_workspace_size(1024, 1000, 3, 4096)
    assert w >= s + 3 * lora.lora_v_slices(4096) * 1024 * 128 * 4
    # projections beyond one launch reuse the same v area
    assert L.lora_workspace_size(8, 4, 16, 256) == L.lora_workspace_size(8, 4, 40, 256)


class _Buf:
    """Host buffers whose addresses stand in for device pointers; every call
    below fails host-side validation, so nothing is dereferenced."""

    def __init__(self):
        self.a = np.zeros(4096, np.float32)
        self.base = self.a.ctypes.data
        assert self.base % 16 == 0

    def p(self, off=0):
        return self.base + off


def _descs(b, **kw):
    d = dict(T=8, N=4, d_in=64, d_out=64, pw=64, dtype=lora.LORA_DTYPE_BF16)
    d.update(kw)
    ad = lora.lora_adapters_t(b.p(), b.p(64), d["N"])
    pool = lora.lora_pool_t(kw.get("pool_base", b.p()), 4, d["pw"], d["dtype"])
    proj = lora.lora_proj_t(kw.get("X", b.p()), kw.get("ldx", d["d_in"]), b.p(), d["d_out"],
                            kw.get("Y", b.p(256)), kw.get("ldy", d["d_out"]), d["d_in"], d["d_out"],
                            b.p(), b.p(), b.p(), b.p())
    seg = lora.lora_segments_t()
    assert lora.lib().lora_segments_init(ctypes.c_void_p(b.p()), 1 << 14, d["T"], d["N"], ctypes.byref(seg)) == 0
    return ad, pool, proj, seg


@pytest.mark.parametrize("case,code", [
    (dict(d_in=60), -1), (dict(d_out=12), -1), (dict(ldx=32), -1), (dict(X=0), -1),
    (dict(pw=96), -6), (dict(pw=32), -6), (dict(dtype=7), -6),
    (dict(X="mis"), -7), (dict(ldy=68), -7), (dict(pool_base="mis"), -7),
])
def test_shrink_expand_apply_reject_bad_arguments(case, code):
    b = _Buf()
    kw = dict(case)
    if kw.get("X") == "mis":
        kw["X"] = b.p(2)
    if kw.get("pool_base") == "mis":
        kw["pool_base"] = b.p(4)
    ad, pool, proj, seg = _descs(b, **kw)
    L = lora.lib()
    r = ctypes.byref
    v = ctypes.c_void_p(b.p())
    vs = (ctypes.c_void_p * 1)(b.p())
    assert L.lora_shrink(r(proj), 1, r(ad), r(seg), r(pool), vs, 8 * 128, None) == code
    assert L.lora_expand(r(proj), 1, r(ad), r(seg), r(pool), vs, 1, 8 * 128, None) == code
    arr = (lora.lora_proj_t * 1)(proj)
    assert L.lora_apply(None, r(seg), 8, arr, 1, r(ad), r(pool), v, 1 << 30, None) == code


def test_other_rejections():
    b = _Buf()
    ad, pool, proj, seg = _descs(b)
    L = lora.lib()
    r = ctypes.byref
    v = ctypes.c_void_p(b.p())
    vs = (ctypes.c_void_p * 1)(b.p())
    # v_stride below T * 128
    assert L.lora_shrink(r(proj), 1, r(ad), r(seg), r(pool), vs, 8 * 127, None) == -1
    # v_slices < 0; no v array; a null v pointer; negative projection count
    assert L.lora_expand(r(proj), 1, r(ad), r(seg), r(pool), vs, -1, 8 * 128, None) == -1
    assert L.lora_expand(r(proj), 1, r(ad), r(seg), r(pool), None, 0, 8 * 128, None) == -1
    assert L.lora_shrink(r(proj), 1, r(ad), r(seg), r(pool), (ctypes.c_void_p * 1)(None), 8 * 128, None) == -1
    assert L.lora_shrink(r(proj), -1, r(ad), r(seg), r(pool), vs, 8 * 128, None) == -1
    arr = (lora.lora_proj_t * 1)(proj)
    # neither ids nor segments; T above the segment buffer's capacity;
    # workspace too small (T below the capacity is a valid call: a buffer laid
    # out for a larger batch serves a smaller one)
    assert L.lora_apply(None, None, 8, arr, 1, r(ad), r(pool), v, 1 << 30, None) == -1
    assert L.lora_apply(None, r(seg), 9, arr, 1, r(ad), r(pool), v, 1 << 30, None) == -1
    assert L.lora_apply(v, r(seg), 9, arr, 1, r(ad), r(pool), v, 1 << 30, None) == -1
    assert L.lora_apply(None, r(seg), 8, arr, 1, r(ad), r(pool), v, 64, None) == -4
    # adapters without rank array; too many adapters for the segment buffer
    bad = lora.lora_adapters_t(None, b.p(), 4)
    assert L.lora_apply(None, r(seg), 8, arr, 1, r(bad), r(pool), v, 1 << 30, None) == -1
    big = lora.lora_adapters_t(b.p(), b.p(), 5)
    assert L.lora_build_segments(v, 8, r(big), r(seg), v, 1 << 20, None) == -4
    assert L.lora_build_segments(v, 9, r(ad), r(seg), v, 1 << 20, None) == -4
    assert L.lora_build_segments(None, 8, r(ad), r(seg), v, 1 << 20, None) == -1
    assert L.lora_build_segments(v, 8, r(ad), r(seg), v, 4, None) == -4
    # Y aliasing Y_base with another leading dimension
    p2 = lora.lora_proj_t(b.p(), 64, b.p(512), 64, b.p(512), 72, 64, 64, b.p(), b.p(), b.p(), b.p())
    assert L.lora_shrink(r(p2), 1, r(ad), r(seg), r(pool), vs, 8 * 128, None) == -1
    # segment buffer: misaligned / too small
    s2 = lora.lora_segments_t()
    assert L.lora_segments_init(ctypes.c_void_p(b.p(4)), 1 << 14, 8, 4, r(s2)) == -7
    assert L.lora_segments_init(ctypes.c_void_p(b.p()), 16, 8, 4, r(s2)) == -4


def test_size_limits_refused_before_device_work():
    """Past LORA_MAX_TOKENS, or past LORA_MAX_LAUNCH_ITEMS in any launch group,
    every entry point returns UNSUPPORTED while validating its arguments (the
    descriptors point at host memory: nothing is dereferenced or launched)."""
    b = _Buf()
    L = lora.lib()
    r = ctypes.byref
    v = ctypes.c_void_p(b.p())
    vs = (ctypes.c_void_p * 16)(*([b.p()] * 16))
    ad = lora.lora_adapters_t(b.p(), b.p(64), 4)
    pool = lora.lora_pool_t(b.p(), 4, 512, lora.LORA_DTYPE_BF16)

    def proj(d_in, d_out):
        return lora.lora_proj_t(b.p(), d_in, b.p(), d_out, b.p(), d_out, d_in, d_out, b.p(), b.p(), b.p(), b.p())

    def segs(T):
        return lora.lora_segments_t(T, 4, *([b.p()] * 6))

    big = lora.LORA_MAX_TOKENS + 1
    assert L.lora_segments_size(big, 4) == 0 and L.lora_workspace_size(big, 4, 1, 4096) == 0
    assert L.lora_segments_size(lora.LORA_MAX_TOKENS, 4) > 0
    assert L.lora_segments_size(8, lora.LORA_MAX_ADAPTERS + 1) == 0
    s = lora.lora_segments_t()
    assert L.lora_segments_init(ctypes.c_void_p(b.p()), 1 << 14, big, 4, r(s)) == -6
    one = (lora.lora_proj_t * 1)(proj(4096, 4096))
    assert L.lora_build_segments(v, big, r(ad), r(segs(big)), v, 1 << 40, None) == -6
    assert L.lora_apply(v, None, big, one, 1, r(ad), r(pool), v, 1 << 40, None) == -6
    assert L.lora_shrink(one, 1, r(ad), r(segs(big)), r(pool), vs, big * 128, None) == -6
    assert L.lora_expand(one, 1, r(ad), r(segs(big)), r(pool), vs, 0, big * 128, None) == -6
    # 1M tokens: one 4096 x 4096 projection fits (the call goes on to the
    # workspace check); 16 projections of 4096 -> 11008 exceed the expand's
    # item limit, 16 of 11008 -> 4096 the shrink's
    T = 1 << 20
    assert L.lora_apply(v, None, T, one, 1, r(ad), r(pool), v, 64, None) == -4
    up = (lora.lora_proj_t * 16)(*[proj(4096, 11008)] * 16)
    down = (lora.lora_proj_t * 16)(*[proj(11008, 4096)] * 16)
    assert 16 * 22 * (6 * T + 2) > lora.LORA_MAX_LAUNCH_ITEMS
    assert 16 * 22 * (21 * T + 2) > lora.LORA_MAX_LAUNCH_ITEMS
    for arr in (up, down):
        assert L.lora_apply(v, None, T, arr, 16, r(ad), r(pool), v, 1 << 40, None) == -6
    assert L.lora_expand(up, 16, r(ad), r(segs(T)), r(pool), vs, 0, T * 128, None) == -6
    assert L.lora_shrink(down, 16, r(ad), r(segs(T)), r(pool), vs, T * 128, None) == -6
    # the second group of a 17-projection call is over the limit: refused
    # before the first group (or the segment build) is enqueued
    mix = (lora.lora_proj_t * 17)(*([proj(512, 512)] * 16 + [proj(11008, 4096)]))
    T2 = 2_800_000
    assert 22 * (21 * T2 + 2) > lora.LORA_MAX_LAUNCH_ITEMS >= 16 * 1 * (21 * T2 + 2)
    assert L.lora_apply(v, None, T2, mix, 17, r(ad), r(pool), v, 1 << 40, None) == -6


def test_validate_tables():
    import workloads as W
    ranks = np.array([8, 16, 40, 1], np.int32)
    tabs, npg = W.plan_tables(ranks, [("p", 300, 700)], 128, True, 3)
    t = tabs[0]
    ok = lora.lora_validate_tables(ranks, 300, 700, 128, npg, t.a_indptr, t.a_pages, t.b_indptr, t.b_pages)
    assert ok == 0
    bad = t.a_pages.copy()
    bad[3] = npg
    assert lora.lora_validate_tables(ranks, 300, 700, 128, npg, t.a_indptr, bad, t.b_indptr, t.b_pages) == -3
    r2 = ranks.copy()
    r2[1] = 129
    assert lora.lora_validate_tables(r2, 300, 700, 128, npg, t.a_indptr, t.a_pages, t.b_indptr, t.b_pages) == -2
    # table sized for another rank
    r3 = ranks.copy()
    r3[0] = 20
    assert lora.lora_validate_tables(r3, 300, 700, 128, npg, t.a_indptr, t.a_pages, t.b_indptr, t.b_pages) == -1


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(lora, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(lora, "_lib", None)
    with pytest.raises(ImportError):
        lora.lib()


PLAN_CHECK = r"""
#include <cstdio>
#include <cstdlib>
#include <vector>
#include <algorithm>
#include "lora_plan.h"
using namespace lora;
// Item totals of the tables for one batch, from the same per-segment item
// functions the segment builder uses.
static int check(int T, int N, const std::vector<int>& ids, const std::vector<int>& rank) {
  std::vector<int> cnt(N, 0);
  for (int t = 0; t < T; ++t) if (ids[t] >= 0 && ids[t] < N && rank[ids[t]] >= 1 && rank[ids[t]] <= 128) cnt[ids[t]]++;
  long long S = 0, sm = 0, sv = 0, em = 0, ev = 0;
  for (int a = 0; a < N; ++a) {
    if (!cnt[a]) continue;
    const int n = cnt[a], r = rank[a];
    ++S; sm += shrink_items_mfma(n, r); sv += shrink_items_valu(n, r);
    em += expand_items_mfma(n); ev += expand_items_valu(n, r);
  }
  const PlanLayout L = plan_layout(T, N);
  if (S > L.s_cap || sm > L.cap_shrink_mfma || sv > L.cap_shrink_valu || em > L.cap_expand_mfma ||
      ev > L.cap_expand_valu) {
    printf("FAIL T=%d N=%d S=%lld sm=%lld sv=%lld em=%lld ev=%lld\n", T, N, S, sm, sv, em, ev);
    return 1;
  }
  // the tables fit their regions, in order, inside the plan
  if (!(L.shrink_mfma >= 8 * L.s_cap && L.shrink_valu - L.shrink_mfma >= L.cap_shrink_mfma &&
        L.expand_mfma - L.shrink_valu >= kValuItemInts * L.cap_shrink_valu &&
        L.expand_valu - L.expand_mfma >= L.cap_expand_mfma &&
        L.total - L.expand_valu >= kValuItemInts * L.cap_expand_valu)) {
    printf("FAIL layout T=%d N=%d\n", T, N);
    return 1;
  }
  return 0;
}
int main() {
  srand(12345);
  int bad = 0;
  const int rk[] = {1, 8, 15, 16, 17, 31, 32, 33, 64, 100, 127, 128};
  for (int T : {1, 2, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1000, 1024, 4099}) {
    for (int N : {1, 2, 7, 64, 1000, 5000}) {
      for (int mode = 0; mode < 6; ++mode) {
        std::vector<int> rank(N), ids(T);
        for (int a = 0; a < N; ++a) rank[a] = mode == 0 ? 128 : mode == 1 ? 1 : rk[rand() % 12];
        for (int t = 0; t < T; ++t) {
          if (mode == 0 || mode == 1) ids[t] = t % N;           // as many segments as possible
          else if (mode == 2) ids[t] = 0;                        // one segment
          else if (mode == 3) ids[t] = (t / 16) % N;             // segments of 16 (MBGMM)
          else if (mode == 4) ids[t] = (t / 15) % N;             // segments of 15 (MBGMV)
          else ids[t] = rand() % (N + 2) - 1;                    // random, with base-only tokens
        }
        bad += check(T, N, ids, rank);
      }
    }
  }
  printf(bad ? "FAILED\n" : "OK\n");
  return bad != 0;
}
"""


def test_plan_capacities_bound_every_item_table(tmp_path):
    """The capacities the compute kernels check the segment buffer's counters
    against (plan_layout) bound the item totals of every batch the builder can
    produce, and the tables they size fit their regions of the plan.  Checked
    by compiling the plan header with the host compiler and counting items with
    the same per-segment functions the builder uses."""
    import subprocess
    src = tmp_path / "plan_check.cpp"
    src.write_text(PLAN_CHECK)
    exe = tmp_path / "plan_check"
    inc = os.path.join(ROOT, "heterogeneous_adapters_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", f"-I{inc}", str(src), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout


QUEUE_CHECK = r"""
#include <cstdio>
#include <vector>
#include "lora_plan.h"
using namespace lora;
int main() {
  int bad = 0;
  for (int sh : {0, 3}) {
    for (int total = 0; total < 3000; total += (total < 300 ? 1 : 37)) {
      std::vector<int> seen(total, 0);
      const int nx = 1 << sh;
      int sum = 0, lo = 1 << 30, hi = 0;
      for (int x = 0; x < nx; ++x) {
        const int m = xcd_block_items(total, x, sh);
        sum += m; lo = m < lo ? m : lo; hi = m > hi ? m : hi;
        for (int l = 0; l < m; ++l) {
          const int i = xcd_block_item(l, x, sh);
          if (i < 0 || i >= total) { printf("FAIL range sh=%d total=%d x=%d l=%d i=%d\n", sh, total, x, l, i); bad++; break; }
          // whole blocks of consecutive items stay on one XCD
          if ((i / kExpandItemBlock) % nx != x) { printf("FAIL xcd sh=%d total=%d\n", sh, total); bad++; break; }
          seen[i]++;
        }
      }
      for (int i = 0; i < total; ++i)
        if (seen[i] != 1) { printf("FAIL cover sh=%d total=%d i=%d seen=%d\n", sh, total, i, seen[i]); bad++; break; }
      if (sum != total || hi - lo > kExpandItemBlock) { printf("FAIL share sh=%d total=%d\n", sh, total); bad++; }
      // every work-group of an XCD's MBGMM set finds the same split
      for (int grid : {8, 64, 768}) {
        if ((grid % 8 == 0 ? 3 : 0) != sh) continue;
        for (int tv : {0, total / 2, 100 * total + 1}) {
          for (int x = 0; x < nx; ++x) {
            const QueueSplit a = expand_queue_split(total, tv, grid, x), b = expand_queue_split(total, tv, grid, grid - nx + x);
            if (a.Gm != b.Gm || a.m != b.m || a.x != x || b.x != x || (a.m > 0) != (a.Gm > 0) || a.Gm > grid / nx) {
              printf("FAIL split total=%d tv=%d grid=%d x=%d\n", total, tv, grid, x); bad++;
            }
          }
        }
      }
    }
  }
  printf(bad ? "FAILED\n" : "OK\n");
  return bad != 0;
}
"""


def test_expand_queue_blocks_cover_every_item_once(tmp_path):
    """The expand kernel's MBGMM item queues: the blocks dealt over the XCDs
    cover every item of the list exactly once, whole blocks stay on one XCD,
    the XCDs' shares differ by at most one block, and every work-group of an
    XCD computes the same split (the queue's arrival count relies on it).
    Compiled from the plan header with the host compiler."""
    import subprocess
    src = tmp_path / "queue_check.cpp"
    src.write_text(QUEUE_CHECK)
    exe = tmp_path / "queue_check"
    inc = os.path.join(ROOT, "heterogeneous_adapters_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", f"-I{inc}", str(src), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout


def test_noalloc_refuses_batches_beyond_its_array():
    """lora_apply_noalloc sizes the call before anything else: a batch whose
    workspace exceeds the library's fixed array is refused with WORKSPACE
    (the descriptors point at host memory: nothing is dereferenced)."""
    b = _Buf()
    L = lora.lib()
    r = ctypes.byref
    v = ctypes.c_void_p(b.p())
    ad = lora.lora_adapters_t(b.p(), b.p(64), 16)
    pool = lora.lora_pool_t(b.p(), 4, 4096, lora.LORA_DTYPE_BF16)
    one = (lora.lora_proj_t * 1)(lora.lora_proj_t(b.p(), 4096, b.p(), 4096, b.p(), 4096, 4096, 4096,
                                                  b.p(), b.p(), b.p(), b.p()))
    T = 38781  # a prefill batch: 8 slices x T x 128 x 4 bytes of partial sums
    assert L.lora_workspace_size(T, 16, 1, 4096) > lora.LORA_NOALLOC_SCRATCH_BYTES
    assert L.lora_apply_noalloc(v, None, T, one, 1, r(ad), r(pool), None) == -4
    assert L.lora_apply_noalloc(v, None, -1, one, 1, r(ad), r(pool), None) == -1
    assert L.lora_apply_noalloc(v, None, 8, None, 1, r(ad), r(pool), None) == -1
    assert L.lora_apply_noalloc(v, None, 8, one, 1, None, r(pool), None) == -1
    txt = open(HEADERS[0]).read()
    assert re.search(r"#define LORA_NOALLOC_SCRATCH_BYTES \(64u << 20\)", txt)
    assert lora.LORA_NOALLOC_SCRATCH_BYTES == 64 << 20


def test_launch_mode_values():
    L = lora.lib()
    for m in (lora.LORA_LAUNCH_AUTO, lora.LORA_LAUNCH_SINGLE, lora.LORA_LAUNCH_TWO):
        assert L.lora_set_launch_mode(m) == 0
    assert L.lora_set_launch_mode(3) == -1 and L.lora_set_launch_mode(-1) == -1
    assert L.lora_set_launch_mode(lora.LORA_LAUNCH_AUTO) == 0
    txt = open(HEADERS[0]).read()
    for name, v in (("LORA_LAUNCH_AUTO", 0), ("LORA_LAUNCH_SINGLE", 1), ("LORA_LAUNCH_TWO", 2)):
        assert re.search(rf"#define {name} {v}\b", txt), name
