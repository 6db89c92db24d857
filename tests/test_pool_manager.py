"""Host tests of the pool manager (include/lora_pool.h): page allocation,
least-recently-used eviction with pinning, and the host-side checks of the
page upload.  No GPU needed.

Pins: the hit rates the [MLSA] page prints for its adapter-cache LRU
simulator (tests/golden/mlsa_lru_hit_rates.txt) reached through the native
cache, and a small independent model of the same policy (least recently
used unpinned adapters evicted until the new one fits, lowest free page ids
assigned) compared call by call on random traffic.
"""
import collections
import ctypes
import os
import random

import numpy as np
import pytest

import workloads as W
from heterogeneous_adapters_amd import lora

GOLD = os.path.join(os.path.dirname(__file__), "golden")
INVALID_ARG, PAGE_RANGE, UNSUPPORTED, POOL_FULL = -1, -3, -6, -8


def _gold_rows():
    rows = []
    with open(os.path.join(GOLD, "mlsa_lru_hit_rates.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


_SEQ = {}


def _requests(s):
    """The simulator's request stream: 200,000 draws over 500 adapters, seed 7."""
    if s not in _SEQ:
        zs = W.ZipfSampler(500, s, 7)
        _SEQ[s] = [zs.sample() for _ in range(200_000)]
    return _SEQ[s]


@pytest.mark.parametrize("row", _gold_rows())
def test_native_cache_reproduces_lru_hit_rates(row):
    """Every adapter takes 3 pages and the pool holds slots*3: the page-level
    cache then keeps exactly `slots` adapters and must hit at the printed rate."""
    s, slots, pct = float(row[0]), int(row[1]), int(row[2])
    cache = lora.PageCache(3 * slots)
    hits = 0
    for a in _requests(s):
        hit, pages, ev = cache.admit(a, 3)
        hits += hit
        assert len(ev) <= 1
    assert cache.num_resident == slots and cache.free_pages == 0
    assert round(100 * hits / 200_000) == pct, (s, slots, hits)


class Model:
    """The eviction policy written out plainly (sets and an ordered dict)."""

    def __init__(self, n):
        self.n, self.free, self.lru = n, set(range(n)), collections.OrderedDict()  # last = most recent

    def admit(self, key, n, max_ev):
        if key in self.lru:
            pages, pinned = self.lru[key]
            if len(pages) != n:
                return "INVALID"
            self.lru.move_to_end(key)
            return True, list(pages), []
        if n > self.n:
            return "FULL"
        victims, avail = [], len(self.free)
        for k, (pages, pinned) in self.lru.items():
            if avail >= n:
                break
            if not pinned:
                victims.append(k)
                avail += len(pages)
        if avail < n or len(victims) > max_ev:
            return "FULL"
        for k in victims:
            self.free |= set(self.lru.pop(k)[0])
        pages = sorted(self.free)[:n]
        self.free -= set(pages)
        self.lru[key] = (pages, False)
        return False, pages, victims

    def pin(self, key, p):
        if key not in self.lru:
            return "INVALID"
        self.lru[key] = (self.lru[key][0], p)

    def release(self, key):
        if key not in self.lru:
            return "INVALID"
        self.free |= set(self.lru.pop(key)[0])


def _check_disjoint(model, num_pages):
    used = [p for pages, _ in model.lru.values() for p in pages]
    assert len(used) == len(set(used))
    assert sorted(used + sorted(model.free)) == list(range(num_pages))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_cache_matches_policy_model(seed):
    """Adapters of different sizes (pages by rank), random pins and releases:
    the native cache agrees with the model on every return value."""
    rng = random.Random(seed)
    num_pages = 97
    sizes = {k: rng.choice([1, 2, 4, 8, 16, 3, 5]) for k in range(60)}
    cache, model = lora.PageCache(num_pages), Model(num_pages)
    for step in range(4000):
        op = rng.random()
        key = min(int(rng.paretovariate(1.0)) - 1, 59) if rng.random() < 0.7 else rng.randrange(60)
        if op < 0.75:
            max_ev = rng.choice([0, 1, 2, 100])
            want = model.admit(key, sizes[key], max_ev)
            try:
                got = cache.admit(key, sizes[key], max_ev)
            except lora.LoraError as e:
                assert want == "FULL" and e.status == POOL_FULL, (step, want)
                continue
            assert want not in ("FULL", "INVALID"), (step, want, got)
            assert got[0] == want[0] and list(got[1]) == want[1] and list(got[2]) == want[2], step
        elif op < 0.9:
            p = rng.random() < 0.5
            want = model.pin(key, p)
            try:
                cache.set_pinned(key, p)
                assert want is None
            except lora.LoraError as e:
                assert want == "INVALID" and e.status == INVALID_ARG
        else:
            want = model.release(key)
            try:
                cache.release(key)
                assert want is None
            except lora.LoraError as e:
                assert want == "INVALID" and e.status == INVALID_ARG
        assert cache.free_pages == len(model.free)
        assert cache.num_resident == len(model.lru)
    _check_disjoint(model, num_pages)


def test_failed_admission_changes_nothing():
    c = lora.PageCache(10)
    for k in range(5):
        c.admit(k, 2)
    c.set_pinned(0, True)
    c.set_pinned(1, True)
    # 7 pages need three victims (2, 3, 4) and 1 more page that only pinned adapters hold
    with pytest.raises(lora.LoraError):
        c.admit(9, 7)
    assert c.num_resident == 5 and c.free_pages == 0
    # allowed evictions below what is needed: refused, nothing evicted
    with pytest.raises(lora.LoraError):
        c.admit(9, 6, max_evicted=2)
    assert c.num_resident == 5
    hit, pages, ev = c.admit(9, 6, max_evicted=3)
    assert not hit and list(ev) == [2, 3, 4] and list(pages) == [4, 5, 6, 7, 8, 9]
    # a resident key with another page count is an argument error
    with pytest.raises(lora.LoraError):
        c.admit(9, 5)
    # larger than the pool
    with pytest.raises(lora.LoraError):
        c.admit(11, 11)


def test_free_ranges_merge_back_to_one_run():
    c = lora.PageCache(64)
    for k in range(16):
        c.admit(k, 4)
    for k in (3, 1, 2, 15, 0, 7, 5, 6, 4, 9, 8, 11, 10, 14, 12, 13):
        c.release(k)
    hit, pages, ev = c.admit(99, 64)
    assert not hit and list(pages) == list(range(64)) and len(ev) == 0


def test_lookup_leaves_recency_alone():
    c = lora.PageCache(6)
    c.admit(0, 2)
    c.admit(1, 2)
    c.admit(2, 2)
    assert list(c.lookup(0)) == [0, 1] and len(c.lookup(5)) == 0
    # 0 is still the least recently used: the next admission evicts it
    _, _, ev = c.admit(3, 2)
    assert list(ev) == [0]
    L = lora.lib()
    n = ctypes.c_int32()
    buf = (ctypes.c_int32 * 1)()
    assert L.lora_cache_lookup(c.h, 1, buf, 1, ctypes.byref(n)) == INVALID_ARG
    assert L.lora_cache_lookup(c.h, 1, None, 1, ctypes.byref(n)) == INVALID_ARG
    assert L.lora_cache_lookup(c.h, 1, None, 0, None) == INVALID_ARG
    assert L.lora_cache_lookup(c.h, 1, None, 0, ctypes.byref(n)) == 0 and n.value == 2


def test_lowest_pages_first_and_hits_keep_pages():
    c = lora.PageCache(16)
    _, p0, _ = c.admit(0, 5)
    _, p1, _ = c.admit(1, 3)
    c.release(0)
    _, p2, _ = c.admit(2, 2)
    assert list(p2) == [0, 1]
    hit, p1b, _ = c.admit(1, 3)
    assert hit and list(p1b) == list(p1) == [5, 6, 7]


def test_cache_rejects_bad_arguments():
    L = lora.lib()
    h = ctypes.c_void_p()
    assert L.lora_cache_create(0, ctypes.byref(h)) == INVALID_ARG
    assert L.lora_cache_create(4, None) == INVALID_ARG
    c = lora.PageCache(4)
    pages = (ctypes.c_int32 * 4)()
    hit, nev = ctypes.c_int32(), ctypes.c_int32()
    assert L.lora_cache_admit(c.h, 1, 0, pages, ctypes.byref(hit), None, 0, ctypes.byref(nev)) == \
        INVALID_ARG
    assert L.lora_cache_admit(c.h, 1, 2, None, ctypes.byref(hit), None, 0, ctypes.byref(nev)) == \
        INVALID_ARG
    assert L.lora_cache_admit(c.h, 1, 2, pages, ctypes.byref(hit), None, 1, ctypes.byref(nev)) == \
        INVALID_ARG
    assert L.lora_cache_admit(None, 1, 2, pages, ctypes.byref(hit), None, 0, ctypes.byref(nev)) == \
        INVALID_ARG
    assert L.lora_cache_set_pinned(c.h, 7, 1) == INVALID_ARG
    assert L.lora_cache_release(c.h, 7) == INVALID_ARG
    assert L.lora_cache_free_pages(None) == 0 and L.lora_cache_num_resident(None) == 0
    L.lora_cache_destroy(None)


def test_upload_rejects_bad_arguments_before_any_copy():
    """All of these return before a HIP call, so they run without a GPU."""
    L = lora.lib()
    src = (ctypes.c_uint16 * (16 * 8 * 2))()
    pool = lora.lora_pool_t(0x1000, 4, 8, lora.LORA_DTYPE_BF16)
    ids = (ctypes.c_int32 * 2)(1, 4)
    assert L.lora_upload_pages(ctypes.byref(pool), src, ids, 2, None) == PAGE_RANGE
    ids = (ctypes.c_int32 * 2)(-1, 0)
    assert L.lora_upload_pages(ctypes.byref(pool), src, ids, 2, None) == PAGE_RANGE
    ids = (ctypes.c_int32 * 2)(0, 1)
    bad = lora.lora_pool_t(0x1000, 4, 8, 7)
    assert L.lora_upload_pages(ctypes.byref(bad), src, ids, 2, None) == UNSUPPORTED
    assert L.lora_upload_pages(None, src, ids, 2, None) == INVALID_ARG
    assert L.lora_upload_pages(ctypes.byref(pool), None, ids, 2, None) == INVALID_ARG
    assert L.lora_upload_pages(ctypes.byref(pool), src, None, 2, None) == INVALID_ARG
    assert L.lora_upload_pages(ctypes.byref(pool), src, ids, -1, None) == INVALID_ARG
    assert L.lora_upload_pages(ctypes.byref(pool), None, None, 0, None) == 0


def _state(n_adapters=8, pages_each=3, capacity=6):
    from heterogeneous_adapters_amd.pool import PoolState
    ip = np.arange(n_adapters + 1, dtype=np.int64)          # one A slot per adapter
    ipb = np.arange(n_adapters + 1, dtype=np.int64) * (pages_each - 1)  # the rest B slots
    return PoolState([(ip, ipb)], capacity)


def test_upload_order_after_a_failed_batch():
    """A batch that does not fit evicts resident adapters before it fails; its
    rollback frees the pages it had taken, which the evicted adapters' work,
    already enqueued, may still read.  The next batch that takes those pages
    without evicting anything itself must still order its uploads after that
    work (the decision ManagedPool.ensure acts on)."""
    st = _state()
    for a in (0, 1):
        missed, plan, fence = st.admit([a])
        assert missed == [a] and len(plan) == 1 and not fence
        st.unpin([a])
    assert st.cache.free_pages == 0
    with pytest.raises(lora.LoraError):
        st.admit([2, 3, 4])        # evicts 0 and 1, then 4 does not fit
    assert st.pinned == set() and st.cache.num_resident == 0 and st.cache.free_pages == 6
    missed, plan, fence = st.admit([5])
    assert missed == [5] and fence, "pages of evicted adapters reused without waiting for their readers"
    st.unpin([5])
    # the wait covered every page freed so far: the next miss into free pages needs none
    missed, plan, fence = st.admit([6])
    assert missed == [6] and not fence
    # a batch of hits uploads nothing and keeps a pending wait for the next upload
    st.unpin([6])
    with pytest.raises(lora.LoraError):
        st.admit([6, 1, 2])        # 6 hits, 1 evicts 5, then 2 does not fit
    assert st.fence_pending
    missed, plan, fence = st.admit([6])
    assert missed == [] and plan == [] and not fence and st.fence_pending
    st.unpin([6])
    missed, plan, fence = st.admit([0])
    assert missed == [0] and fence and not st.fence_pending


def test_upload_order_evictions_in_a_successful_batch():
    st = _state()
    st.admit([0]); st.unpin([0])
    st.admit([1]); st.unpin([1])
    missed, plan, fence = st.admit([2])   # evicts 0
    assert missed == [2] and fence
