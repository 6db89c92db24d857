"""Two-tier adapter storage: every adapter's pages in pinned host memory, a
bounded set of them resident in a device page pool.

[MLSP] "Tiered Storage Hierarchy": hot adapters live in GPU memory, the rest
in host memory, and a miss moves an adapter in; [MLSP] "Unified Paging
Architecture" and [MLSA] "S-LoRA unified paging": the device copy lives in
fixed-size pages of one pool, addressed through page tables, so an adapter
need not be contiguous.  Page allocation and LRU eviction run in the native
cache of ``lora_pool.h`` (``lora.PageCache``); the copies run as
``lora_upload_pages`` on a side stream.  This module keeps the page tables
in step with the cache: plumbing only, no arithmetic of the method.

An adapter's host image is its pages in table order: for each projection,
its A slots then its B slots (the slot order of ``lora.h``).
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence

import numpy as np
import torch

from . import lora


class PoolState:
    """Host side of a managed pool: which adapters are resident (the native
    cache), the host copy of every projection's page tables, the adapters a
    batch in flight pins, and whether the next upload must wait for the work
    already enqueued on the compute stream.

    That wait is needed whenever pages that enqueued work may still read have
    become free since the last wait: an eviction, or the release of the
    adapters a failed batch had admitted (their pages may be an evicted
    adapter's).  The flag is sticky until an upload waits, so a batch that
    reuses such pages without evicting anything itself still orders its
    uploads after that work."""

    def __init__(self, indptrs: Sequence[tuple], capacity: int):
        self.indptrs = [(np.asarray(a, np.int64), np.asarray(b, np.int64)) for a, b in indptrs]
        N = len(self.indptrs[0][0]) - 1
        counts = np.zeros(N, np.int64)
        for a_ip, b_ip in self.indptrs:
            counts += np.diff(a_ip) + np.diff(b_ip)
        self.offsets = np.concatenate([[0], np.cumsum(counts)])
        self.N = N
        self.cache = lora.PageCache(capacity)
        # page tables; slots of non-resident adapters hold page 0 (never read)
        self.host_pages = [(np.zeros(a[-1], np.int32), np.zeros(b[-1], np.int32)) for a, b in self.indptrs]
        self.pinned = set()  # adapters pinned by admit() and not yet unpinned
        self.fence_pending = False  # freed pages may still be read by enqueued work
        self.hits = self.misses = self.evictions = 0

    def n_pages(self, a: int) -> int:
        return int(self.offsets[a + 1] - self.offsets[a])

    def _write_tables(self, a: int, pages: np.ndarray) -> None:
        k = 0
        for (a_ip, b_ip), (a_pg, b_pg) in zip(self.indptrs, self.host_pages):
            na, nb = a_ip[a + 1] - a_ip[a], b_ip[a + 1] - b_ip[a]
            a_pg[a_ip[a]:a_ip[a + 1]] = pages[k:k + na]
            b_pg[b_ip[a]:b_ip[a + 1]] = pages[k + na:k + na + nb]
            k += na + nb

    def admit(self, adapters: Iterable[int]):
        """Make ``adapters`` resident and pinned and rewrite the host tables.
        Returns (missed adapters, [(adapter, pages)] to upload, whether those
        uploads must first wait for the enqueued compute work).  A batch that
        does not fit raises lora.LoraError and leaves nothing of it pinned or
        admitted."""
        want = [int(a) for a in dict.fromkeys(int(x) for x in adapters)]
        for a in want:
            if not 0 <= a < self.N:
                raise ValueError(f"adapter {a} outside 0..{self.N - 1}")
        missed, plan, newly_pinned = [], [], []
        try:
            for a in want:
                hit, pages, ev = self.cache.admit(a, self.n_pages(a))
                if len(ev):
                    self.fence_pending = True
                    self.evictions += len(ev)
                if not hit:
                    plan.append((a, pages))
                # pin at once so that a later admission of this batch cannot evict it
                self.cache.set_pinned(a, True)
                if a not in self.pinned:
                    self.pinned.add(a)
                    newly_pinned.append(a)
                if hit:
                    self.hits += 1
                else:
                    self.misses += 1
                    missed.append(a)
                self._write_tables(a, pages)
        except lora.LoraError:
            # the batch does not fit: nothing of it stays pinned, and adapters
            # admitted by this call (pages assigned, nothing uploaded) leave;
            # their pages may have been an evicted adapter's
            for a in newly_pinned:
                self.pinned.discard(a)
                self.cache.set_pinned(a, False)
            for a, _ in plan:
                self.cache.release(a)
            raise
        fence = bool(plan) and self.fence_pending
        if fence:
            self.fence_pending = False
        return missed, plan, fence

    def unpin(self, adapters: Iterable[int]) -> None:
        for a in dict.fromkeys(int(x) for x in adapters):
            self.cache.set_pinned(a, False)
            self.pinned.discard(a)


class ManagedPool:
    """Device pool of ``capacity`` pages caching the adapters of a host tier.

    indptrs: per projection, (a_indptr, b_indptr) int32 arrays over the N
    adapters (slot counts per adapter, fixed by rank and shape).
    host_tier: pinned CPU tensor (total pages, 16*page_width) holding every
    adapter's image; adapter a's image is rows offsets[a]:offsets[a+1].
    """

    def __init__(self, indptrs: Sequence[tuple], host_tier: torch.Tensor, page_width: int, capacity: int,
                 device="cuda"):
        self.state = PoolState(indptrs, capacity)
        st = self.state
        self.indptrs, self.offsets, self.N, self.cache = st.indptrs, st.offsets, st.N, st.cache
        if host_tier.dim() != 2 or host_tier.shape[0] != self.offsets[-1] or host_tier.device.type != "cpu":
            raise ValueError("host tier must hold every adapter's pages on the host")
        self.host_tier, self.page_width = host_tier, page_width
        self.base = torch.empty((capacity, host_tier.shape[1]), dtype=host_tier.dtype, device=device)
        self.pool = lora.Pool(self.base, page_width)
        i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(device)
        self.tables = [(i32(a_ip), i32(a_pg), i32(b_ip), i32(b_pg))
                       for (a_ip, b_ip), (a_pg, b_pg) in zip(self.indptrs, st.host_pages)]
        self.upload_stream = torch.cuda.Stream(device=device)
        self.pages_uploaded = 0

    @property
    def pinned(self):
        return self.state.pinned

    @property
    def hits(self):
        return self.state.hits

    @property
    def misses(self):
        return self.state.misses

    @property
    def evictions(self):
        return self.state.evictions

    def n_pages(self, a: int) -> int:
        return self.state.n_pages(a)

    def ensure(self, adapters: Iterable[int], compute_stream: Optional[torch.cuda.Stream] = None) -> List[int]:
        """Make ``adapters`` resident and pinned, upload the misses, rewrite the
        page tables, and make ``compute_stream`` (default: current) wait for
        the uploads.  Returns the adapters that missed.  When pages freed since
        the last such wait are reused (PoolState), the uploads first wait for
        the work already on ``compute_stream``: it may still read them."""
        compute_stream = compute_stream or torch.cuda.current_stream()
        missed, plan, fence = self.state.admit(adapters)
        if plan:
            if fence:
                self.upload_stream.wait_stream(compute_stream)
            for a, pages in plan:
                lora.lora_upload_pages(self.pool, self.host_tier[self.offsets[a]:self.offsets[a + 1]], pages,
                                       stream=self.upload_stream)
                self.pages_uploaded += len(pages)
            compute_stream.wait_stream(self.upload_stream)
        # tables: small, copied on the compute stream after it has passed the
        # work that read the old ones
        with torch.cuda.stream(compute_stream):
            for (_, a_pg_d, _, b_pg_d), (a_pg, b_pg) in zip(self.tables, self.state.host_pages):
                a_pg_d.copy_(torch.from_numpy(a_pg))
                b_pg_d.copy_(torch.from_numpy(b_pg))
        return missed

    def unpin(self, adapters: Iterable[int]) -> None:
        """The batch that used ``adapters`` has been enqueued; they may be
        evicted by later admissions (which then order their uploads after it)."""
        self.state.unpin(adapters)

    def proj(self, p: int, X: torch.Tensor, Y_base: torch.Tensor, Y: torch.Tensor) -> lora.Proj:
        a_ip, a_pg, b_ip, b_pg = self.tables[p]
        return lora.Proj(X, Y_base, Y, a_ip, a_pg, b_ip, b_pg)


def host_tier_from_pool(pool_host: torch.Tensor, tables: Sequence, N: int, pin: bool = True) -> torch.Tensor:
    """Gather each adapter's pages (table order) from a host pool laid out by
    any page tables into one host tier tensor (pinned if ``pin``)."""
    order = []
    for a in range(N):
        for t in tables:
            order.append(np.asarray(t.a_pages[t.a_indptr[a]:t.a_indptr[a + 1]], np.int64))
            order.append(np.asarray(t.b_pages[t.b_indptr[a]:t.b_indptr[a + 1]], np.int64))
    idx = torch.from_numpy(np.concatenate(order) if order else np.zeros(0, np.int64))
    out = torch.empty((len(idx), pool_host.shape[1]), dtype=pool_host.dtype, pin_memory=pin)
    torch.index_select(pool_host, 0, idx, out=out)
    return out
