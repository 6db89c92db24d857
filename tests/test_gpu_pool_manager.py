"""The pool manager on the GPU: adapters uploaded on demand into a pool
smaller than the adapter set, through the native cache's page assignment and
evictions, give the same Y as the generator's full pool, bit for bit.

Also checks that each resident adapter's pages in the device pool equal its
host image byte for byte after uploads that evict and re-admit.
"""
import numpy as np
import pytest
import torch

import workloads as W
from heterogeneous_adapters_amd import batch, lora
from heterogeneous_adapters_amd.pool import ManagedPool, host_tier_from_pool

pytestmark = pytest.mark.gpu


def _host_pool_tensor(w):
    if w.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(w.pool).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(w.pool, np.float32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_managed_pool_batches_match_full_pool(dtype):
    ranks = [8, 16, 64, 24, 32, 8, 1, 40, 128, 16]
    w = W.make_workload(2, dict(T=64, N=len(ranks), ranks_override=ranks, page_width=512, dtype=dtype,
                                projs=(("a", 1024, 768), ("b", 768, 1096))))
    tier = host_tier_from_pool(_host_pool_tensor(w), w.tables, w.N)
    mp = ManagedPool([(t.a_indptr, t.b_indptr) for t in w.tables], tier, w.page_width, capacity=60)
    sizes = [mp.n_pages(a) for a in range(w.N)]
    full = batch.to_device(w)
    rng = np.random.default_rng(5)
    stream = torch.cuda.current_stream()
    for step in range(8):
        # a batch over a few adapters whose pages fit the pool together
        order = rng.permutation(w.N)
        chosen, used = [], 0
        for a in order:
            if used + sizes[a] <= 60 and len(chosen) < 4:
                chosen.append(int(a))
                used += sizes[a]
        ids = rng.choice(np.asarray(chosen + [-1], np.int32), size=w.T).astype(np.int32)
        print(f"step {step}: adapters {chosen} pages {used}", flush=True)
        mp.ensure(chosen, stream)
        ids_d = torch.from_numpy(ids).cuda()
        ys = {}
        for which in ("managed", "full"):
            Y = [torch.empty_like(y) for y in full.Y_base]
            if which == "managed":
                projs = [mp.proj(p, full.X[p], full.Y_base[p], Y[p]) for p in range(w.n_projs)]
                pool = mp.pool
            else:
                projs = [lora.Proj(full.X[p], full.Y_base[p], Y[p], *full.tables[p]) for p in range(w.n_projs)]
                pool = full.pool
            segs = lora.Segments(w.T, w.N)
            ws = lora.workspace(w.T, w.N, w.n_projs, max(t.d_in for t in w.tables))
            lora.lora_apply(ids_d, segs, w.T, projs, full.adapters, pool, ws)
            torch.cuda.synchronize()
            ys[which] = [batch.device_to_host(y) for y in Y]
            assert int(segs.counts().cpu()[lora.COUNT_FLAGS]) == 0
        for p in range(w.n_projs):
            assert np.array_equal(ys["managed"][p], ys["full"][p]), (step, p)
        # resident pages hold their host image
        for a in chosen:
            pages = mp.cache.lookup(a)
            assert len(pages) == sizes[a]
            got = mp.base[torch.from_numpy(pages.astype(np.int64)).cuda()].cpu()
            want = tier[mp.offsets[a]:mp.offsets[a + 1]]
            bits = torch.int16 if dtype == "bf16" else torch.int32  # NaN padding compares by bits
            assert torch.equal(got.view(bits), want.view(bits)), (step, a)
        mp.unpin(chosen)
    # the pool is too small for the adapters: the run went through evictions
    assert mp.evictions > 0 and mp.misses > 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_managed_pool_async_serving_loop(dtype):
    """A serving loop with no synchronisation between batches: each batch's
    adapters are made resident (uploads on the pool's side stream, evicting
    adapters that earlier batches still being computed read), its lora_apply
    is enqueued on the compute stream, and its adapters are unpinned at once.
    Every batch's Y, checked after one final synchronisation, equals the same
    batch run on the generator's full pool, bit for bit."""
    ranks = [8, 16, 64, 24, 32, 8, 1, 40, 128, 16, 64, 8]
    w = W.make_workload(2, dict(T=96, N=len(ranks), ranks_override=ranks, page_width=512, dtype=dtype,
                                projs=(("a", 1024, 768), ("b", 768, 1096))))
    tier = host_tier_from_pool(_host_pool_tensor(w), w.tables, w.N)
    cap = 64
    mp = ManagedPool([(t.a_indptr, t.b_indptr) for t in w.tables], tier, w.page_width, capacity=cap)
    sizes = [mp.n_pages(a) for a in range(w.N)]
    full = batch.to_device(w)
    rng = np.random.default_rng(23)
    stream = torch.cuda.current_stream()
    kept = []  # per batch: its ids, both Y sets and both segment buffers (alive until the final check)
    for step in range(20):
        order = rng.permutation(w.N)
        chosen, used = [], 0
        for a in order:
            if used + sizes[a] <= cap and len(chosen) < 3:
                chosen.append(int(a))
                used += sizes[a]
        ids = torch.from_numpy(rng.choice(np.asarray(chosen + [-1], np.int32), size=w.T).astype(np.int32)).cuda()
        mp.ensure(chosen, stream)
        out = {}
        for which in ("managed", "full"):
            Y = [torch.empty_like(y) for y in full.Y_base]
            if which == "managed":
                projs = [mp.proj(p, full.X[p], full.Y_base[p], Y[p]) for p in range(w.n_projs)]
                pool = mp.pool
            else:
                projs = [lora.Proj(full.X[p], full.Y_base[p], Y[p], *full.tables[p]) for p in range(w.n_projs)]
                pool = full.pool
            segs = lora.Segments(w.T, w.N)
            ws = lora.workspace(w.T, w.N, w.n_projs, max(t.d_in for t in w.tables))
            lora.lora_apply(ids, segs, w.T, projs, full.adapters, pool, ws)
            out[which] = (Y, segs, ws)
        mp.unpin(chosen)
        kept.append((step, chosen, ids, out))
    torch.cuda.synchronize()
    assert mp.evictions > 0 and mp.misses > 0
    for step, chosen, _, out in kept:
        for which in ("managed", "full"):
            assert int(out[which][1].counts().cpu()[lora.COUNT_FLAGS]) == 0, (step, which)
        for p in range(w.n_projs):
            got = batch.device_to_host(out["managed"][0][p])
            want = batch.device_to_host(out["full"][0][p])
            assert np.array_equal(got, want), (step, chosen, p)


def test_upload_coalesces_runs_and_scatters():
    """lora_upload_pages to scattered and consecutive page ids: every page
    lands where its id says, the other pages are untouched."""
    pw = 64
    pool = torch.full((40, 16 * pw), -1.0, device="cuda")
    P = lora.Pool(pool, pw)
    ids = np.array([3, 4, 5, 17, 9, 10, 39, 0], np.int32)
    src = torch.arange(len(ids) * 16 * pw, dtype=torch.float32).view(len(ids), 16 * pw).pin_memory()
    lora.lora_upload_pages(P, src, ids)
    torch.cuda.synchronize()
    host = pool.cpu()
    for i, p in enumerate(ids):
        assert torch.equal(host[p], src[i])
    untouched = sorted(set(range(40)) - set(ids.tolist()))
    assert bool((host[untouched] == -1.0).all())


def test_managed_pool_rolls_back_a_batch_that_does_not_fit():
    """A batch whose adapters cannot all be resident raises; nothing of it
    stays pinned, adapters it admitted are released, earlier pins hold."""
    ranks = [8, 16, 64, 24, 32, 8, 1, 40, 128, 16]
    w = W.make_workload(2, dict(T=32, N=len(ranks), ranks_override=ranks, page_width=512, dtype="f32",
                                projs=(("a", 1024, 768), ("b", 768, 1096))))
    tier = host_tier_from_pool(_host_pool_tensor(w), w.tables, w.N)
    mp = ManagedPool([(t.a_indptr, t.b_indptr) for t in w.tables], tier, w.page_width, capacity=60)
    sizes = [mp.n_pages(a) for a in range(w.N)]
    assert (sizes[0], sizes[2], sizes[7]) == (9, 36, 27)
    mp.ensure([0])
    with pytest.raises(lora.LoraError):
        mp.ensure([2, 7])  # 9 pinned + 36 + 27 > 60
    assert mp.pinned == {0}
    assert len(mp.cache.lookup(0)) == 9 and len(mp.cache.lookup(2)) == 0 and len(mp.cache.lookup(7)) == 0
    assert mp.cache.free_pages == 51
    mp.unpin([0])
    mp.ensure([2, 3])  # 36 + 18 fit once adapter 0 may go
    torch.cuda.synchronize()
    assert mp.pinned == {2, 3}
    for a in (2, 3):
        got = mp.base[torch.from_numpy(mp.cache.lookup(a).astype(np.int64)).cuda()].cpu()
        assert torch.equal(got.view(torch.int32), tier[mp.offsets[a]:mp.offsets[a + 1]].view(torch.int32))
