"""Device-resident synthetic workloads too large for host generation (the full
32-layer x 7-projection decode step with 1000 resident adapters: a pool of
about 1.3 M pages of 16 x 4096 bf16, ~160 GiB of HBM).

Same recipe as the host generator -- bounded-Zipf ids and ranks from the same
seeds, X and Y_base ~ N(0, 1), A ~ N(0, 1/d_in), B ~ N(0, 1/r), NaN in every
page element that belongs to no rank or feature, pages scattered over the
pool by a seeded permutation -- but the values come from a seeded
``torch.Generator`` on the device.  Also holds ``host_subset``, which copies
the pages that a set of adapters uses back to the host, with re-numbered
page tables, for checks against the CPU oracle.  No arithmetic of the method
lives here.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Sequence

import numpy as np
import torch

from . import (CONFIGS, PAGE_ROWS, ProjTables, config_seed, draw_ids_and_ranks, n_blocks, n_groups,
               plan_tables)


@dataclass
class DeviceWorkload:
    cfg: int
    name: str
    dtype: str
    T: int
    N: int
    ids: np.ndarray
    ranks: np.ndarray
    alpha: np.ndarray
    page_width: int
    tables: List[ProjTables]
    num_pages: int
    pool: torch.Tensor              # (num_pages, 16*PW) on the device
    X: List[torch.Tensor]
    Y_base: List[torch.Tensor]
    shapes: List[tuple]

    @property
    def n_projs(self) -> int:
        return len(self.tables)


def _page_meta(tables: Sequence[ProjTables], ranks: np.ndarray, pw: int, num_pages: int):
    """Per physical page: value scale, valid ranks, valid features, kind (0=A, 1=B)."""
    scale = np.zeros(num_pages, np.float32)
    vr = np.zeros(num_pages, np.int16)
    vf = np.zeros(num_pages, np.int32)
    kind = np.zeros(num_pages, np.int8)
    G = (ranks.astype(np.int64) + PAGE_ROWS - 1) // PAGE_ROWS
    for t in tables:
        for is_b, indptr, pages, d in ((0, t.a_indptr, t.a_pages, t.d_in), (1, t.b_indptr, t.b_pages, t.d_out)):
            nc = n_blocks(d, pw)
            cnt = np.diff(indptr.astype(np.int64))
            owner = np.repeat(np.arange(len(ranks)), cnt)
            local = np.arange(indptr[-1]) - np.repeat(indptr[:-1].astype(np.int64), cnt)
            g, c = local // nc, local % nc
            pg = pages.astype(np.int64)
            r = ranks[owner].astype(np.int64)
            scale[pg] = (1.0 / np.sqrt(r)) if is_b else np.float32(1.0 / math.sqrt(d))
            vr[pg] = np.minimum(PAGE_ROWS, r - PAGE_ROWS * g)
            vf[pg] = np.minimum(pw, d - c * pw)
            kind[pg] = is_b
            assert np.all(G[owner] * nc == np.repeat(cnt, cnt))
    return scale, vr, vf, kind


def make_device_workload(k: int, device="cuda", overrides=None, chunk_pages: int = 4096) -> DeviceWorkload:
    c = dict(CONFIGS[k])
    if overrides:
        c.update(overrides)
    seed = c.get("seed", config_seed(k))
    ids, ranks, alpha, _ = draw_ids_and_ranks(k, c)
    T = len(ids)
    shapes = [(n, di, do) for _ in range(c["layers"]) for (n, di, do) in c["projs"]]
    pw = c["page_width"]
    assert c["dtype"] == "bf16"
    tables, num_pages = plan_tables(ranks, shapes, pw, c["scatter"], seed)
    scale, vr, vf, kind = _page_meta(tables, ranks, pw, num_pages)
    g = torch.Generator(device=device)
    g.manual_seed(seed + 100)
    pool = torch.empty((num_pages, PAGE_ROWS * pw), dtype=torch.bfloat16, device=device)
    scale_d = torch.from_numpy(scale).to(device)
    for s in range(0, num_pages, chunk_pages):
        e = min(num_pages, s + chunk_pages)
        tmp = torch.randn((e - s, PAGE_ROWS * pw), generator=g, device=device, dtype=torch.float32)
        tmp.mul_(scale_d[s:e, None])
        pool[s:e].copy_(tmp)
        del tmp
    # NaN in every element that belongs to no rank or no feature
    nan = float("nan")
    for kd in (0, 1):
        for r_ok in np.unique(vr):
            for f_ok in np.unique(vf):
                sel = np.nonzero((kind == kd) & (vr == r_ok) & (vf == f_ok))[0]
                if len(sel) == 0 or (r_ok == PAGE_ROWS and f_ok == pw):
                    continue
                for s in range(0, len(sel), chunk_pages):
                    idx = torch.from_numpy(sel[s:s + chunk_pages]).to(device)
                    sub = pool.index_select(0, idx)
                    if kd == 0:   # A page: [16 ranks][PW inputs]
                        v = sub.view(-1, PAGE_ROWS, pw)
                        v[:, int(r_ok):, :] = nan
                        v[:, :, int(f_ok):] = nan
                    else:         # B page: [2 halves][PW outputs][8 ranks]
                        half = PAGE_ROWS // 2
                        v = sub.view(-1, 2, pw, half)
                        v[:, 0, :, min(int(r_ok), half):] = nan
                        v[:, 1, :, max(int(r_ok) - half, 0):] = nan
                        v[:, :, int(f_ok):, :] = nan
                    pool.index_copy_(0, idx, sub)
    # share_x: groups of projection names that read one input inside a layer
    # (q/k/v, gate/up of a transformer block); their X is one tensor
    share = {n: gi for gi, grp in enumerate(c.get("share_x", ())) for n in grp}
    nproj = len(c["projs"])
    xs = {}
    X = []
    for i, (n, di, _) in enumerate(shapes):
        key = (i // nproj, ("g", share[n]) if n in share else ("p", n))
        if key not in xs:
            xs[key] = torch.randn((T, di), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
        X.append(xs[key])
    Yb = [torch.randn((T, do), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
          for (_, _, do) in shapes]
    return DeviceWorkload(cfg=k, name=c["name"], dtype="bf16", T=T, N=len(ranks), ids=ids, ranks=ranks,
                          alpha=alpha, page_width=pw, tables=tables, num_pages=num_pages, pool=pool, X=X,
                          Y_base=Yb, shapes=shapes)


def host_subset(pool: torch.Tensor, tables: Sequence[ProjTables], adapters: np.ndarray):
    """Copy the pages of ``adapters`` in ``tables`` to the host.  Returns the
    host pool (bf16 bits, uint16) and page tables re-numbered into it; tables
    of adapters outside the set are left empty."""
    adapters = np.unique(np.asarray(adapters, np.int64))
    N = len(tables[0].a_indptr) - 1
    chosen, new_tables = [], []
    base = 0
    for t in tables:
        parts = {}
        for name, indptr, pages in (("a", t.a_indptr, t.a_pages), ("b", t.b_indptr, t.b_pages)):
            cnt = np.zeros(N, np.int64)
            sel = []
            for a in adapters:
                sl = pages[indptr[a]:indptr[a + 1]]
                cnt[a] = len(sl)
                sel.append(sl)
            sel = np.concatenate(sel) if sel else np.zeros(0, np.int32)
            ip = np.zeros(N + 1, np.int64)
            ip[1:] = np.cumsum(cnt)
            parts[name] = (ip.astype(np.int32), (base + np.arange(len(sel))).astype(np.int32))
            chosen.append(sel)
            base += len(sel)
        new_tables.append(ProjTables(t.name, t.d_in, t.d_out, parts["a"][0], parts["a"][1],
                                     parts["b"][0], parts["b"][1]))
    ids = torch.from_numpy(np.concatenate(chosen).astype(np.int64)).to(pool.device)
    host = pool.index_select(0, ids).cpu().view(torch.int16).numpy().view(np.uint16)
    return host, new_tables


def tensor_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
