"""Seeded synthetic workloads for the multi-LoRA adapter branch.

This module only *draws inputs*: adapter ids, ranks, alphas, prompt lengths,
activation and weight values, and the physical placement of adapter pages in
the pool.  It holds none of the method's arithmetic (no grouping, no shrink,
no expand, no page-table reads) and is shared by the CPU oracle's tests and
by the HIP path's tests and benchmark alike.

Sources (the three web pages this project follows):
  [MLSP] "Multi-LoRA Serving in Production: Architecture, Dynamic Adapter
         Swapping, and GPU Memory Management" (llms.blog)
  [MLSA] "Multi-LoRA Serving Architecture: Serving Hundreds of Fine-Tuned
         Adapters on One GPU with vLLM and S-LoRA (2026)"
  [LAST] "LoRA Adapters at Serve Time with vLLM Multi-LoRA"

Adapter popularity follows the bounded Zipf law of [MLSA] section "An
adapter-cache LRU simulator": weight 1/i^s for i = 1..n, sampled by bisecting
the cumulative weights with a uniform draw scaled by the total, from
``random.Random(seed)``.  Adapter id = i - 1, so id 0 is the most popular.

Pool page format (the same format the C header documents):
  * a page is 16 x PW elements of the pool dtype;
  * A of adapter a (d_in x r in the [MLSP] "Mathematical Anatomy" orientation)
    is stored as its r x d_in transpose (the [MLSA] "Context and Background"
    orientation), cut into 16-rank groups g and PW-wide column blocks c; slot
    g*ceil(d_in/PW) + c of the adapter's A table holds the page, element
    (rank k, input i) at in-page offset (k-16g)*PW + (i-c*PW);
  * B of adapter a (r x d_out) is stored as its d_out x r transpose (again the
    [MLSA] orientation), cut into PW-row blocks c and 16-rank groups g; slot
    g*ceil(d_out/PW) + c holds the page as two halves of 8 ranks, element
    (output j, rank k) at in-page offset h*8*PW + (j-c*PW)*8 + (k-16g-8h),
    h = (k-16g)//8;
  * elements of a page that belong to no rank (< r) or feature (< d) are
    filled with NaN so that any read of padding shows in the results.
"""
from __future__ import annotations

import bisect
import math
import random
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

PAGE_ROWS = 16
BF16_NAN = np.uint16(0x7FC0)

LLAMA7B_PROJS: Tuple[Tuple[str, int, int], ...] = (
    ("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096),
    ("o_proj", 4096, 4096), ("gate_proj", 4096, 11008), ("up_proj", 4096, 11008),
    ("down_proj", 11008, 4096))

# The benchmark workloads.  Seeds: workload k uses seed 7 + k (7 is the seed
# of the [MLSA] LRU simulator run).
CONFIGS: Dict[int, dict] = {
    0: dict(name="tiny-decode-sgmv", phase="decode", T=16, N=4, rank_choices=(8,),
            ids="uniform", projs=(("proj", 256, 256),), layers=1, dtype="f32",
            page_width=256, scatter=False),
    1: dict(name="uniform-rank-decode-q_proj", phase="decode", T=256, N=32,
            rank_choices=(16,), ids="zipf", zipf_s=1.1,
            projs=(("q_proj", 4096, 4096),), layers=1, dtype="bf16",
            page_width=4096, scatter=False),
    2: dict(name="hetero-rank-decode-mlp", phase="decode", T=512, N=128,
            rank_choices=(8, 16, 32, 64), ids="zipf", zipf_s=1.1,
            projs=(("up_proj", 4096, 11008), ("down_proj", 11008, 4096)), layers=1,
            dtype="bf16", page_width=4096, scatter=True),
    3: dict(name="prefill-mbgmm", phase="prefill", nseq=32, len_lo=128, len_hi=2048,
            N=16, rank_choices=(8, 16, 32, 64), ids="per-sequence",
            projs=(("proj", 4096, 4096),), layers=1, dtype="bf16",
            page_width=4096, scatter=True),
    # q/k/v read one input (the attention block's normed hidden state), and
    # so do gate/up (the MLP's): share_x makes them one activation tensor
    4: dict(name="llama2-7b-decode-step", phase="decode", T=1024, N=1000,
            rank_choices=(8, 16, 32, 64), ids="zipf", zipf_s=1.2,
            projs=LLAMA7B_PROJS, layers=32, dtype="bf16", page_width=4096,
            scatter=True, share_x=(("q_proj", "k_proj", "v_proj"), ("gate_proj", "up_proj"))),
    # A continuous-batching step (not one of the five): chunked-prefill
    # segments of new requests next to single decode tokens of running ones
    # in one batch ([MLSP] "Multi-Size Batched Gather Kernels": MBGMV and
    # MBGMM segments side by side).  Chunk lengths uniform on
    # [chunk_lo, chunk_hi], each chunk's adapter uniform over N; decode ids
    # bounded-Zipf; chunks first, then decode tokens.
    5: dict(name="mixed-prefill-decode", phase="mixed", nchunks=4, chunk_lo=256, chunk_hi=512,
            ndecode=1024, N=1000, rank_choices=(8, 16, 32, 64), ids="mixed", zipf_s=1.2,
            projs=(("q_proj", 4096, 4096),), layers=1, dtype="bf16", page_width=4096,
            scatter=True),
}


def config_seed(k: int) -> int:
    return 7 + k


# ----------------------------------------------------------------- ids / ranks
def zipf_cumulative(n: int, s: float) -> List[float]:
    """Cumulative bounded-Zipf weights, built the way the [MLSA] LRU simulator
    builds them: normalised weights 1/i^s, then a running sum."""
    w = [1.0 / (i ** s) for i in range(1, n + 1)]
    tot = sum(w)
    cum, acc = [], 0.0
    for x in w:
        acc += x / tot
        cum.append(acc)
    return cum


class ZipfSampler:
    """Bounded Zipf over n adapters driven by ``random.Random(seed)``; one
    ``rng.random()`` draw per sample, mapped by bisection on the cumulative
    weights scaled by their total (the [MLSA] simulator's method)."""

    def __init__(self, n: int, s: float, seed: int):
        self.cum = zipf_cumulative(n, s)
        self.rng = random.Random(seed)

    def sample(self) -> int:
        return bisect.bisect_left(self.cum, self.rng.random() * self.cum[-1])


def zipf_ids(T: int, n: int, s: float, seed: int) -> np.ndarray:
    zs = ZipfSampler(n, s, seed)
    return np.array([zs.sample() for _ in range(T)], dtype=np.int32)


def uniform_ids(T: int, n: int, seed: int) -> np.ndarray:
    rng = random.Random(seed)
    return np.array([rng.randrange(n) for _ in range(T)], dtype=np.int32)


def draw_ranks(N: int, choices: Sequence[int], rng: np.random.Generator) -> np.ndarray:
    """One rank per adapter, i.i.d. uniform over ``choices``, shared by every
    layer and projection of that adapter."""
    if len(choices) == 1:
        return np.full(N, choices[0], dtype=np.int32)
    return rng.choice(np.asarray(choices, dtype=np.int32), size=N).astype(np.int32)


# ------------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit patterns, via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------- pool packing
def n_groups(r: int) -> int:
    return (int(r) + PAGE_ROWS - 1) // PAGE_ROWS


def n_blocks(d: int, pw: int) -> int:
    return (int(d) + pw - 1) // pw


def pack_a_pages(A: np.ndarray, pw: int, fill) -> np.ndarray:
    """A: (d_in, r) -> pages (G*nci, 16*pw) in table-slot order g*nci + c."""
    d_in, r = A.shape
    G, nci = n_groups(r), n_blocks(d_in, pw)
    pad = np.full((G * PAGE_ROWS, nci * pw), fill, dtype=A.dtype)
    pad[:r, :d_in] = A.T
    return pad.reshape(G, PAGE_ROWS, nci, pw).transpose(0, 2, 1, 3).reshape(G * nci, PAGE_ROWS * pw)


def pack_b_pages(B: np.ndarray, pw: int, fill) -> np.ndarray:
    """B: (r, d_out) -> pages (G*nco, 16*pw) in table-slot order g*nco + c."""
    r, d_out = B.shape
    G, nco = n_groups(r), n_blocks(d_out, pw)
    pad = np.full((nco * pw, G * PAGE_ROWS), fill, dtype=B.dtype)
    pad[:d_out, :r] = B.T
    # [c, j', g, h, k'] -> page (g, c) = [h][j'][k']
    half = PAGE_ROWS // 2
    return pad.reshape(nco, pw, G, 2, half).transpose(2, 0, 3, 1, 4).reshape(G * nco, pw * PAGE_ROWS)


@dataclass
class ProjTables:
    """Page tables of one projection (CSR over adapters)."""
    name: str
    d_in: int
    d_out: int
    a_indptr: np.ndarray
    a_pages: np.ndarray
    b_indptr: np.ndarray
    b_pages: np.ndarray


def plan_tables(ranks: np.ndarray, shapes: Sequence[Tuple[str, int, int]], pw: int,
                scatter: bool, seed: int) -> Tuple[List[ProjTables], int]:
    """Allocate one page per (projection, adapter, matrix, slot) and return the
    page tables.  Logical allocation order is projection, adapter, A then B;
    ``scatter`` maps logical pages to a seeded random permutation of physical
    pages, otherwise they are consecutive (contiguous per-adapter storage)."""
    N = len(ranks)
    G = (ranks.astype(np.int64) + PAGE_ROWS - 1) // PAGE_ROWS
    tables, nxt = [], 0
    for name, d_in, d_out in shapes:
        nci, nco = n_blocks(d_in, pw), n_blocks(d_out, pw)
        a_cnt, b_cnt = G * nci, G * nco
        a_indptr = np.zeros(N + 1, np.int64)
        b_indptr = np.zeros(N + 1, np.int64)
        a_indptr[1:] = np.cumsum(a_cnt)
        b_indptr[1:] = np.cumsum(b_cnt)
        # logical ids: adapter a's A slots, then its B slots, adapters in order
        per_ad = a_cnt + b_cnt
        start = nxt + np.concatenate([[0], np.cumsum(per_ad)[:-1]])
        a_pages = np.repeat(start, a_cnt) + (np.arange(a_indptr[-1]) - np.repeat(a_indptr[:-1], a_cnt))
        b_pages = np.repeat(start + a_cnt, b_cnt) + (np.arange(b_indptr[-1]) - np.repeat(b_indptr[:-1], b_cnt))
        nxt += int(per_ad.sum())
        tables.append(ProjTables(name, d_in, d_out, a_indptr.astype(np.int32), a_pages,
                                 b_indptr.astype(np.int32), b_pages))
    num_pages = nxt
    perm = (np.random.default_rng(seed + 200).permutation(num_pages) if scatter
            else np.arange(num_pages))
    for t in tables:
        t.a_pages = perm[t.a_pages].astype(np.int32)
        t.b_pages = perm[t.b_pages].astype(np.int32)
    return tables, num_pages


# ------------------------------------------------------------------ workloads
@dataclass
class Workload:
    """One batch of synthetic input.  Activations are per projection; every
    floating array is stored as fp32 values (``dtype == 'f32'``) or bf16 bit
    patterns in uint16 (``dtype == 'bf16'``)."""
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
    pool: Optional[np.ndarray] = None          # (num_pages, 16*PW)
    X: List[np.ndarray] = field(default_factory=list)       # (T, d_in) each
    Y_base: List[np.ndarray] = field(default_factory=list)  # (T, d_out) each
    A: Optional[List[List[np.ndarray]]] = None  # [proj][adapter] (d_in, r) values as stored
    B: Optional[List[List[np.ndarray]]] = None  # [proj][adapter] (r, d_out)
    seq_lens: Optional[np.ndarray] = None

    @property
    def n_projs(self) -> int:
        return len(self.tables)


def _to_store(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, np.float32)


def draw_ids_and_ranks(k: int, cfg: Optional[dict] = None):
    c = dict(CONFIGS[k]) if cfg is None else cfg
    seed = c.get("seed", config_seed(k))
    nrng = np.random.default_rng(seed)
    ranks = draw_ranks(c["N"], c["rank_choices"], nrng)
    seq_lens = None
    if c["ids"] == "per-sequence":
        seq_lens = nrng.integers(c["len_lo"], c["len_hi"] + 1, size=c["nseq"]).astype(np.int64)
        prng = random.Random(seed)
        seq_ad = [prng.randrange(c["N"]) for _ in range(c["nseq"])]
        ids = np.repeat(np.asarray(seq_ad, np.int32), seq_lens)
    elif c["ids"] == "mixed":
        lens = nrng.integers(c["chunk_lo"], c["chunk_hi"] + 1, size=c["nchunks"]).astype(np.int64)
        prng = random.Random(seed)
        chunk_ad = [prng.randrange(c["N"]) for _ in range(c["nchunks"])]
        ids = np.concatenate([np.repeat(np.asarray(chunk_ad, np.int32), lens),
                              zipf_ids(c["ndecode"], c["N"], c["zipf_s"], seed + 1)])
        seq_lens = lens
    elif c["ids"] == "zipf":
        ids = zipf_ids(c["T"], c["N"], c["zipf_s"], seed)
    else:
        ids = uniform_ids(c["T"], c["N"], seed)
    alpha = (2.0 * ranks).astype(np.float32)
    return ids.astype(np.int32), ranks, alpha, seq_lens


def make_workload(k: int, overrides: Optional[dict] = None, keep_dense: bool = True) -> Workload:
    """Host-side workload (configs 0-3, or any override small enough for host
    memory).  Values: X, Y_base ~ N(0, 1); A ~ N(0, 1/d_in); B ~ N(0, 1/r)
    (second argument = variance), drawn in fp32 from
    ``numpy.random.default_rng(seed + 100)`` and cast to bf16 by RNE."""
    c = dict(CONFIGS[k])
    if overrides:
        c.update(overrides)
    seed = c.get("seed", config_seed(k))
    ids, ranks, alpha, seq_lens = draw_ids_and_ranks(k, c)
    if "ids_override" in c:
        ids = np.asarray(c["ids_override"], np.int32)
    if "ranks_override" in c:
        ranks = np.asarray(c["ranks_override"], np.int32)
        alpha = (2.0 * ranks).astype(np.float32)
    if "alpha_override" in c:
        alpha = np.asarray(c["alpha_override"], np.float32)
    T = len(ids)
    shapes = [(n, di, do) for _ in range(c["layers"]) for (n, di, do) in c["projs"]]
    pw, dtype = c["page_width"], c["dtype"]
    tables, num_pages = plan_tables(ranks, shapes, pw, c["scatter"], seed)
    vrng = np.random.default_rng(seed + 100)
    X, Yb = [], []
    for (_, d_in, d_out) in shapes:
        X.append(_to_store(vrng.standard_normal((T, d_in), dtype=np.float32), dtype))
        Yb.append(_to_store(vrng.standard_normal((T, d_out), dtype=np.float32), dtype))
    store_t = np.uint16 if dtype == "bf16" else np.float32
    fill = BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    pool = np.full((num_pages, PAGE_ROWS * pw), fill, dtype=store_t)
    As, Bs = [], []
    for p, (_, d_in, d_out) in enumerate(shapes):
        tb = tables[p]
        Ap, Bp = [], []
        for a in range(len(ranks)):
            r = int(ranks[a])
            Aa = _to_store(vrng.standard_normal((d_in, r), dtype=np.float32) / np.float32(math.sqrt(d_in)), dtype)
            Ba = _to_store(vrng.standard_normal((r, d_out), dtype=np.float32) / np.float32(math.sqrt(r)), dtype)
            pool[tb.a_pages[tb.a_indptr[a]:tb.a_indptr[a + 1]]] = pack_a_pages(Aa, pw, fill)
            pool[tb.b_pages[tb.b_indptr[a]:tb.b_indptr[a + 1]]] = pack_b_pages(Ba, pw, fill)
            if keep_dense:
                Ap.append(Aa)
                Bp.append(Ba)
        As.append(Ap)
        Bs.append(Bp)
    return Workload(cfg=k, name=c["name"], dtype=dtype, T=T, N=len(ranks), ids=ids, ranks=ranks,
                    alpha=alpha, page_width=pw, tables=tables, num_pages=num_pages, pool=pool,
                    X=X, Y_base=Yb, A=As if keep_dense else None, B=Bs if keep_dense else None,
                    seq_lens=seq_lens)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values (fp32 or bf16 bits) as float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, np.float64)


def pad_to_rank(w: Workload, r_max: int, seed: int = 0) -> Workload:
    """The same adapters stored the way a fixed-rank slot layout stores them:
    every adapter at rank ``r_max``, A and B zero-filled beyond the adapter's
    own rank, alpha scaled by r_max / r so that alpha / rank is unchanged
    ([MLSA] "What vLLM actually gives you" and "Practical Recommendations":
    slots sized by --max-lora-rank).  Needs the dense A and B (keep_dense)."""
    if w.A is None or w.B is None:
        raise ValueError("pad_to_rank needs a workload built with keep_dense=True")
    if int(w.ranks.max()) > r_max:
        raise ValueError("an adapter's rank exceeds r_max")
    N = w.N
    ranks = np.full(N, r_max, np.int32)
    alpha = (w.alpha.astype(np.float64) * r_max / w.ranks.astype(np.float64)).astype(np.float32)
    shapes = [(t.name, t.d_in, t.d_out) for t in w.tables]
    pw = w.page_width
    scatter = not all(np.array_equal(t.a_pages, np.sort(t.a_pages)) for t in w.tables)
    tables, num_pages = plan_tables(ranks, shapes, pw, scatter, seed)
    store_t = w.pool.dtype
    fill = BF16_NAN if w.dtype == "bf16" else np.float32(np.nan)
    pool = np.full((num_pages, PAGE_ROWS * pw), fill, dtype=store_t)
    As, Bs = [], []
    for p, (_, d_in, d_out) in enumerate(shapes):
        tb = tables[p]
        Ap, Bp = [], []
        for a in range(N):
            r = int(w.ranks[a])
            Aa = np.zeros((d_in, r_max), store_t)
            Aa[:, :r] = w.A[p][a]
            Ba = np.zeros((r_max, d_out), store_t)
            Ba[:r, :] = w.B[p][a]
            pool[tb.a_pages[tb.a_indptr[a]:tb.a_indptr[a + 1]]] = pack_a_pages(Aa, pw, fill)
            pool[tb.b_pages[tb.b_indptr[a]:tb.b_indptr[a + 1]]] = pack_b_pages(Ba, pw, fill)
            Ap.append(Aa)
            Bp.append(Ba)
        As.append(Ap)
        Bs.append(Bp)
    return Workload(cfg=w.cfg, name=w.name + f"-padded-r{r_max}", dtype=w.dtype, T=w.T, N=N, ids=w.ids,
                    ranks=ranks, alpha=alpha, page_width=pw, tables=tables, num_pages=num_pages, pool=pool,
                    X=w.X, Y_base=w.Y_base, A=As, B=Bs, seq_lens=w.seq_lens)
