"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Segments and every integer output must be bit-exact.  Y must agree within the
row-wise infinity-norm relative error 1e-2 in bf16 mode and 1e-5 in fp32 mode
(error measure: max over rows of max_j |Y - Y_ref| / max_j |Y_ref|).
Closed forms, isolation, permutation and determinism are checked bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from heterogeneous_adapters_amd import batch, lora

pytestmark = pytest.mark.gpu
TOL = {"bf16": 1e-2, "f32": 1e-5}


def rowwise_rel(Y, Yref):
    Y = np.asarray(Y, np.float64)
    Yref = np.asarray(Yref, np.float64)
    if len(Y) == 0:
        return 0.0
    den = np.maximum(np.abs(Yref).max(axis=1), 1e-30)
    return float((np.abs(Y - Yref).max(axis=1) / den).max())


def fence_tables(b):
    """Give each page table a tail of ids past any pool (INT32_MAX), read
    through views of the table's own length, so that a read past a table's
    end takes such an id and raises LORA_FLAG_PAGE_RANGE (which every parity
    case checks)."""
    def fenced(t):
        f = torch.full((t.numel() + 64,), 2 ** 31 - 1, dtype=t.dtype, device=t.device)
        f[:t.numel()] = t
        return f[:t.numel()]
    b.tables = [(ai, fenced(ap), bi, fenced(bp)) for ai, ap, bi, bp in b.tables]


def gpu_apply(w, in_place=False, pool=None, ids=None, via="apply"):
    """Run the whole branch on the GPU; returns host Y per projection and
    the segment arrays.  Page tables are fenced (fence_tables)."""
    b = batch.to_device(w, pool=pool)
    fence_tables(b)
    if ids is not None:
        b.ids = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    segs = lora.Segments(w.T, w.N)
    projs = [b.proj(p, in_place) for p in range(w.n_projs)]
    max_din = max(t.d_in for t in w.tables)
    ws = lora.workspace(w.T, w.N, w.n_projs, max_din)
    if via == "apply":
        lora.lora_apply(b.ids, segs, w.T, projs, b.adapters, b.pool, ws)
    elif via == "split_group":
        # the whole group through lora_shrink then lora_expand: the launches of lora_apply
        lora.lora_build_segments(b.ids, b.adapters, segs, ws)
        stride = max(w.T, 1) * lora.LORA_MAX_RANK
        vs = [torch.empty(lora.lora_v_slices(t.d_in) * stride, dtype=torch.float32, device="cuda")
              for t in w.tables]
        lora.lora_shrink(projs, b.adapters, segs, b.pool, vs, stride)
        lora.lora_expand(projs, b.adapters, segs, b.pool, vs, 0, stride)
    else:
        lora.lora_build_segments(b.ids, b.adapters, segs, ws)
        for p, pr in enumerate(projs):
            nq = lora.lora_v_slices(w.tables[p].d_in)
            stride = max(w.T, 1) * lora.LORA_MAX_RANK
            v = torch.empty(nq * stride, dtype=torch.float32, device="cuda")
            lora.lora_shrink(pr, b.adapters, segs, b.pool, v, stride)
            lora.lora_expand(pr, b.adapters, segs, b.pool, v, nq, stride)
    torch.cuda.synchronize()
    out = [batch.device_to_host(b.Y_base[p] if in_place else b.Y[p]) for p in range(w.n_projs)]
    return out, segs.arrays()


def oracle_Y(w, p, ids=None, pool=None):
    return oracle.apply(w.X[p], w.Y_base[p], w.ids if ids is None else ids, w.ranks, w.alpha, w.tables[p],
                        w.pool if pool is None else pool, w.page_width, w.dtype)


def check_segments(got, want):
    assert got["S"] == want["S"]
    assert got["n_invalid"] == want["n_invalid"]
    assert got["T_valid"] == want["T_valid"]
    assert got["V_total"] == want["V_total"]
    for k in ("perm", "seg_indptr", "seg_adapter", "v_indptr"):
        assert np.array_equal(got[k], want[k]), k
    assert got["flags"] == 0


# ----------------------------------------------------------------- runtime
def test_one_hip_runtime_mapped():
    lora.lib()
    torch.zeros(1, device="cuda")
    maps = lora.hip_runtimes_mapped()
    assert len(maps) == 1, maps


# ---------------------------------------------------------------- segments
def _segments_gpu(ids, ranks):
    T, N = len(ids), len(ranks)
    ad = lora.Adapters(torch.from_numpy(np.asarray(ranks, np.int32)).cuda(),
                       torch.ones(N, dtype=torch.float32, device="cuda"))
    segs = lora.Segments(T, N)
    ws = lora.workspace(T, N, 0, 0)
    lora.lora_build_segments(torch.from_numpy(np.asarray(ids, np.int32)).cuda(), ad, segs, ws)
    return segs.arrays()


@pytest.mark.parametrize("k", [0, 1, 2, 3, 4])
def test_segments_bit_exact_configs(k):
    ids, ranks, _, _ = W.draw_ids_and_ranks(k)
    print(f"segments config {k}: T={len(ids)} N={len(ranks)}", flush=True)
    check_segments(_segments_gpu(ids, ranks), oracle.segments(ids, ranks))


@pytest.mark.parametrize("case", ["T1", "all_base", "invalid_mix", "bad_rank", "one_adapter_long",
                                  "many_adapters", "ragged_chunks", "max_adapters"])
def test_segments_bit_exact_edges(case):
    rng = np.random.default_rng(hash(case) % 2 ** 31)
    if case == "T1":
        ids, ranks = np.array([2], np.int32), np.array([8, 8, 8], np.int32)
    elif case == "all_base":
        ids, ranks = np.full(37, -1, np.int32), np.array([16, 8], np.int32)
    elif case == "invalid_mix":
        ranks = rng.choice([8, 16, 64], 20).astype(np.int32)
        ids = rng.integers(-5, 25, 3000).astype(np.int32)
    elif case == "bad_rank":
        ranks = rng.choice([0, 8, 129, 16], 30).astype(np.int32)
        ids = rng.integers(0, 30, 2500).astype(np.int32)
    elif case == "one_adapter_long":
        ranks = np.array([32], np.int32)
        ids = np.zeros(5000, np.int32)
    elif case == "many_adapters":
        ranks = rng.choice([8, 16, 32, 64], 5000).astype(np.int32)
        ids = rng.integers(0, 5000, 700).astype(np.int32)
    elif case == "ragged_chunks":
        ranks = rng.choice([1, 24, 128], 7).astype(np.int32)
        ids = rng.integers(0, 7, 2 * 1024 + 17).astype(np.int32)
    else:  # the largest adapter count the ABI accepts: sparse ids, two hot adapters at both ends
        N = lora.LORA_MAX_ADAPTERS
        ranks = rng.integers(1, lora.LORA_MAX_RANK + 1, N).astype(np.int32)
        ids = np.concatenate([rng.integers(0, N, 2500), np.full(300, N - 1), np.zeros(200), [-1, N, N + 5]])
        ids = rng.permutation(ids.astype(np.int32)).astype(np.int32)
    print(f"segments edge {case}: T={len(ids)} N={len(ranks)}", flush=True)
    check_segments(_segments_gpu(ids, ranks), oracle.segments(ids, ranks))


# ------------------------------------------------------------------- apply
def _tile_boundary_ids():
    """Adapters 0-9 hold exactly 16, 17, 31, 32, 33, 47, 48, 63, 64 and 65
    tokens (MBGMM segments around the 16- and 32-token tile sizes), adapters
    10-14 one to three (MBGMV), interleaved by a seeded shuffle."""
    counts = [16, 17, 31, 32, 33, 47, 48, 63, 64, 65, 1, 2, 3, 1, 2]
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    return np.random.default_rng(11).permutation(ids).astype(np.int32)


_TILE_RANKS = [8, 16, 24, 32, 64, 128, 1, 40, 17, 96, 8, 16, 32, 64, 128]


def _long_tile_ids():
    """Adapters 0-6 hold 511, 512, 513, 575, 576, 577 and 639 tokens (both
    sides of the segment length that switches the MBGMM shrink to its long
    items, and of their 64-token tiles of two rank groups: ranks 64, 128 and
    40 sit on 576, 577 and 639 tokens, so a tile takes two, four and two
    items, the last with one group past the rank), adapters 7-8 one and two
    (MBGMV), interleaved by a seeded shuffle."""
    counts = [511, 512, 513, 575, 576, 577, 639, 1, 2]
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    return np.random.default_rng(13).permutation(ids).astype(np.int32)


_LONG_TILE_RANKS = [8, 16, 24, 32, 64, 128, 40, 16, 64]


def _last_adapter_long_ids():
    """300 tokens of the last adapter (an MBGMM segment whose page-table row
    is the table's last) among 100 spread over the others, shuffled."""
    ids = np.concatenate([np.full(300, 4, np.int32), np.arange(100, dtype=np.int32) % 4])
    return np.random.default_rng(17).permutation(ids).astype(np.int32)

def _prefill_base_only_ids():
    """14 sequences of 600 tokens over 7 adapters, two of them base-model
    sequences (id -1), plus 40 scattered base-model tokens."""
    ids = np.concatenate([np.full(600, -1 if q in (3, 9) else q % 7, np.int32) for q in range(14)])
    ids[np.random.default_rng(23).choice(len(ids), 40, replace=False)] = -1
    return ids


PARITY_CASES = {
    "cfg0": (0, {}),
    "cfg1": (1, {}),
    "cfg2": (2, {}),
    "cfg2_f32": (2, dict(dtype="f32")),
    "cfg3": (3, {}),
    "tails_bf16": (2, dict(T=300, N=7, ranks_override=[1, 4, 24, 40, 17, 128, 8], page_width=256,
                           projs=(("a", 1000, 744), ("b", 2056, 520)))),
    "tails_f32": (2, dict(T=300, N=7, ranks_override=[1, 4, 24, 40, 17, 128, 8], page_width=64,
                          dtype="f32", projs=(("a", 1000, 744), ("b", 520, 2056)))),
    "hot_segments": (2, dict(T=700, N=3, ranks_override=[8, 64, 128], page_width=512,
                             projs=(("a", 4096, 1032),))),
    "pw64_contig": (1, dict(T=96, N=5, page_width=64, projs=(("q", 512, 512),))),
    # an output narrower than an MBGMM expand item's columns (4 waves x 128):
    # two waves of each item have no columns, and their page column lies past
    # the table row of the last adapter
    "small_dout_last_adapter": (2, dict(N=5, ranks_override=[8, 16, 40, 64, 128], ids_override=_last_adapter_long_ids(),
                                        page_width=256, scatter=False, projs=(("a", 648, 136),))),
    # segment lengths on both sides of the MBGMM tile sizes; page width 256 puts
    # the fp32 case on the wide kernel with MBGMM items as wide as a page
    "tile_lengths_bf16": (2, dict(N=15, ranks_override=_TILE_RANKS, ids_override=_tile_boundary_ids(),
                                  page_width=256, projs=(("a", 1000, 1032), ("b", 1032, 520)))),
    "tile_lengths_f32": (2, dict(N=15, ranks_override=_TILE_RANKS, ids_override=_tile_boundary_ids(),
                                 page_width=256, dtype="f32", projs=(("a", 1000, 1032), ("b", 1032, 520)))),
    "long_tile_lengths_bf16": (2, dict(N=9, ranks_override=_LONG_TILE_RANKS, ids_override=_long_tile_ids(),
                                       page_width=512, projs=(("a", 1032, 520),))),
    "long_tile_lengths_f32": (2, dict(N=9, ranks_override=_LONG_TILE_RANKS, ids_override=_long_tile_ids(),
                                      page_width=256, dtype="f32", projs=(("a", 1032, 520),))),
    # very wide projections: 65 and 41 split-K slices, the last 8 columns wide,
    # and ragged last column blocks, on the wide-page bf16 and narrow-page fp32
    # kernels, with MBGMV and MBGMM segments
    "wide_dims_bf16": (2, dict(T=200, N=6, ranks_override=[1, 16, 33, 64, 128, 8], page_width=512,
                               projs=(("a", 32776, 16392),))),
    "wide_dims_f32": (2, dict(T=120, N=6, ranks_override=[1, 16, 33, 64, 128, 8], page_width=128,
                              dtype="f32", projs=(("a", 20488, 12296),))),
    # the narrowest projections the ABI accepts (8 columns: one 16-byte bf16
    # row, a lone ragged slice / column block), MBGMV and MBGMM segments
    "min_dims_bf16": (2, dict(T=300, N=7, ranks_override=[1, 4, 24, 40, 17, 128, 8], page_width=64,
                              projs=(("a", 8, 8), ("b", 8, 1032), ("c", 1032, 8)))),
    "min_dims_f32": (2, dict(T=300, N=7, ranks_override=[1, 4, 24, 40, 17, 128, 8], page_width=256,
                             dtype="f32", projs=(("a", 8, 8), ("b", 8, 1032), ("c", 1032, 8)))),
    # continuous batching: prefill chunks (MBGMM) beside decode tokens (MBGMV)
    "mixed": (5, dict(nchunks=3, chunk_lo=40, chunk_hi=120, ndecode=300, N=50, page_width=512,
                      projs=(("a", 1024, 1536),))),
    # prefill batches with more than three MBGMM expand items per block of the
    # grid (the expand kernel's per-XCD queues): fp32 (2196 items for 512
    # blocks), and bf16 with a ragged last column block (2525 items for 768)
    "prefill_queues_f32": (3, dict(dtype="f32", nseq=8, len_lo=600, len_hi=900, N=6, page_width=1024,
                                   projs=(("a", 512, 11008),))),
    "prefill_queues_ragged_bf16": (3, dict(nseq=12, len_lo=500, len_hi=900, N=7, page_width=512,
                                           projs=(("a", 520, 9000),))),
    # the same queues beside copy items: base-model rows written out of place
    "prefill_queues_base_only": (3, dict(N=7, page_width=512, ids_override=_prefill_base_only_ids(),
                                         projs=(("a", 520, 11008),))),
}


@pytest.mark.parametrize("name", list(PARITY_CASES))
def test_apply_matches_oracle(name):
    k, kw = PARITY_CASES[name]
    w = W.make_workload(k, kw, keep_dense=False)
    print(f"apply parity {name}: T={w.T} N={w.N} dtype={w.dtype} projs={[(t.d_in, t.d_out) for t in w.tables]}",
          flush=True)
    Ys, seg = gpu_apply(w)
    check_segments(seg, oracle.segments(w.ids, w.ranks))
    for p in range(w.n_projs):
        ref = oracle_Y(w, p)
        got = W.as_f64(Ys[p], w.dtype)
        assert np.isfinite(got).all()
        err = rowwise_rel(got, W.as_f64(ref, w.dtype))
        print(f"  proj {p}: rowwise rel err {err:.3e}", flush=True)
        assert err < TOL[w.dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_shrink_expand_entry_points(dtype):
    w = W.make_workload(2, dict(T=200, N=6, dtype=dtype, ranks_override=[8, 16, 64, 24, 1, 32],
                                projs=(("a", 4096, 1000),), page_width=256), keep_dense=False)
    Y1, seg = gpu_apply(w, via="apply")
    Y2, _ = gpu_apply(w, via="split")
    assert np.array_equal(Y1[0], Y2[0])
    Y3, _ = gpu_apply(w, via="split_group")
    for p in range(w.n_projs):
        assert np.array_equal(Y1[p], Y3[p])
    # shrink alone: sum of the partial slices against the oracle's v
    b = batch.to_device(w)
    segs = lora.Segments(w.T, w.N)
    ws = lora.workspace(w.T, w.N, 1, 4096)
    lora.lora_build_segments(b.ids, b.adapters, segs, ws)
    stride = w.T * 128
    nq = lora.lora_v_slices(4096)
    v = torch.zeros(nq * stride, dtype=torch.float32, device="cuda")
    lora.lora_shrink(b.proj(0), b.adapters, segs, b.pool, v, stride)
    torch.cuda.synchronize()
    vh = v.cpu().numpy().reshape(nq, stride)
    V = seg["V_total"]
    vg = vh[:, :V].sum(axis=0)
    vo = oracle.shrink(w.X[0], oracle.segments(w.ids, w.ranks), w.ranks, w.tables[0], w.pool,
                       w.page_width, w.dtype)
    tol = 1e-5 if dtype == "f32" else 1e-3
    assert np.abs(vg - vo).max() <= tol * np.abs(vo).max()
    # expand alone, fed the oracle's v as one slice
    vin = torch.zeros(stride, dtype=torch.float32, device="cuda")
    vin[:V] = torch.from_numpy(vo)
    lora.lora_expand(b.proj(0), b.adapters, segs, b.pool, vin, 1, stride)
    torch.cuda.synchronize()
    got = W.as_f64(batch.device_to_host(b.Y[0]), w.dtype)
    assert rowwise_rel(got, W.as_f64(oracle_Y(w, 0), w.dtype)) < TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_hot_closed_form_exact_on_gpu(dtype):
    """One-hot A and B: each sum has a single non-zero term, so the GPU must
    agree with the oracle bit for bit on both the MBGMV and MBGMM paths."""
    w = W.make_workload(2, dict(T=120, N=4, dtype=dtype, ranks_override=[8, 16, 5, 64],
                                ids_override=np.r_[np.zeros(60), np.ones(30), np.full(20, 2), np.full(10, 3)]
                                .astype(np.int32)[np.random.default_rng(0).permutation(120)],
                                projs=(("a", 1536, 768),), page_width=256), keep_dense=False)
    rng = np.random.default_rng(9)
    pool = w.pool.copy()
    tb = w.tables[0]
    fill = W.BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    for a in range(w.N):
        r = int(w.ranks[a])
        A = np.zeros((1536, r), np.float32)
        B = np.zeros((r, 768), np.float32)
        A[rng.permutation(1536)[:r], np.arange(r)] = 1.0
        B[np.arange(r), rng.permutation(768)[:r]] = 1.0
        if dtype == "bf16":
            A, B = W.f32_to_bf16_bits(A), W.f32_to_bf16_bits(B)
        pool[tb.a_pages[tb.a_indptr[a]:tb.a_indptr[a + 1]]] = W.pack_a_pages(A, w.page_width, fill)
        pool[tb.b_pages[tb.b_indptr[a]:tb.b_indptr[a + 1]]] = W.pack_b_pages(B, w.page_width, fill)
    pool_d = batch.host_to_device(pool, dtype, "cuda")
    Y, _ = gpu_apply(w, pool=pool_d)
    assert np.array_equal(Y[0], oracle_Y(w, 0, pool=pool))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_isolation_bit_exact_on_gpu(dtype):
    w = W.make_workload(2, dict(T=256, N=8, dtype=dtype, projs=(("a", 1024, 2048),), page_width=512),
                        keep_dense=False)
    b = int(np.bincount(w.ids).argmax())
    tb = w.tables[0]
    pages = np.concatenate([tb.a_pages[tb.a_indptr[b]:tb.a_indptr[b + 1]],
                            tb.b_pages[tb.b_indptr[b]:tb.b_indptr[b + 1]]])
    pool2 = w.pool.copy()
    if dtype == "bf16":
        pool2[pages] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(pool2[pages]) * np.float32(-3.0))
    else:
        pool2[pages] *= np.float32(-3.0)
    Y0, _ = gpu_apply(w)
    Y1, _ = gpu_apply(w, pool=batch.host_to_device(pool2, dtype, "cuda"))
    other = w.ids != b
    assert np.array_equal(Y0[0][other], Y1[0][other])
    assert not np.array_equal(Y0[0][~other], Y1[0][~other])


def test_permutation_and_determinism_on_gpu():
    w = W.make_workload(2, dict(T=400, N=6, projs=(("a", 2048, 1024),), page_width=1024), keep_dense=False)
    Y0, _ = gpu_apply(w)
    Y0b, _ = gpu_apply(w)
    assert np.array_equal(Y0[0], Y0b[0])
    perm = np.random.default_rng(4).permutation(w.T)
    w2 = W.make_workload(2, dict(T=400, N=6, projs=(("a", 2048, 1024),), page_width=1024), keep_dense=False)
    w2.ids = w.ids[perm]
    w2.X = [w.X[0][perm]]
    w2.Y_base = [w.Y_base[0][perm]]
    Y1, _ = gpu_apply(w2)
    assert np.array_equal(Y1[0], Y0[0][perm])


@pytest.mark.parametrize("in_place", [False, True])
def test_base_only_and_invalid_tokens(in_place):
    w = W.make_workload(2, dict(T=160, N=5, projs=(("a", 1024, 512),), page_width=256), keep_dense=False)
    ids = w.ids.copy()
    ids[::7] = -1
    ids[3::11] = 99
    Y, seg = gpu_apply(w, in_place=in_place, ids=ids)
    want = oracle.segments(ids, w.ranks)
    check_segments(seg, want)
    excl = (ids < 0) | (ids >= w.N)
    assert np.array_equal(Y[0][excl], w.Y_base[0][excl])
    err = rowwise_rel(W.as_f64(Y[0], w.dtype), W.as_f64(oracle_Y(w, 0, ids=ids), w.dtype))
    assert err < TOL[w.dtype]


def test_in_place_equals_out_of_place():
    w = W.make_workload(2, dict(T=333, N=9, projs=(("a", 2048, 3000),), page_width=1024), keep_dense=False)
    Y0, _ = gpu_apply(w, in_place=False)
    Y1, _ = gpu_apply(w, in_place=True)
    assert np.array_equal(Y0[0], Y1[0])


def test_wide_f32_against_float64_definition():
    """The fp32 oracle sums d_in products in sequence, so its own error grows
    about as sqrt(d_in) * 2^-24: at d_in = 20488 it lies 9e-6 from the float64
    value of the definition.  The HIP path (512-input partial sums added in
    ascending order) is checked here against that float64 value directly."""
    k, kw = PARITY_CASES["wide_dims_f32"]
    w = W.make_workload(k, kw, keep_dense=True)
    Ys, _ = gpu_apply(w)
    X = np.asarray(w.X[0], np.float64)
    Y64 = np.asarray(w.Y_base[0], np.float64).copy()
    for t in range(w.T):
        a = int(w.ids[t])
        if 0 <= a < w.N:
            A = np.asarray(w.A[0][a], np.float64)
            B = np.asarray(w.B[0][a], np.float64)
            Y64[t] += float(w.alpha[a]) / int(w.ranks[a]) * ((X[t] @ A) @ B)
    err_gpu = rowwise_rel(W.as_f64(Ys[0], w.dtype), Y64)
    err_oracle = rowwise_rel(W.as_f64(oracle_Y(w, 0), w.dtype), Y64)
    print(f"  vs float64 definition: HIP {err_gpu:.3e}, oracle {err_oracle:.3e}", flush=True)
    assert err_gpu < TOL["f32"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strided_rows_match_contiguous(dtype):
    """Projections whose rows are column slices of wider tensors: X inside
    padded rows (ldx = d_in + 24), Y_base and Y slices of one fused q/k/v
    output (ldy = 3 d_out, plus 8 pad columns for Y).  Y is bit-identical to
    the run on contiguous rows, in and out of place, and no column outside
    the slices is written."""
    d_in, d_out = 1032, 520
    w = W.make_workload(2, dict(T=300, N=9, ranks_override=[8, 16, 64, 24, 1, 32, 128, 40, 8], page_width=256,
                                dtype=dtype, projs=(("q", d_in, d_out), ("k", d_in, d_out), ("v", d_in, d_out))),
                        keep_dense=False)
    Yref, _ = gpu_apply(w)
    for in_place in (False, True):
        b = batch.to_device(w)
        T, dt = w.T, b.X[0].dtype
        Xw = [torch.zeros(T, d_in + 24, dtype=dt, device="cuda") for _ in range(3)]
        Ybw = torch.empty(T, 3 * d_out, dtype=dt, device="cuda")
        Yw = torch.full((T, 3 * d_out + 8), 5.0, dtype=dt, device="cuda")
        for p in range(3):
            Xw[p][:, 8:8 + d_in] = b.X[p]
            Ybw[:, p * d_out:(p + 1) * d_out] = b.Y_base[p]
        out = Ybw if in_place else Yw
        projs = [lora.Proj(Xw[p][:, 8:8 + d_in], Ybw[:, p * d_out:(p + 1) * d_out],
                           out[:, p * d_out:(p + 1) * d_out], *b.tables[p]) for p in range(3)]
        assert projs[0].c.ldx == d_in + 24 and projs[0].c.ldyb == 3 * d_out
        assert projs[0].c.ldy == (3 * d_out if in_place else 3 * d_out + 8)
        segs = lora.Segments(T, w.N)
        lora.lora_apply(b.ids, segs, T, projs, b.adapters, b.pool, lora.workspace(T, w.N, 3, d_in))
        torch.cuda.synchronize()
        for p in range(3):
            got = batch.device_to_host(out[:, p * d_out:(p + 1) * d_out])
            assert np.array_equal(got, Yref[p]), (in_place, p)
        if not in_place:
            assert bool((Yw[:, 3 * d_out:].float() == 5.0).all())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_page_ids_outside_the_pool_read_as_zero(dtype):
    """A page id outside the pool (here num_pages + 3 in an A table and -1 in
    a B table, for the hottest adapter (MBGMM path) and for the one with the
    fewest tokens (MBGMV path)) is read as a page of zeros and sets LORA_FLAG_PAGE_RANGE; no
    access leaves the pool.  Expected Y: the oracle on the same tables with
    those ids pointing at an appended all-zero page."""
    import dataclasses
    w = W.make_workload(2, dict(T=300, N=9, ranks_override=[8, 16, 64, 24, 40, 32, 128, 17, 8], page_width=256,
                                dtype=dtype, projs=(("a", 1032, 744),)), keep_dense=False)
    seg = oracle.segments(w.ids, w.ranks)
    cnt = np.diff(seg["seg_indptr"])
    hot = int(seg["seg_adapter"][np.argmax(cnt)])
    cold = int(seg["seg_adapter"][np.argmin(cnt)])
    assert cnt.max() >= 16 > cnt.min() and hot != cold
    t = w.tables[0]
    bad, zero = dataclasses.replace(t), dataclasses.replace(t)
    for f in ("a_pages", "b_pages"):
        setattr(bad, f, getattr(t, f).copy())
        setattr(zero, f, getattr(t, f).copy())
    for a, k in ((hot, 1), (cold, 0)):
        ia, ib = int(t.a_indptr[a]) + k, int(t.b_indptr[a + 1]) - 1 - k
        bad.a_pages[ia], bad.b_pages[ib] = w.num_pages + 3, -1
        zero.a_pages[ia] = zero.b_pages[ib] = w.num_pages
    pool0 = np.concatenate([w.pool, np.zeros((1, w.pool.shape[1]), w.pool.dtype)])
    want = oracle.apply(w.X[0], w.Y_base[0], w.ids, w.ranks, w.alpha, zero, pool0, w.page_width, w.dtype)
    plain = oracle_Y(w, 0)
    touched = (w.ids == hot) | (w.ids == cold)
    assert not np.array_equal(want[touched], plain[touched])  # the zeroed pages matter
    Ys, segs = gpu_apply(dataclasses.replace(w, tables=[bad]))
    assert segs["flags"] & 1
    assert rowwise_rel(W.as_f64(Ys[0], w.dtype), W.as_f64(want, w.dtype)) < TOL[w.dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_invalid_ranks_leave_base_rows(dtype):
    """Adapters whose rank lies outside [1, 128] (0, 129, -4, 200) are
    counted invalid: their tokens' rows equal Y_base bit for bit, their page
    tables are never read, and the other tokens match the oracle."""
    import dataclasses
    w = W.make_workload(2, dict(T=300, N=6, ranks_override=[8, 8, 8, 16, 8, 64], page_width=256, dtype=dtype,
                                projs=(("a", 1032, 744),)), keep_dense=False)
    w = dataclasses.replace(w, ranks=np.array([8, 0, 129, 16, -4, 200], np.int32))
    Ys, segs = gpu_apply(w)
    check_segments(segs, oracle.segments(w.ids, w.ranks))
    bad = np.isin(w.ids, [1, 2, 4, 5])
    assert bad.any() and segs["n_invalid"] == int(bad.sum())
    assert np.array_equal(Ys[0][bad], w.Y_base[0][bad])
    assert rowwise_rel(W.as_f64(Ys[0], w.dtype), W.as_f64(oracle_Y(w, 0), w.dtype)) < TOL[w.dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_alpha_returns_base_exactly(dtype):
    """alpha = 0 scales every adapter's update by zero, so Y = Y_base bit for
    bit on both paths (the weights are finite)."""
    w = W.make_workload(2, dict(T=200, N=12, ranks_override=[8, 64, 128, 1, 24, 16] * 2, page_width=256,
                                dtype=dtype, alpha_override=[0.0] * 12, projs=(("a", 1032, 744),)), keep_dense=False)
    seg = oracle.segments(w.ids, w.ranks)
    assert max(np.diff(seg["seg_indptr"])) >= 16 and min(np.diff(seg["seg_indptr"])) < 16
    Ys, _ = gpu_apply(w)
    assert np.array_equal(Ys[0], w.Y_base[0])


def test_empty_batch():
    """T = 0: every entry point accepts the empty batch, its kernels find no
    items and nothing is written (the buffers of a real batch stand behind
    the descriptors, so a stray row store would show).  torch hands an empty
    ids tensor over as a null pointer, which lora_apply reads as "reuse
    segments"; at T = 0 it builds them all the same, so a buffer holding a
    stale flags word (every item count zero) comes back cleared."""
    w = W.make_workload(2, dict(T=64, N=5, projs=(("a", 1024, 512), ("b", 512, 1024)), page_width=256),
                        keep_dense=False)
    b = batch.to_device(w)
    for y in b.Y:
        y.fill_(3.0)
    projs = [b.proj(p, False) for p in range(w.n_projs)]
    ids0 = b.ids[:0]
    want = oracle.segments(w.ids[:0], w.ranks)
    segs = lora.Segments(0, w.N)
    ws = lora.workspace(0, w.N, w.n_projs, 1024)
    segs.counts().zero_()
    segs.counts()[lora.COUNT_FLAGS] = 5
    lora.lora_apply(ids0, segs, 0, projs, b.adapters, b.pool, ws)
    check_segments(segs.arrays(), want)
    stride = lora.LORA_MAX_RANK
    vs = [torch.zeros(lora.lora_v_slices(t.d_in) * stride, dtype=torch.float32, device="cuda") for t in w.tables]
    segs.counts()[lora.COUNT_FLAGS] = 5
    lora.lora_build_segments(ids0, b.adapters, segs, ws)
    check_segments(segs.arrays(), want)
    lora.lora_shrink(projs, b.adapters, segs, b.pool, vs, stride)
    lora.lora_expand(projs, b.adapters, segs, b.pool, vs, 0, stride)
    lora.lora_apply(None, segs, 0, projs, b.adapters, b.pool, ws)
    lora.lora_apply(ids0, None, 0, projs, b.adapters, b.pool, lora.workspace(0, w.N, w.n_projs, 1024))
    torch.cuda.synchronize()
    check_segments(segs.arrays(), want)
    for y in b.Y:
        assert bool((y.float() == 3.0).all())
    for v in vs:
        assert bool((v == 0).all())


def test_many_projections_in_one_call():
    """More projections than one launch holds: the call is split in groups."""
    w = W.make_workload(2, dict(T=64, N=5, projs=(("a", 256, 512),), layers=19, page_width=256),
                        keep_dense=False)
    Ys, _ = gpu_apply(w)
    for p in range(w.n_projs):
        assert rowwise_rel(W.as_f64(Ys[p], w.dtype), W.as_f64(oracle_Y(w, p), w.dtype)) < TOL[w.dtype]
    # the same groups through lora_shrink / lora_expand: bit-identical
    Yg, _ = gpu_apply(w, via="split_group")
    for p in range(w.n_projs):
        assert np.array_equal(Ys[p], Yg[p])


def test_excluded_token_at_last_chunk_position():
    """Regression: a token without an adapter at position 1023 of a full
    1024-token chunk must still be placed (its sort key is distinct from the
    padding key)."""
    ids = np.zeros(2048, np.int32)
    ids[1023] = -1
    ids[2047] = 77
    ids[5] = -1
    ranks = np.array([16, 8], np.int32)
    check_segments(_segments_gpu(ids, ranks), oracle.segments(ids, ranks))


def test_graph_capture_replays_match_eager():
    """The whole branch (segment build + apply) captured in a HIP graph:
    every replay, with eager work and synchronisation in between, equals the
    eager result bit for bit (the library records only kernel launches)."""
    w = W.make_workload(2, dict(T=300, N=9, ranks_override=[8, 16, 64, 24, 1, 32, 128, 40, 8], page_width=512,
                                projs=(("a", 2048, 1032), ("b", 1032, 2048))), keep_dense=False)
    Yref, _ = gpu_apply(w)
    b = batch.to_device(w)
    segs = lora.Segments(w.T, w.N)
    projs = [b.proj(p) for p in range(w.n_projs)]
    ws = lora.workspace(w.T, w.N, w.n_projs, 2048)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lora.lora_apply(b.ids, segs, w.T, projs, b.adapters, b.pool, ws, side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        lora.lora_apply(b.ids, segs, w.T, projs, b.adapters, b.pool, ws, side)
    torch.cuda.synchronize()
    for rep in range(3):
        for y in b.Y:
            y.fill_(7.0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for p in range(w.n_projs):
            assert np.array_equal(batch.device_to_host(b.Y[p]), Yref[p]), (rep, p)


def test_prefill_item_queues_repeat_and_replay():
    """A prefill batch (32 sequences, 38,781 tokens: about six MBGMM expand
    items per work-group) takes the expand kernel's per-XCD item queues,
    whose counters the last work-group of each XCD puts back to zero.  Calls
    in a row on one segment buffer built once (the builder would zero the
    counters), and graph replays of the call, must each produce every row: Y
    is overwritten with NaN before every call and must come out bit-identical
    to the first call's."""
    w = W.make_workload(3, keep_dense=False)
    b = batch.to_device(w)
    segs = lora.Segments(w.T, w.N)
    projs = [b.proj(p) for p in range(w.n_projs)]
    ws = lora.workspace(w.T, w.N, w.n_projs, max(t.d_in for t in w.tables))
    lora.lora_build_segments(b.ids, b.adapters, segs, lora.workspace(w.T, w.N, 0, 0))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    first = None
    for rep in range(3):
        for y in b.Y:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            lora.lora_apply(None, segs, w.T, projs, b.adapters, b.pool, ws, side)
        torch.cuda.synchronize()
        got = [y.clone() for y in b.Y]
        if first is None:
            first = got
            assert all(not torch.isnan(y.float()).any() for y in got)
        else:
            assert all(torch.equal(a.view(torch.int16), c.view(torch.int16)) for a, c in zip(got, first)), rep
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        lora.lora_apply(None, segs, w.T, projs, b.adapters, b.pool, ws, side)
    torch.cuda.synchronize()
    for rep in range(3):
        for y in b.Y:
            y.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a.view(torch.int16), c.view(torch.int16)) for a, c in zip(b.Y, first)), ("replay", rep)


def test_padded_slot_layout_matches_unpadded():
    """The fixed-rank (padded) layout through the same kernels gives the same
    Y as the heterogeneous-rank layout, within the bf16 tolerance, and both
    match the oracle."""
    w = W.make_workload(2, dict(T=400, N=8, ranks_override=[8, 16, 32, 64, 8, 24, 1, 40], page_width=512,
                                projs=(("a", 2048, 1536),)))
    wp = W.pad_to_rank(w, 64)
    Y, _ = gpu_apply(w)
    Yp, _ = gpu_apply(wp)
    ref = W.as_f64(oracle_Y(w, 0), w.dtype)
    assert rowwise_rel(W.as_f64(Y[0], w.dtype), ref) < TOL["bf16"]
    assert rowwise_rel(W.as_f64(Yp[0], w.dtype), ref) < TOL["bf16"]


def test_shared_activation_group_matches_separate_inputs():
    """q/k/v reading one X tensor: the launch walks the three projections'
    shrink items side by side (shared X).  The result equals the same
    projections run with three separate copies of X, bit for bit."""
    w = W.make_workload(2, dict(T=350, N=7, ranks_override=[8, 16, 64, 24, 32, 8, 128], page_width=512,
                                projs=(("q", 1536, 1536), ("k", 1536, 512), ("v", 1536, 512))))
    ys = {}
    for mode in ("separate", "shared"):
        b = batch.to_device(w)
        if mode == "shared":
            for p in (1, 2):
                b.X[p] = b.X[0]
        else:
            for p in (1, 2):
                b.X[p] = b.X[0].clone()
        segs = lora.Segments(w.T, w.N)
        ws = lora.workspace(w.T, w.N, 3, 1536)
        lora.lora_apply(b.ids, segs, w.T, [b.proj(p) for p in range(3)], b.adapters, b.pool, ws)
        torch.cuda.synchronize()
        ys[mode] = [batch.device_to_host(b.Y[p]) for p in range(3)]
    for p in range(3):
        assert np.array_equal(ys["shared"][p], ys["separate"][p])
    # and the shared run against the oracle (X of projection 0 for all three)
    Xh = batch.device_to_host(batch.to_device(w).X[0])
    for p in range(3):
        ref = oracle.apply(Xh, w.Y_base[p], w.ids, w.ranks, w.alpha, w.tables[p], w.pool, w.page_width, w.dtype)
        assert rowwise_rel(W.as_f64(ys["shared"][p], w.dtype), W.as_f64(ref, w.dtype)) < TOL["bf16"]


def test_segment_buffer_larger_than_the_batch():
    """A segment buffer laid out for a larger batch (capacity T + 37 tokens,
    N + 5 adapters) serves the batch through every entry point, bit-identical
    to a buffer of the batch's own size.  Prebuilt segments reused with
    another token count, a buffer that was never built, and one whose item
    totals exceed its capacity are not walked: nothing is written and
    LORA_FLAG_SEGMENTS is raised."""
    w = W.make_workload(2, dict(T=300, N=9, ranks_override=[8, 16, 64, 24, 1, 32, 128, 40, 8], page_width=512,
                                projs=(("a", 1024, 1536), ("b", 1536, 1024))), keep_dense=False)
    Yref, segref = gpu_apply(w)
    b = batch.to_device(w)
    projs = [b.proj(p) for p in range(w.n_projs)]
    Tc, Nc = w.T + 37, w.N + 5
    big = lora.Segments(Tc, Nc)
    ws = lora.workspace(Tc, Nc, w.n_projs, 1536)

    def fetch():
        torch.cuda.synchronize()
        return [batch.device_to_host(b.Y[p]) for p in range(w.n_projs)]

    def check_big():
        got = big.arrays()
        assert got["flags"] == 0
        assert np.array_equal(got["perm"][:w.T], segref["perm"])
        for k in ("seg_indptr", "seg_adapter", "v_indptr", "S", "T_valid", "V_total", "n_invalid"):
            assert np.array_equal(got[k], segref[k]), k
        assert int(big.counts()[lora.COUNT_T]) == w.T

    # prebuilt into the larger buffer, then applied
    lora.lora_build_segments(b.ids, b.adapters, big, ws)
    lora.lora_apply(None, big, w.T, projs, b.adapters, b.pool, ws)
    Y = fetch()
    check_big()
    for p in range(w.n_projs):
        assert np.array_equal(Y[p], Yref[p]), p
    # built inside lora_apply into the larger buffer
    for y in b.Y:
        y.fill_(7.0)
    lora.lora_apply(b.ids, big, w.T, projs, b.adapters, b.pool, ws)
    Y = fetch()
    check_big()
    for p in range(w.n_projs):
        assert np.array_equal(Y[p], Yref[p]), p
    # the split entry points on the larger buffer (v strided by its capacity)
    for y in b.Y:
        y.fill_(7.0)
    stride = Tc * lora.LORA_MAX_RANK
    vs = [torch.empty(lora.lora_v_slices(t.d_in) * stride, dtype=torch.float32, device="cuda") for t in w.tables]
    lora.lora_shrink(projs, b.adapters, big, b.pool, vs, stride)
    lora.lora_expand(projs, b.adapters, big, b.pool, vs, 0, stride)
    Y = fetch()
    for p in range(w.n_projs):
        assert np.array_equal(Y[p], Yref[p]), p
    # reused with another token count: nothing computed, flag raised
    for y in b.Y:
        y.fill_(7.0)
    lora.lora_apply(None, big, w.T - 1, projs, b.adapters, b.pool, ws)
    Y = fetch()
    assert int(big.counts()[lora.COUNT_FLAGS]) & lora.FLAG_SEGMENTS
    for p in range(w.n_projs):
        assert bool((b.Y[p].float() == 7.0).all()), p
    # a buffer never built (zeroed counters): nothing computed, flag raised
    fresh = lora.Segments(w.T, w.N)
    fresh.buf.zero_()
    lora.lora_apply(None, fresh, w.T, projs, b.adapters, b.pool, ws)
    lora.lora_shrink(projs, b.adapters, fresh, b.pool, vs, stride)
    lora.lora_expand(projs, b.adapters, fresh, b.pool, vs, 0, stride)
    torch.cuda.synchronize()
    assert int(fresh.counts()[lora.COUNT_FLAGS]) & lora.FLAG_SEGMENTS
    for p in range(w.n_projs):
        assert bool((b.Y[p].float() == 7.0).all()), p
    # built, then one item total (index 4..7: shrink MBGMM / MBGMV, expand
    # MBGMM / MBGMV) pushed past the buffer's capacity: not walked either
    for idx in range(4, 8):
        segs_c = lora.Segments(w.T, w.N)
        lora.lora_build_segments(b.ids, b.adapters, segs_c, ws)
        torch.cuda.synchronize()
        segs_c.counts()[idx] = 1 << 29
        lora.lora_apply(None, segs_c, w.T, projs, b.adapters, b.pool, ws)
        lora.lora_shrink(projs, b.adapters, segs_c, b.pool, vs, stride)
        lora.lora_expand(projs, b.adapters, segs_c, b.pool, vs, 0, stride)
        torch.cuda.synchronize()
        assert int(segs_c.counts()[lora.COUNT_FLAGS]) & lora.FLAG_SEGMENTS, idx
        for p in range(w.n_projs):
            assert bool((b.Y[p].float() == 7.0).all()), (idx, p)


def test_single_launch_wait_give_up_is_flagged_and_recovers():
    """The apply kernel's bounded wait between its shrink and expand phases,
    forced to give up from the host (its target made unreachable): the launch
    still ends, LORA_FLAG_SYNC is raised, and the next call on the same
    segment buffer -- whose barrier bookkeeping the forced call advanced as
    usual -- is bit-identical to the two-launch path."""
    w = W.make_workload(2, dict(T=200, N=9, ranks_override=[8, 16, 64, 24, 1, 32, 128, 40, 8], page_width=512,
                                projs=(("a", 1024, 1536), ("b", 1536, 1024))), keep_dense=False)
    Ysplit, _ = gpu_apply(w, via="split_group")
    b = batch.to_device(w)
    projs = [b.proj(p) for p in range(w.n_projs)]
    segs = lora.Segments(w.T, w.N)
    ws = lora.workspace(w.T, w.N, w.n_projs, 1536)
    lora.lora_build_segments(b.ids, b.adapters, segs, ws)
    lora.lora_set_launch_mode(lora.LORA_LAUNCH_SINGLE)
    try:
        lora.lora_set_wait_limit(-200_000)  # every wait gives up after 0.2 ms
        lora.lora_apply(None, segs, w.T, projs, b.adapters, b.pool, ws)
        torch.cuda.synchronize()
    finally:
        lora.lora_set_wait_limit(0)
    assert int(segs.counts()[lora.COUNT_FLAGS]) & lora.FLAG_SYNC
    for rep in range(3):
        for y in b.Y:
            y.fill_(7.0)
        lora.lora_apply(None, segs, w.T, projs, b.adapters, b.pool, ws)
        torch.cuda.synchronize()
        for p in range(w.n_projs):
            assert np.array_equal(batch.device_to_host(b.Y[p]), Ysplit[p]), (rep, p)
    lora.lora_build_segments(b.ids, b.adapters, segs, ws)
    lora.lora_apply(None, segs, w.T, projs, b.adapters, b.pool, ws)
    torch.cuda.synchronize()
    lora.lora_set_launch_mode(lora.LORA_LAUNCH_AUTO)
    assert segs.arrays()["flags"] == 0


@pytest.mark.parametrize("k", [1, 2, 3, 5])
@pytest.mark.parametrize("mode", ["single", "two", "auto"])
def test_launch_modes_match_split_entry_points(k, mode):
    """lora_apply in each launch mode (one launch per group, two launches, or
    the automatic choice by batch size) against lora_shrink + lora_expand
    called directly: bit-identical Y on the benchmark configs (5: the mixed
    prefill + decode batch)."""
    w = W.make_workload(k, keep_dense=False)
    Ys, _ = gpu_apply(w, via="split_group")
    code = {"single": lora.LORA_LAUNCH_SINGLE, "two": lora.LORA_LAUNCH_TWO, "auto": lora.LORA_LAUNCH_AUTO}[mode]
    try:
        lora.lora_set_launch_mode(code)
        Ya, seg = gpu_apply(w)
    finally:
        lora.lora_set_launch_mode(lora.LORA_LAUNCH_AUTO)
    assert seg["flags"] == 0
    for p in range(w.n_projs):
        assert np.array_equal(Ya[p], Ys[p]), p


def _random_case(seed):
    """One seeded draw over the shapes the boundary admits: dtype, batch size
    (decode sizes, the single-launch limit and beyond it), adapter count,
    ranks 1-128 (multiples of 16 and ragged ones), page width, one to three
    projections with ragged or wide dimensions (multiples of 8), pool layout,
    base-only and out-of-range ids, and a run of one adapter long enough for
    the MFMA path."""
    rng = np.random.default_rng(5000 + seed)
    dtype = "f32" if seed % 4 == 3 else "bf16"
    T = int(rng.choice([1, 2, 7, 40, 130, 300, 700, 1500, 2100, 2600]))
    N = int(rng.integers(1, 65))
    ranks = np.where(rng.random(N) < 0.6, rng.choice([8, 16, 32, 64, 128], N),
                     rng.integers(1, 129, N)).astype(np.int32)
    pw = int(rng.choice([64, 128, 256, 512, 1024, 4096]))
    nproj = int(rng.integers(1, 4))
    # keep the oracle's work (tokens x rank x dims) to a few seconds
    dmax = 4096 if T <= 700 else 1536
    projs = tuple((f"p{i}", 8 * int(rng.integers(1, dmax // 8 + 1)), 8 * int(rng.integers(1, dmax // 8 + 1)))
                  for i in range(nproj))
    p_ad = rng.dirichlet(np.full(N, 0.3))
    ids = rng.choice(N, size=T, p=p_ad).astype(np.int32)
    if T >= 40:  # a run of one adapter: an MBGMM segment (or a long one)
        n_long = int(rng.integers(16, max(17, T // 2)))
        ids[rng.choice(T, n_long, replace=False)] = int(rng.integers(0, N))
    special = rng.random(T)
    ids[special < 0.05] = -1                    # base-only tokens
    ids[(special >= 0.05) & (special < 0.07)] = N + 3  # out of range: excluded and counted
    mode = [lora.LORA_LAUNCH_AUTO, lora.LORA_LAUNCH_SINGLE, lora.LORA_LAUNCH_TWO][seed % 3]
    kw = dict(T=T, N=N, dtype=dtype, page_width=pw, projs=projs, scatter=bool(seed % 2), seed=100 + seed,
              ids_override=ids, ranks_override=ranks)
    return kw, mode


@pytest.mark.parametrize("seed", range(16))
def test_random_shapes_match_oracle(seed):
    """Seeded random draws (see _random_case) through lora_apply in a drawn
    launch mode, against the oracle: segments bit-exact, Y within the mode's
    tolerance, rows of base-only and excluded tokens equal to Y_base."""
    kw, mode = _random_case(seed)
    print(f"random case {seed}: T={kw['T']} N={kw['N']} dtype={kw['dtype']} pw={kw['page_width']} "
          f"projs={[p[1:] for p in kw['projs']]} ranks<= {int(kw['ranks_override'].max())} mode={mode}", flush=True)
    w = W.make_workload(2, kw, keep_dense=False)
    try:
        lora.lora_set_launch_mode(mode)
        Ys, seg = gpu_apply(w)
    finally:
        lora.lora_set_launch_mode(lora.LORA_LAUNCH_AUTO)
    check_segments(seg, oracle.segments(w.ids, w.ranks))
    base = (w.ids < 0) | (w.ids >= w.N)
    for p in range(w.n_projs):
        ref = oracle_Y(w, p)
        got = W.as_f64(Ys[p], w.dtype)
        assert np.isfinite(got).all()
        err = rowwise_rel(got, W.as_f64(ref, w.dtype))
        print(f"  proj {p}: rowwise rel err {err:.3e}", flush=True)
        assert err < TOL[w.dtype]
        assert np.array_equal(got[base], W.as_f64(w.Y_base[p], w.dtype)[base])


@pytest.mark.parametrize("seed", range(12))
def test_random_layouts_match_contiguous(seed):
    """Seeded random draws run twice: contiguous rows through lora_apply
    (itself checked against the oracle by the draws above), and again with
    every layout option the boundary offers drawn at random -- rows inside
    wider tensors (ldx, ldyb, ldy), Y written in place over Y_base, one X
    tensor shared by projections of equal d_in, and the entry point
    (lora_apply in a drawn launch mode, or lora_shrink + lora_expand for the
    group or per projection).  Y must be bit-identical, and no column outside
    the rows' slices may be written."""
    kw, mode = _random_case(200 + seed)
    rng = np.random.default_rng(9000 + seed)
    share = bool(rng.integers(0, 2)) and len(kw["projs"]) > 1
    if share:
        d_in = kw["projs"][0][1]
        kw["projs"] = tuple((n, d_in, do) for n, _, do in kw["projs"])
    in_place = bool(rng.integers(0, 2))
    via = ["apply", "split_group", "split_each"][int(rng.integers(0, 3))]
    pads = [8 * int(rng.integers(0, 5)) for _ in range(3)]  # extra columns of X, Y_base and Y rows
    print(f"layout case {seed}: T={kw['T']} N={kw['N']} {kw['dtype']} pw={kw['page_width']} "
          f"projs={[p[1:] for p in kw['projs']]} share={share} in_place={in_place} via={via} pads={pads} "
          f"mode={mode}", flush=True)
    w = W.make_workload(2, kw, keep_dense=False)
    if share:  # one activation for every projection, in the reference run as well (as separate copies)
        w.X = [w.X[0]] * w.n_projs
    Yref, _ = gpu_apply(w)
    for p in range(w.n_projs):  # the contiguous run against the oracle as well
        assert rowwise_rel(W.as_f64(Yref[p], w.dtype), W.as_f64(oracle_Y(w, p), w.dtype)) < TOL[w.dtype]
    b = batch.to_device(w)
    fence_tables(b)
    T, dt, P = w.T, b.X[0].dtype, w.n_projs
    d_ins = [t.d_in for t in w.tables]
    d_outs = [t.d_out for t in w.tables]
    off = 8 if pads[0] else 0
    if share:
        Xs = torch.zeros(T, d_ins[0] + pads[0], dtype=dt, device="cuda")
        Xs[:, off:off + d_ins[0]] = b.X[0]
        Xv = [Xs[:, off:off + d_ins[0]]] * P
    else:
        Xw = [torch.zeros(T, d_ins[p] + pads[0], dtype=dt, device="cuda") for p in range(P)]
        for p in range(P):
            Xw[p][:, off:off + d_ins[p]] = b.X[p]
        Xv = [Xw[p][:, off:off + d_ins[p]] for p in range(P)]
    Ybw = [torch.empty(T, d_outs[p] + pads[1], dtype=dt, device="cuda") for p in range(P)]
    for p in range(P):
        Ybw[p][:, :d_outs[p]] = b.Y_base[p]
    Yw = [torch.full((T, d_outs[p] + pads[2]), 5.0, dtype=dt, device="cuda") for p in range(P)]
    Ybv = [Ybw[p][:, :d_outs[p]] for p in range(P)]
    outv = Ybv if in_place else [Yw[p][:, :d_outs[p]] for p in range(P)]
    projs = [lora.Proj(Xv[p], Ybv[p], outv[p], *b.tables[p]) for p in range(P)]
    segs = lora.Segments(T, w.N)
    ws = lora.workspace(T, w.N, P, max(d_ins))
    stride = max(T, 1) * lora.LORA_MAX_RANK
    try:
        lora.lora_set_launch_mode(mode)
        if via == "apply":
            lora.lora_apply(b.ids, segs, T, projs, b.adapters, b.pool, ws)
        else:
            lora.lora_build_segments(b.ids, b.adapters, segs, ws)
            vs = [torch.empty(lora.lora_v_slices(d) * stride, dtype=torch.float32, device="cuda") for d in d_ins]
            if via == "split_group":
                lora.lora_shrink(projs, b.adapters, segs, b.pool, vs, stride)
                lora.lora_expand(projs, b.adapters, segs, b.pool, vs, 0, stride)
            else:
                for p in range(P):
                    lora.lora_shrink(projs[p], b.adapters, segs, b.pool, vs[p], stride)
                    lora.lora_expand(projs[p], b.adapters, segs, b.pool, vs[p], lora.lora_v_slices(d_ins[p]), stride)
        torch.cuda.synchronize()
    finally:
        lora.lora_set_launch_mode(lora.LORA_LAUNCH_AUTO)
    assert segs.arrays()["flags"] == 0
    for p in range(P):
        got = batch.device_to_host(outv[p])
        assert np.array_equal(got, Yref[p]), p
        if not in_place and pads[2]:
            assert bool((Yw[p][:, d_outs[p]:].float() == 5.0).all()), p


@pytest.mark.parametrize("seed", range(6))
def test_random_graph_replays_match_eager(seed):
    """Seeded random draws (as test_random_shapes_match_oracle, in a drawn
    launch mode) captured in a HIP graph with their segment build: three
    replays, with eager work and a synchronisation before each, all equal the
    eager run bit for bit."""
    kw, mode = _random_case(440 + seed)  # batches of 7 to 2100 tokens, one and two launches
    print(f"graph case {seed}: T={kw['T']} N={kw['N']} {kw['dtype']} pw={kw['page_width']} "
          f"projs={[p[1:] for p in kw['projs']]} mode={mode}", flush=True)
    w = W.make_workload(2, kw, keep_dense=False)
    try:
        lora.lora_set_launch_mode(mode)
        Yref, _ = gpu_apply(w)
        b = batch.to_device(w)
        fence_tables(b)
        segs = lora.Segments(w.T, w.N)
        projs = [b.proj(p) for p in range(w.n_projs)]
        ws = lora.workspace(w.T, w.N, w.n_projs, max(t.d_in for t in w.tables))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            lora.lora_apply(b.ids, segs, w.T, projs, b.adapters, b.pool, ws, side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            lora.lora_apply(b.ids, segs, w.T, projs, b.adapters, b.pool, ws, side)
        torch.cuda.synchronize()
        for rep in range(3):
            for y in b.Y:
                y.fill_(7.0)  # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert segs.arrays()["flags"] == 0, rep
            for p in range(w.n_projs):
                assert np.array_equal(batch.device_to_host(b.Y[p]), Yref[p]), (rep, p)
    finally:
        lora.lora_set_launch_mode(lora.LORA_LAUNCH_AUTO)
