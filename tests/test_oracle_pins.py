"""Pins of the CPU oracle against what the pages and the mathematics fix.

Page citations:
  [MLSP] "Multi-LoRA Serving in Production: Architecture, Dynamic Adapter
         Swapping, and GPU Memory Management"
  [MLSA] "Multi-LoRA Serving Architecture: Serving Hundreds of Fine-Tuned
         Adapters on One GPU with vLLM and S-LoRA (2026)"
  [LAST] "LoRA Adapters at Serve Time with vLLM Multi-LoRA"

Each check is chosen so that a plausible slip in the oracle (a dropped term,
a transposed operand, a wrong scale, an off-by-one page index, a token that
sees another token's adapter) fails at least one of them.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def rowwise_rel(Y, Yref):
    """Row-wise infinity-norm relative error: max_t max_j |dY| / max_j |Yref|."""
    Y = np.asarray(Y, np.float64)
    Yref = np.asarray(Yref, np.float64)
    den = np.maximum(np.abs(Yref).max(axis=1), 1e-30)
    return float((np.abs(Y - Yref).max(axis=1) / den).max()) if len(Y) else 0.0


def small(k=2, **kw):
    base = dict(T=24, N=6, projs=(("up", 192, 320), ("down", 320, 192)), page_width=64,
                scatter=True)
    if k == 0:
        base = dict(T=16, N=4, page_width=64, scatter=True, projs=(("p", 256, 256),))
    base.update(kw)
    return W.make_workload(k, base)


def dense_reference(w, p, alpha=None, ids=None):
    """float64 brute force: one dense loop per adapter over its own tokens."""
    ids = w.ids if ids is None else ids
    alpha = w.alpha if alpha is None else alpha
    X = W.as_f64(w.X[p], w.dtype)
    Y = W.as_f64(w.Y_base[p], w.dtype).copy()
    for a in range(w.N):
        rows = np.nonzero(ids == a)[0]
        if len(rows) == 0:
            continue
        A = W.as_f64(w.A[p][a], w.dtype)
        B = W.as_f64(w.B[p][a], w.dtype)
        s = float(np.float32(alpha[a]) / np.float32(w.ranks[a]))
        Y[rows] += s * ((X[rows] @ A) @ B)
    return Y


def run_oracle(w, p, **kw):
    return oracle.apply(w.X[p], w.Y_base[p], kw.get("ids", w.ids), kw.get("ranks", w.ranks),
                        kw.get("alpha", w.alpha), w.tables[p], kw.get("pool", w.pool),
                        w.page_width, w.dtype)


# ------------------------------------------------------------ bf16 rounding
def test_bf16_rounding_matches_library_cast():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),           # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38,
                  1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, 1.0 + 3 * 2 ** -9],
                 np.float32)])
    # exact ties: low 16 bits == 0x8000
    ties = (rng.integers(0, 2 ** 15, 500, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    vals = np.concatenate([vals, ties[np.isfinite(ties)]])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.round_bf16(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, want)
    nan = oracle.round_bf16(float("nan"))
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


# ---------------------------------------------------------------- segments
def brute_segments(ids, ranks):
    N = len(ranks)
    valid = [t for t in range(len(ids)) if 0 <= ids[t] < N and 1 <= ranks[ids[t]] <= 128]
    order = sorted(valid, key=lambda t: ids[t])           # Python's sort is stable
    excl = [t for t in range(len(ids)) if t not in set(valid)]
    segs = []
    for t in order:
        if not segs or segs[-1][0] != ids[t]:
            segs.append([ids[t], 0])
        segs[-1][1] += 1
    return order + excl, segs, sum(1 for t in excl if ids[t] != -1)


@pytest.mark.parametrize("seed", range(6))
def test_segments_match_stable_sort(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 40))
    T = int(rng.integers(0, 300))
    ranks = rng.choice([1, 4, 8, 16, 24, 64, 128], N).astype(np.int32)
    if seed % 2:
        ranks[rng.integers(0, N)] = 0           # an adapter with an invalid rank
        ranks[rng.integers(0, N)] = 200
    ids = rng.integers(-3, N + 3, T).astype(np.int32)
    got = oracle.segments(ids, ranks)
    perm, segs, n_inv = brute_segments(list(ids), list(ranks))
    assert got["perm"].tolist() == perm
    assert got["S"] == len(segs)
    assert got["seg_adapter"].tolist() == [a for a, _ in segs]
    assert np.diff(got["seg_indptr"]).tolist() == [c for _, c in segs]
    assert np.diff(got["v_indptr"]).tolist() == [c * int(ranks[a]) for a, c in segs]
    assert got["n_invalid"] == n_inv
    assert got["T_valid"] == sum(c for _, c in segs)


def test_segments_invariant_under_token_permutation():
    w = small(2)
    seg = oracle.segments(w.ids, w.ranks)
    p = np.random.default_rng(1).permutation(w.T)
    seg2 = oracle.segments(w.ids[p], w.ranks)
    for k in ("seg_indptr", "seg_adapter", "v_indptr"):
        assert np.array_equal(seg[k], seg2[k])


# ---------------------------------------------------- page-table round trip
@pytest.mark.parametrize("k,kw", [(0, {}), (2, {}), (2, dict(ranks_override=[1, 4, 24, 40, 16, 17])),
                                  (2, dict(scatter=False, page_width=256))])
def test_page_gather_round_trip(k, kw):
    """Reading every adapter through the oracle's page arithmetic returns the
    generator's dense matrices bit for bit ([MLSP] "Unified Paging
    Architecture": weights gathered from non-contiguous physical pages)."""
    w = small(k, **kw)
    for p, tb in enumerate(w.tables):
        for a in range(w.N):
            A, B = oracle.gather_adapter(w.pool, tb, a, int(w.ranks[a]), w.page_width, w.dtype)
            assert np.array_equal(A.astype(np.float64), W.as_f64(w.A[p][a], w.dtype))
            assert np.array_equal(B.astype(np.float64), W.as_f64(w.B[p][a], w.dtype))


def test_pool_padding_is_never_read():
    """Padding holds NaN; a finite result proves no padding value was used
    ([MLSP] MBGMV: no padding to the maximum rank)."""
    w = small(2, ranks_override=[1, 4, 24, 40, 16, 8])
    assert np.isnan(W.as_f64(w.pool, w.dtype)).any()
    for p in range(w.n_projs):
        assert np.isfinite(W.as_f64(run_oracle(w, p), w.dtype)).all()


# ------------------------------------------------------------ algebra pins
def test_merge_identity_float64():
    """X(W0 + s A B) == X W0 + s (X A) B  ([MLSP] "Mathematical Anatomy":
    single-tenant pre-merge; [MLSA] "Why merging per tenant does not scale")."""
    w = small(0, page_width=64, ranks_override=[3, 8, 16, 20], alpha_override=[7.0, 16.0, 3.0, 40.0])
    rng = np.random.default_rng(11)
    X = W.as_f64(w.X[0], w.dtype)
    W0 = rng.standard_normal((256, 256)) / 16.0
    Yb = (X @ W0).astype(np.float32)
    Y = oracle.apply(w.X[0], Yb, w.ids, w.ranks, w.alpha, w.tables[0], w.pool, w.page_width, w.dtype)
    ref = np.zeros_like(X)
    for t in range(w.T):
        a = w.ids[t]
        A = W.as_f64(w.A[0][a], w.dtype)
        B = W.as_f64(w.B[0][a], w.dtype)
        s = float(np.float32(w.alpha[a]) / np.float32(w.ranks[a]))
        ref[t] = X[t] @ (W0 + s * (A @ B))
    assert rowwise_rel(Y, ref) < 1e-5


@pytest.mark.parametrize("k,kw,tol", [
    (0, {}, 1e-5),
    (2, {}, 4e-3),
    (2, dict(dtype="f32"), 1e-5),
    (2, dict(ranks_override=[1, 4, 24, 40, 17, 128]), 4e-3),
])
def test_brute_force_per_adapter(k, kw, tol):
    """Oracle == float64 per-adapter dense loop ([MLSA] "Heterogeneous
    batching": one gather-based shrink/expand per token's own adapter) within
    fp32 accumulation (1e-5) or bf16 output rounding (2^-8, plus margin)."""
    w = small(k, **kw)
    for p in range(w.n_projs):
        Y = W.as_f64(run_oracle(w, p), w.dtype)
        assert rowwise_rel(Y, dense_reference(w, p)) < tol


def test_shrink_matches_float64():
    w = small(2, dtype="f32", ranks_override=[1, 4, 24, 40, 17, 128])
    seg = oracle.segments(w.ids, w.ranks)
    for p in range(w.n_projs):
        v = oracle.shrink(w.X[p], seg, w.ranks, w.tables[p], w.pool, w.page_width, w.dtype)
        X = W.as_f64(w.X[p], w.dtype)
        for s in range(seg["S"]):
            a = seg["seg_adapter"][s]
            r = int(w.ranks[a])
            toks = seg["perm"][seg["seg_indptr"][s]:seg["seg_indptr"][s + 1]]
            ref = X[toks] @ W.as_f64(w.A[p][a], w.dtype)
            got = v[seg["v_indptr"][s]:seg["v_indptr"][s + 1]].reshape(len(toks), r)
            assert np.abs(got - ref).max() <= 1e-5 * max(np.abs(ref).max(), 1.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_B_leaves_base(dtype):
    w = small(2, dtype=dtype)
    pool = w.pool.copy()
    for tb in w.tables:
        pool[tb.b_pages] = 0
    for p in range(w.n_projs):
        Y = run_oracle(w, p, pool=pool)
        assert np.array_equal(Y, w.Y_base[p])


def test_alpha_equals_rank_is_unscaled_form():
    """alpha = r gives h = W0 x + B(A x) ([LAST] "Architecture of Multi-LoRA
    in vLLM"); the default alpha = 2r gives a different answer."""
    w = small(2, dtype="f32")
    a_eq_r = w.ranks.astype(np.float32)
    for p in range(w.n_projs):
        Y1 = run_oracle(w, p, alpha=a_eq_r)
        ref = dense_reference(w, p, alpha=a_eq_r)
        assert rowwise_rel(Y1, ref) < 1e-5
        Y2 = run_oracle(w, p)
        assert rowwise_rel(Y2, ref) > 1e-2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_token_permutation_permutes_rows_exactly(dtype):
    w = small(2, dtype=dtype)
    perm = np.random.default_rng(3).permutation(w.T)
    for p in range(w.n_projs):
        Y = run_oracle(w, p)
        Yp = oracle.apply(w.X[p][perm], w.Y_base[p][perm], w.ids[perm], w.ranks, w.alpha,
                          w.tables[p], w.pool, w.page_width, w.dtype)
        assert np.array_equal(Yp, Y[perm])


def test_one_hot_closed_form_exact():
    """A[:, k] = e_pi(k), B[k, :] = e_sigma(k): every sum has one non-zero
    term, so Y[t, sigma(k)] = Y_base + s*X[t, pi(k)] with one rounding."""
    w = small(0, dtype="f32", ranks_override=[8, 8, 5, 16])
    rng = np.random.default_rng(5)
    pool = w.pool.copy()
    tb = w.tables[0]
    pis, sigmas = {}, {}
    for a in range(w.N):
        r = int(w.ranks[a])
        pi = rng.permutation(256)[:r]
        sg = rng.permutation(256)[:r]
        A = np.zeros((256, r), np.float32)
        B = np.zeros((r, 256), np.float32)
        A[pi, np.arange(r)] = 1.0
        B[np.arange(r), sg] = 1.0
        pool[tb.a_pages[tb.a_indptr[a]:tb.a_indptr[a + 1]]] = W.pack_a_pages(A, w.page_width, np.nan)
        pool[tb.b_pages[tb.b_indptr[a]:tb.b_indptr[a + 1]]] = W.pack_b_pages(B, w.page_width, np.nan)
        pis[a], sigmas[a] = pi, sg
    Y = run_oracle(w, 0, pool=pool)
    want = w.Y_base[0].copy()
    for t in range(w.T):
        a = w.ids[t]
        s = np.float32(w.alpha[a]) / np.float32(w.ranks[a])
        want[t, sigmas[a]] = w.Y_base[0][t, sigmas[a]] + s * w.X[0][t, pis[a]]
    assert np.array_equal(Y, want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_isolation_other_rows_bit_identical(dtype):
    """Perturbing one adapter's pages changes only that adapter's tokens
    ([MLSA] "Trade-offs, Gotchas": each token sees only its own adapter; an
    indexing slip is a cross-tenant leak)."""
    w = small(2, dtype=dtype)
    b = int(np.bincount(w.ids).argmax())
    pool = w.pool.copy()
    for tb in w.tables:
        pages = np.concatenate([tb.a_pages[tb.a_indptr[b]:tb.a_indptr[b + 1]],
                                tb.b_pages[tb.b_indptr[b]:tb.b_indptr[b + 1]]])
        if dtype == "bf16":
            pool[pages] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(pool[pages]) * np.float32(1.5))
        else:
            pool[pages] *= np.float32(1.5)
    for p in range(w.n_projs):
        Y0, Y1 = run_oracle(w, p), run_oracle(w, p, pool=pool)
        other = w.ids != b
        assert np.array_equal(Y0[other], Y1[other])
        assert not np.array_equal(Y0[~other], Y1[~other])


def test_base_only_and_invalid_tokens_keep_base():
    w = small(2)
    ids = w.ids.copy()
    ids[[0, 3]] = -1
    ids[5] = w.N + 4
    ids[7] = -9
    seg = oracle.segments(ids, w.ranks)
    assert seg["n_invalid"] == 2 and seg["T_valid"] == w.T - 4
    for p in range(w.n_projs):
        Y = run_oracle(w, p, ids=ids)
        for t in (0, 3, 5, 7):
            assert np.array_equal(Y[t], w.Y_base[p][t])
        assert rowwise_rel(W.as_f64(Y, w.dtype), dense_reference(w, p, ids=ids)) < 4e-3


def test_single_adapter_is_dense_chain():
    w = small(2, dtype="f32", ids_override=np.full(24, 2, np.int32))
    for p in range(w.n_projs):
        X = W.as_f64(w.X[p], w.dtype)
        s = float(np.float32(w.alpha[2]) / np.float32(w.ranks[2]))
        ref = W.as_f64(w.Y_base[p], w.dtype) + s * (X @ W.as_f64(w.A[p][2], w.dtype)) @ W.as_f64(w.B[p][2], w.dtype)
        assert rowwise_rel(run_oracle(w, p), ref) < 1e-5


def test_out_of_pool_page_is_reported():
    w = small(2)
    tb = w.tables[0]
    bad = W.ProjTables(tb.name, tb.d_in, tb.d_out, tb.a_indptr, tb.a_pages.copy(), tb.b_indptr, tb.b_pages)
    bad.a_pages[tb.a_indptr[w.ids[0]]] = w.num_pages + 3
    with pytest.raises(ValueError):
        oracle.apply(w.X[0], w.Y_base[0], w.ids, w.ranks, w.alpha, bad, w.pool, w.page_width, w.dtype)


def test_thread_count_does_not_change_results():
    w = small(2)
    for p in range(w.n_projs):
        Y1 = oracle.apply(w.X[p], w.Y_base[p], w.ids, w.ranks, w.alpha, w.tables[p], w.pool,
                          w.page_width, w.dtype, nthreads=1)
        Y4 = oracle.apply(w.X[p], w.Y_base[p], w.ids, w.ranks, w.alpha, w.tables[p], w.pool,
                          w.page_width, w.dtype, nthreads=4)
        assert np.array_equal(Y1, Y4)


def test_zero_padding_to_max_rank_changes_nothing():
    """A fixed-rank slot layout (every adapter zero-padded to r_max, alpha
    scaled by r_max / r) computes the same branch: the padded terms are
    exact zeros and alpha'/r_max equals alpha/r bit for bit (division by a
    power of two), so the oracle's Y is identical."""
    w = W.make_workload(2, dict(T=90, N=6, ranks_override=[8, 16, 5, 64, 24, 1], page_width=256,
                                projs=(("a", 512, 768),), dtype="f32"))
    wp = W.pad_to_rank(w, 64)
    assert (wp.ranks == 64).all()
    y = oracle.apply(w.X[0], w.Y_base[0], w.ids, w.ranks, w.alpha, w.tables[0], w.pool, w.page_width, w.dtype)
    yp = oracle.apply(wp.X[0], wp.Y_base[0], wp.ids, wp.ranks, wp.alpha, wp.tables[0], wp.pool, wp.page_width,
                      wp.dtype)
    assert np.array_equal(y, yp)
    # and the padded pool really holds more pages (what the layout costs)
    assert wp.num_pages > w.num_pages
