"""lora_apply_noalloc (the library's fixed device array as workspace) against
lora_apply (a caller workspace) through the C ABI: two calls in a row, the
second on a smaller batch, so the second runs on an array that still holds
the first call's contents.  Same kernels on the same inputs: Y and the
segments must be bit-identical, and Y must match the oracle within the
bf16 tolerance."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from heterogeneous_adapters_amd import batch, lora

pytestmark = pytest.mark.gpu


def _rowwise(Y, Yref):
    Y, Yref = np.asarray(Y, np.float64), np.asarray(Yref, np.float64)
    den = np.maximum(np.abs(Yref).max(axis=1), 1e-30)
    return float((np.abs(Y - Yref).max(axis=1) / den).max())


def _run(w, noalloc, prebuilt):
    b = batch.to_device(w)
    projs = [b.proj(p) for p in range(w.n_projs)]
    segs = lora.Segments(w.T, w.N)
    max_din = max(t.d_in for t in w.tables)
    if prebuilt:
        lora.lora_build_segments(b.ids, b.adapters, segs, lora.workspace(w.T, w.N, 0, 0))
        ids, sg = None, segs
    else:
        ids, sg = b.ids, segs
    if noalloc:
        lora.lora_apply_noalloc(ids, sg, w.T, projs, b.adapters, b.pool)
    else:
        ws = lora.workspace(w.T, w.N, w.n_projs, max_din)
        lora.lora_apply(ids, sg, w.T, projs, b.adapters, b.pool, ws)
    torch.cuda.synchronize()
    return [batch.device_to_host(b.Y[p]) for p in range(w.n_projs)], segs.arrays()


def _workloads():
    big = W.make_workload(2, dict(T=600, N=40, projs=(("up", 1024, 2048), ("down", 2048, 1024)),
                                  page_width=512), keep_dense=False)
    small = W.make_workload(2, dict(T=70, N=9, projs=(("q", 512, 768),), page_width=512, seed=21),
                            keep_dense=False)
    return big, small


@pytest.mark.parametrize("prebuilt", [False, True])
def test_noalloc_matches_apply_on_two_calls(prebuilt):
    torch.cuda.set_device(0)
    for w in _workloads():
        print(f"noalloc case T={w.T} N={w.N} projs={w.n_projs} prebuilt={prebuilt}", flush=True)
        ref, ref_seg = _run(w, noalloc=False, prebuilt=prebuilt)
        got, got_seg = _run(w, noalloc=True, prebuilt=prebuilt)
        for k in ("perm", "seg_indptr", "seg_adapter", "v_indptr"):
            assert np.array_equal(got_seg[k], ref_seg[k]), k
        assert got_seg["flags"] == 0 and ref_seg["flags"] == 0
        for p in range(w.n_projs):
            assert np.array_equal(got[p], ref[p]), (w.T, p)
            want = oracle.apply(w.X[p], w.Y_base[p], w.ids, w.ranks, w.alpha, w.tables[p], w.pool,
                                w.page_width, w.dtype)
            assert _rowwise(W.as_f64(got[p], w.dtype), W.as_f64(want, w.dtype)) < 1e-2


def test_noalloc_rejects_a_batch_beyond_its_array():
    """A prefill batch whose workspace exceeds the array is refused with
    LORA_ERR_WORKSPACE before any device work."""
    w = W.make_workload(2, dict(T=2500, N=8, projs=(("w1", 16384, 256), ("w2", 16384, 256)), page_width=512),
                        keep_dense=False)
    need = lora.lora_workspace_size(w.T, w.N, 2, 16384)
    assert need > lora.LORA_NOALLOC_SCRATCH_BYTES
    b = batch.to_device(w)
    for y in b.Y:
        y.fill_(5.0)
    with pytest.raises(lora.LoraError) as e:
        lora.lora_apply_noalloc(b.ids, None, w.T, [b.proj(0), b.proj(1)], b.adapters, b.pool)
    assert e.value.status == -4
    torch.cuda.synchronize()
    for y in b.Y:
        assert bool((y.float() == 5.0).all())
