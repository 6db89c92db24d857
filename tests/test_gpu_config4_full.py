"""Full-size parity for the Llama-2-7B-shaped decode step (32 layers x 7
projections, 1024 tokens, 1000 adapters in a ~160 GiB paged pool), run in the
launch configuration the benchmark times (segments built once, then q/k/v,
o, gate/up and down per layer).  Segments are compared in full; Y on sampled
tokens of all 224 projections, each computed by the oracle token by token
from the pages those tokens use, and on every token of one whole layer."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from heterogeneous_adapters_amd import lora
from workloads.device import host_subset, make_device_workload, tensor_bits

pytestmark = pytest.mark.gpu


def test_config4_full_size_sampled_parity():
    print("config 4: generating the device workload", flush=True)
    dw = make_device_workload(4, "cuda")
    T, N = dw.T, dw.N
    dev = "cuda"
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    ids = i32(dw.ids)
    adapters = lora.Adapters(i32(dw.ranks), torch.from_numpy(dw.alpha).to(dev))
    pool = lora.Pool(dw.pool, dw.page_width)
    tabs = [(i32(t.a_indptr), i32(t.a_pages), i32(t.b_indptr), i32(t.b_pages)) for t in dw.tables]
    Y = [torch.empty_like(y) for y in dw.Y_base]
    projs = [lora.Proj(dw.X[p], dw.Y_base[p], Y[p], *tabs[p]) for p in range(dw.n_projs)]
    segs = lora.Segments(T, N)
    lora.lora_build_segments(ids, adapters, segs, lora.workspace(T, N, 0, 0))
    ws = lora.workspace(T, N, 3, 11008)
    print("config 4: running one decode step", flush=True)
    for l in range(32):
        for grp in ((0, 1, 2), (3,), (4, 5), (6,)):
            lora.lora_apply(None, segs, T, [projs[7 * l + i] for i in grp], adapters, pool, ws)
    torch.cuda.synchronize()
    got_seg = segs.arrays()
    want_seg = oracle.segments(dw.ids, dw.ranks)
    for k in ("perm", "seg_indptr", "seg_adapter", "v_indptr"):
        assert np.array_equal(got_seg[k], want_seg[k]), k
    assert got_seg["S"] == want_seg["S"] and got_seg["flags"] == 0

    rng = np.random.default_rng(0)
    hot = np.nonzero(dw.ids == np.bincount(dw.ids).argmax())[0]
    counts = np.bincount(dw.ids, minlength=N)
    single = np.nonzero(counts[dw.ids] == 1)[0]
    sample = np.unique(np.concatenate([rng.choice(T, 24, replace=False), hot[:12], single[:12]]))
    sub_ids = dw.ids[sample]
    worst = 0.0
    for l in range(32):
        idx = list(range(7 * l, 7 * l + 7))
        hp, ht = host_subset(dw.pool, [dw.tables[p] for p in idx], np.unique(sub_ids))
        for j, p in enumerate(idx):
            Xs = tensor_bits(dw.X[p])[sample]
            Ybs = tensor_bits(dw.Y_base[p])[sample]
            ref = W.as_f64(oracle.apply(Xs, Ybs, sub_ids, dw.ranks, dw.alpha, ht[j], hp, dw.page_width, "bf16"),
                           "bf16")
            got = W.as_f64(tensor_bits(Y[p])[sample], "bf16")
            assert np.isfinite(got).all(), p
            err = float((np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)).max())
            worst = max(worst, err)
            assert err < 1e-2, (p, err)
        print(f"config 4: layer {l}: 7 projections on {len(sample)} sampled tokens, worst so far {worst:.3e}",
              flush=True)
    # every token of one whole layer (the oracle on all 1024 rows)
    l = 17
    idx = list(range(7 * l, 7 * l + 7))
    valid = dw.ids[(dw.ids >= 0) & (dw.ids < N)]
    hp, ht = host_subset(dw.pool, [dw.tables[p] for p in idx], np.unique(valid))
    for j, p in enumerate(idx):
        ref = W.as_f64(oracle.apply(tensor_bits(dw.X[p]), tensor_bits(dw.Y_base[p]), dw.ids, dw.ranks, dw.alpha,
                                    ht[j], hp, dw.page_width, "bf16"), "bf16")
        got = W.as_f64(tensor_bits(Y[p]), "bf16")
        assert np.isfinite(got).all(), p
        err = float((np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)).max())
        print(f"config 4: layer {l} projection {j}: all {T} tokens, rowwise rel err {err:.3e}", flush=True)
        assert err < 1e-2, (p, err)
    del projs, Y, pool, dw, tabs
    gc.collect()
    torch.cuda.empty_cache()
