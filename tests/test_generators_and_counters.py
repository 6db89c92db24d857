"""Pins of the input generator and the algorithmic byte counter against the
numbers the pages print (fixtures under tests/golden/, each citing its page).

The printed LRU hit rates that the bounded-Zipf draws must reproduce are
pinned through the native page cache in test_pool_manager.py.
"""
import os

import numpy as np
import pytest

import workloads as W
from heterogeneous_adapters_amd import traffic

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_zipf_ids_properties():
    ids = W.zipf_ids(20000, 50, 1.1, 3)
    assert ids.min() >= 0 and ids.max() < 50
    counts = np.bincount(ids, minlength=50)
    # popularity decreases with id (law 1/i^s): id 0 is the hottest and the
    # ratio of the first two is near 2^1.1
    assert counts.argmax() == 0
    assert abs(counts[0] / counts[1] - 2 ** 1.1) < 0.15
    assert np.array_equal(ids, W.zipf_ids(20000, 50, 1.1, 3))


MEM = {k: v for k, v in _read("mlsa_memory_arithmetic.txt")}
LLAMA3_8B = [(4096, 4096), (4096, 1024), (4096, 1024), (4096, 4096), (4096, 14336),
             (4096, 14336), (14336, 4096)]


def _approx(key, value):
    txt = MEM[key]
    assert txt.startswith("~")
    want = float(txt[1:])
    digits = len(txt[1:].split("e")[0].replace(".", ""))
    assert float(f"{value:.{digits}g}") == pytest.approx(want, rel=1e-12), (key, value, want)


def test_memory_arithmetic_matches_page():
    assert traffic.adapter_params(1, LLAMA3_8B) == int(MEM["params_per_unit_rank_per_layer"])
    assert traffic.adapter_params(16, LLAMA3_8B) == int(MEM["params_per_layer_r16"])
    _approx("params_total_r16", 32 * traffic.adapter_params(16, LLAMA3_8B))
    _approx("bytes_total_r16", 2 * 32 * traffic.adapter_params(16, LLAMA3_8B))
    _approx("bytes_total_r64", 2 * 32 * traffic.adapter_params(64, LLAMA3_8B))
    _approx("params_attention_only_r16", 32 * traffic.adapter_params(16, LLAMA3_8B[:4]))
    _approx("bytes_attention_only_r16", 2 * 32 * traffic.adapter_params(16, LLAMA3_8B[:4]))
    _approx("bytes_100_adapters_r16", 100 * 2 * 32 * traffic.adapter_params(16, LLAMA3_8B))
    _approx("bytes_32_slots_r64", 32 * 2 * 32 * traffic.adapter_params(64, LLAMA3_8B))
    _approx("bytes_32_slots_r8", 32 * 2 * 32 * traffic.adapter_params(8, LLAMA3_8B))


def test_algorithmic_bytes_counts_distinct_adapters_once():
    ranks = np.array([8, 16, 64, 32], np.int32)
    # 64 tokens on one adapter read that adapter once; 4 distinct read 4 sets
    one = traffic.split_bytes(np.zeros(64, np.int32), ranks, 4096, 4096, 2)
    many = traffic.split_bytes(np.arange(64, dtype=np.int32) % 4, ranks, 4096, 4096, 2)
    act = 64 * 4096 * 2
    assert one[0] == act + 8 * 4096 * 2 and one[1] == 2 * act + 8 * 4096 * 2
    assert many[0] == act + 120 * 4096 * 2 and many[1] == 2 * act + 120 * 4096 * 2
    # invalid and base-only tokens move no adapter weights and no activations
    ids = np.array([-1, 7, 2, 2], np.int32)
    s, e, m = traffic.split_bytes(ids, ranks, 256, 512, 2)
    assert s == (2 * 256 + 64 * 256) * 2 and e == (2 * 2 * 512 + 64 * 512) * 2
    assert traffic.algorithmic_flops(ids, ranks, 256, 512) == 2 * 2 * 64 * 768


def test_page_tables_cover_pool_once():
    ranks = np.array([8, 16, 24, 64, 1], np.int32)
    shapes = [("a", 300, 700), ("b", 1000, 64)]
    for scatter in (False, True):
        tabs, npg = W.plan_tables(ranks, shapes, 128, scatter, 5)
        allp = np.concatenate([np.concatenate([t.a_pages, t.b_pages]) for t in tabs])
        assert np.array_equal(np.sort(allp), np.arange(npg))
        for t in tabs:
            G = (ranks + 15) // 16
            assert np.array_equal(np.diff(t.a_indptr), G * ((t.d_in + 127) // 128))
            assert np.array_equal(np.diff(t.b_indptr), G * ((t.d_out + 127) // 128))


def test_mixed_batch_ids_structure():
    """Continuous-batching ids: each prefill chunk is one contiguous run of a
    single adapter with its drawn length; the decode tail is bounded-Zipf and
    reproducible from the seed."""
    ids, ranks, alpha, lens = W.draw_ids_and_ranks(5)
    c = W.CONFIGS[5]
    assert len(lens) == c["nchunks"] and all(c["chunk_lo"] <= L <= c["chunk_hi"] for L in lens)
    assert len(ids) == int(sum(lens)) + c["ndecode"]
    pos = 0
    for L in lens:
        run = ids[pos:pos + L]
        assert (run == run[0]).all() and 0 <= run[0] < c["N"]
        pos += L
    tail = ids[pos:]
    assert tail.min() >= 0 and tail.max() < c["N"]
    # the most popular decode adapter is id 0 (bounded Zipf, s = 1.2)
    counts = np.bincount(tail, minlength=c["N"])
    assert counts.argmax() == 0
    ids2, _, _, _ = W.draw_ids_and_ranks(5)
    assert np.array_equal(ids, ids2)


def test_group_bytes_count_a_shared_activation_once():
    """q/k/v of one call reading one X: the group's shrink bytes hold X once,
    everything else (weights, outputs) per projection."""
    ids = np.array([0, 1, 1, 2, -1, 0], np.int32)
    ranks = np.array([8, 16, 64], np.int32)
    per = [traffic.split_bytes(ids, ranks, 4096, d_out, 2) for d_out in (4096, 1024, 1024)]
    shared = traffic.group_split_bytes(ids, ranks, [(4096, 4096, "x"), (4096, 1024, "x"), (4096, 1024, "x")], 2)
    separate = traffic.group_split_bytes(ids, ranks, [(4096, 4096, "a"), (4096, 1024, "b"), (4096, 1024, "c")], 2)
    t_valid = 5
    assert separate == tuple(map(sum, zip(*per)))
    assert shared[0] == separate[0] - 2 * t_valid * 4096 * 2
    assert shared[1:] == separate[1:]
