"""Algorithmic bytes and flops of the adapter branch (what the method must
move and compute; the denominator-free numerator of every GB/s and TFLOP/s
figure this project reports).

Sources:
  [MLSA] "Multi-LoRA Serving Architecture: Serving Hundreds of Fine-Tuned
         Adapters on One GPU with vLLM and S-LoRA (2026)", sections
         "The memory arithmetic that makes it work" (an adapter on a
         projection holds r*(d_in + d_out) parameters) and "Heterogeneous
         batching: the core compute trick" (a batch reads each distinct
         adapter's weights once; cost grows with distinct adapters and rank,
         not with batch size alone).
  [LAST] "LoRA Adapters at Serve Time with vLLM Multi-LoRA", section "The
         Inference Mechanism: A Worked Scenario", step 4 (adapter weights are
         read once for A and once for B).

Per projection call, with e bytes per activation/weight element:
  bytes = T_valid*(d_in + 2*d_out)*e                  X read, Y_base read, Y write
        + sum_{a in distinct adapters} r_a*(d_in + d_out)*e   A and B, unpadded
        + 4*(T + 2*S + 3)                              token/segment metadata
  flops = sum_{valid t} 2*r_{a(t)}*(d_in + d_out)
Unused page rows/columns and any split-K partial round trip are excluded.
Projections of one call that read the same activations (q/k/v, gate/up of a
transformer block) need X once: ``group_split_bytes`` counts it once.
"""
from __future__ import annotations

from typing import Iterable, Sequence, Tuple

import numpy as np

MAX_RANK = 128


def adapter_params(r: int, shapes: Iterable[Tuple[int, int]]) -> int:
    """Parameters of a rank-r adapter over projections (d_in, d_out)."""
    return int(r) * sum(int(di) + int(do) for di, do in shapes)


def _valid(ids: np.ndarray, ranks: np.ndarray) -> np.ndarray:
    ids = np.asarray(ids)
    N = len(ranks)
    ok = (ids >= 0) & (ids < N)
    r = np.where(ok, np.asarray(ranks)[np.clip(ids, 0, max(N - 1, 0))], 0)
    return ok & (r >= 1) & (r <= MAX_RANK)


def distinct_adapters(ids: np.ndarray, ranks: np.ndarray) -> np.ndarray:
    ids = np.asarray(ids)
    return np.unique(ids[_valid(ids, ranks)])


def split_bytes(ids, ranks, d_in: int, d_out: int, elem_bytes: int) -> Tuple[int, int, int]:
    """(shrink bytes, expand bytes, metadata bytes) of one projection call."""
    ids = np.asarray(ids)
    ranks = np.asarray(ranks, np.int64)
    v = _valid(ids, ranks)
    t_valid = int(v.sum())
    dist = distinct_adapters(ids, ranks)
    rsum = int(ranks[dist].sum()) if len(dist) else 0
    shrink = (t_valid * d_in + rsum * d_in) * elem_bytes
    expand = (2 * t_valid * d_out + rsum * d_out) * elem_bytes
    meta = 4 * (len(ids) + 2 * len(dist) + 3)
    return shrink, expand, meta


def algorithmic_bytes(ids, ranks, d_in: int, d_out: int, elem_bytes: int) -> int:
    return sum(split_bytes(ids, ranks, d_in, d_out, elem_bytes))


def algorithmic_flops(ids, ranks, d_in: int, d_out: int) -> int:
    ids = np.asarray(ids)
    ranks = np.asarray(ranks, np.int64)
    v = _valid(ids, ranks)
    return int(2 * ranks[ids[v]].sum() * (d_in + d_out))


def step_totals(ids, ranks, shapes: Sequence[Tuple[int, int]], elem_bytes: int):
    """Summed (bytes, flops, shrink_bytes, expand_bytes) over projections."""
    tb = tf = ts = te = 0
    for di, do in shapes:
        s, e, m = split_bytes(ids, ranks, di, do, elem_bytes)
        tb += s + e + m
        ts += s
        te += e
        tf += algorithmic_flops(ids, ranks, di, do)
    return tb, tf, ts, te


def group_split_bytes(ids, ranks, projs, elem_bytes: int) -> Tuple[int, int, int]:
    """(shrink, expand, metadata) bytes of one call over several projections.
    projs: sequence of (d_in, d_out, x_key); projections with the same x_key
    read one activation matrix, counted once."""
    ids = np.asarray(ids)
    t_valid = int(_valid(ids, np.asarray(ranks, np.int64)).sum())
    shrink = expand = meta = 0
    seen = set()
    for d_in, d_out, key in projs:
        s, e, m = split_bytes(ids, ranks, d_in, d_out, elem_bytes)
        if key in seen:
            s -= t_valid * d_in * elem_bytes
        seen.add(key)
        shrink += s
        expand += e
        meta += m
    return shrink, expand, meta
