"""CPU oracle for the multi-LoRA adapter branch -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain C in
``oracle.c``, fp32 sequential accumulation, OpenMP over tokens) with ctypes and
shares no code with the HIP library.  See ``oracle.c`` for the page citations
and the definition it evaluates.

Parity pins: every function here is checked by the ``-m "not gpu"`` tests
against float64 algebra (merge identity, brute-force per-adapter loops, one-hot
closed forms, B = 0, alpha = r, permutation and isolation invariants) and
against the page-table round trip of the generator.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

from . import build as _build

LIB_PATH = _build.LIB_PATH

DT_F32, DT_BF16 = 0, 1
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_vp = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_segments.argtypes = [_vp, ctypes.c_int32, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp]
        L.oracle_segments.restype = ctypes.c_int
        L.oracle_apply.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                   _vp, ctypes.c_int64, _vp, ctypes.c_int64, _vp, ctypes.c_int64,
                                   _vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        L.oracle_apply.restype = ctypes.c_int
        L.oracle_shrink.argtypes = [ctypes.c_int32, ctypes.c_int, _vp, ctypes.c_int64, _vp, _vp, _vp,
                                    _vp, ctypes.c_int32, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                    ctypes.c_int32, _vp, ctypes.c_int32]
        L.oracle_shrink.restype = ctypes.c_int
        L.oracle_gather_adapter.argtypes = [_vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _vp, _vp,
                                            _vp, _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, _vp, _vp]
        L.oracle_gather_adapter.restype = ctypes.c_int
        L.oracle_round_bf16.argtypes = [ctypes.c_float]
        L.oracle_round_bf16.restype = ctypes.c_uint16
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _dt(dtype: str) -> int:
    return DT_BF16 if dtype == "bf16" else DT_F32


def _store_t(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def round_bf16(x: float) -> int:
    return int(lib().oracle_round_bf16(ctypes.c_float(x)))


def segments(ids: np.ndarray, rank: np.ndarray) -> dict:
    ids = _c(ids, np.int32)
    rank = _c(rank, np.int32)
    T, N = len(ids), len(rank)
    smax = min(T, N)
    perm = np.zeros(max(T, 1), np.int32)
    seg_indptr = np.zeros(smax + 1, np.int32)
    seg_adapter = np.zeros(max(smax, 1), np.int32)
    v_indptr = np.zeros(smax + 1, np.int32)
    counts = np.zeros(4, np.int32)
    rc = lib().oracle_segments(_p(ids), T, _p(rank), N, _p(perm), _p(seg_indptr), _p(seg_adapter),
                               _p(v_indptr), _p(counts))
    if rc != 0:
        raise ValueError(f"oracle_segments failed: {rc}")
    S = int(counts[0])
    return dict(perm=perm[:T], seg_indptr=seg_indptr[:S + 1], seg_adapter=seg_adapter[:S],
                v_indptr=v_indptr[:S + 1], S=S, n_invalid=int(counts[1]), T_valid=int(counts[2]),
                V_total=int(counts[3]))


def apply(X, Y_base, ids, rank, alpha, tables, pool, page_width: int, dtype: str,
          nthreads: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Y for one projection; ``tables`` has a_indptr, a_pages, b_indptr, b_pages,
    d_in, d_out.  X, Y_base, pool are fp32 values or bf16 bit patterns."""
    st = _store_t(dtype)
    X = _c(X, st)
    Y_base = _c(Y_base, st)
    T = X.shape[0]
    d_in, d_out = int(tables.d_in), int(tables.d_out)
    assert X.shape[1] >= d_in and Y_base.shape == (T, Y_base.shape[1]) and Y_base.shape[1] >= d_out
    Y = np.empty((T, d_out), st) if out is None else out
    ids = _c(ids, np.int32)
    rank = _c(rank, np.int32)
    alpha = _c(alpha, np.float32)
    tb = [_c(getattr(tables, k), np.int32) for k in ("a_indptr", "a_pages", "b_indptr", "b_pages")]
    pool = _c(pool, st)
    rc = lib().oracle_apply(T, d_in, d_out, _dt(dtype), _p(X), X.shape[1], _p(Y_base),
                            Y_base.shape[1], _p(Y), Y.shape[1], _p(ids), len(rank), _p(rank),
                            _p(alpha), _p(tb[0]), _p(tb[1]), _p(tb[2]), _p(tb[3]), _p(pool),
                            pool.shape[0], page_width, nthreads)
    if rc != 0:
        raise ValueError(f"oracle_apply failed: {rc}")
    return Y


def shrink(X, seg: dict, rank, tables, pool, page_width: int, dtype: str,
           nthreads: int = 0) -> np.ndarray:
    """Ragged v in grouped order (v[v_indptr[s] + i*r + k])."""
    st = _store_t(dtype)
    X = _c(X, st)
    rank = _c(rank, np.int32)
    pool = _c(pool, st)
    a_ip, a_pg = _c(tables.a_indptr, np.int32), _c(tables.a_pages, np.int32)
    v = np.zeros(max(seg["V_total"], 1), np.float32)
    arrs = [_c(seg[k], np.int32) for k in ("perm", "seg_indptr", "seg_adapter", "v_indptr")]
    rc = lib().oracle_shrink(int(tables.d_in), _dt(dtype), _p(X), X.shape[1], _p(arrs[0]),
                             _p(arrs[1]), _p(arrs[2]), _p(arrs[3]), seg["S"], _p(rank), _p(a_ip),
                             _p(a_pg), _p(pool), pool.shape[0], page_width, _p(v), nthreads)
    if rc != 0:
        raise ValueError(f"oracle_shrink failed: {rc}")
    return v[:seg["V_total"]]


def gather_adapter(pool, tables, a: int, r: int, page_width: int,
                   dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """Dense (A: d_in x r, B: r x d_out) of adapter ``a`` read through the tables."""
    st = _store_t(dtype)
    pool = _c(pool, st)
    d_in, d_out = int(tables.d_in), int(tables.d_out)
    A = np.zeros((d_in, r), np.float32)
    B = np.zeros((r, d_out), np.float32)
    tb = [_c(getattr(tables, k), np.int32) for k in ("a_indptr", "a_pages", "b_indptr", "b_pages")]
    rc = lib().oracle_gather_adapter(_p(pool), _dt(dtype), pool.shape[0], page_width, _p(tb[0]),
                                     _p(tb[1]), _p(tb[2]), _p(tb[3]), d_in, d_out, a, r, _p(A), _p(B))
    if rc != 0:
        raise ValueError(f"oracle_gather_adapter failed: {rc}")
    return A, B
