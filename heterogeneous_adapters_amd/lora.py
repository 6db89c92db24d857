"""Python binding of liblora.so: argument marshalling only.

Every step of the adapter branch runs in the library's HIP kernels; this
module turns torch tensors into the C structs of ``include/lora.h`` (device
pointers, sizes, the current HIP stream) and raises on a non-zero status.
PyTorch provides device memory and streams, nothing else.  The library is
loaded on first use and an import error is raised if it has not been built --
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

from .build import LIB_PATH

LORA_DTYPE_F32, LORA_DTYPE_BF16 = 0, 1
LORA_MAX_RANK = 128
LORA_MAX_ADAPTERS = 1 << 20
LORA_MAX_TOKENS = (1 << 24) - 1
LORA_MAX_LAUNCH_ITEMS = 1 << 30
LORA_KSLICE = 512
COUNT_S, COUNT_INVALID, COUNT_T_VALID, COUNT_V_TOTAL, COUNT_FLAGS, COUNT_T = 0, 1, 2, 3, 8, 9
FLAG_PAGE_RANGE, FLAG_SEGMENTS, FLAG_SYNC = 1, 2, 4
N_COUNTS = 16

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class lora_adapters_t(ctypes.Structure):
    _fields_ = [("rank", _vp), ("alpha", _vp), ("num_adapters", _i32)]


class lora_pool_t(ctypes.Structure):
    _fields_ = [("base", _vp), ("num_pages", _i32), ("page_width", _i32), ("dtype", _i32)]


class lora_proj_t(ctypes.Structure):
    _fields_ = [("X", _vp), ("ldx", _i64), ("Y_base", _vp), ("ldyb", _i64), ("Y", _vp), ("ldy", _i64),
                ("d_in", _i32), ("d_out", _i32), ("a_indptr", _vp), ("a_pages", _vp),
                ("b_indptr", _vp), ("b_pages", _vp)]


class lora_segments_t(ctypes.Structure):
    _fields_ = [("T", _i32), ("num_adapters", _i32), ("perm", _vp), ("seg_indptr", _vp),
                ("seg_adapter", _vp), ("v_indptr", _vp), ("plan", _vp), ("counts", _vp)]


_lib = None
EXPORTS = ("lora_status_string", "lora_v_slices", "lora_segments_size", "lora_segments_init",
           "lora_workspace_size", "lora_build_segments", "lora_shrink", "lora_expand", "lora_apply",
           "lora_validate_tables", "lora_cache_create", "lora_cache_destroy", "lora_cache_free_pages",
           "lora_cache_num_resident", "lora_cache_admit", "lora_cache_set_pinned", "lora_cache_release",
           "lora_cache_lookup", "lora_upload_pages", "lora_apply_noalloc", "lora_set_wait_limit",
           "lora_set_launch_mode")
LORA_LAUNCH_AUTO, LORA_LAUNCH_SINGLE, LORA_LAUNCH_TWO = 0, 1, 2
LORA_NOALLOC_SCRATCH_BYTES = 64 << 20


class LoraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {lib().lora_status_string(status).decode()} ({status})")
        self.status = status


def lib():
    """Load liblora.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"liblora.so is not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.lora_status_string.argtypes = [_i32]
        L.lora_status_string.restype = ctypes.c_char_p
        L.lora_v_slices.argtypes = [_i32]
        L.lora_v_slices.restype = _i32
        L.lora_segments_size.argtypes = [_i32, _i32]
        L.lora_segments_size.restype = ctypes.c_size_t
        L.lora_segments_init.argtypes = [_vp, ctypes.c_size_t, _i32, _i32, P(lora_segments_t)]
        L.lora_workspace_size.argtypes = [_i32, _i32, _i32, _i32]
        L.lora_workspace_size.restype = ctypes.c_size_t
        L.lora_build_segments.argtypes = [_vp, _i32, P(lora_adapters_t), P(lora_segments_t), _vp,
                                          ctypes.c_size_t, _vp]
        L.lora_shrink.argtypes = [P(lora_proj_t), _i32, P(lora_adapters_t), P(lora_segments_t),
                                  P(lora_pool_t), P(_vp), _i64, _vp]
        L.lora_expand.argtypes = [P(lora_proj_t), _i32, P(lora_adapters_t), P(lora_segments_t),
                                  P(lora_pool_t), P(_vp), _i32, _i64, _vp]
        L.lora_apply.argtypes = [_vp, P(lora_segments_t), _i32, P(lora_proj_t), _i32, P(lora_adapters_t),
                                 P(lora_pool_t), _vp, ctypes.c_size_t, _vp]
        L.lora_apply_noalloc.argtypes = [_vp, P(lora_segments_t), _i32, P(lora_proj_t), _i32,
                                         P(lora_adapters_t), P(lora_pool_t), _vp]
        L.lora_validate_tables.argtypes = [_i32, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]
        L.lora_set_wait_limit.argtypes = [_i64]
        L.lora_set_wait_limit.restype = None
        L.lora_set_launch_mode.argtypes = [_i32]
        L.lora_set_launch_mode.restype = _i32
        L.lora_cache_create.argtypes = [_i32, P(_vp)]
        L.lora_cache_destroy.argtypes = [_vp]
        L.lora_cache_destroy.restype = None
        L.lora_cache_free_pages.argtypes = [_vp]
        L.lora_cache_free_pages.restype = _i32
        L.lora_cache_num_resident.argtypes = [_vp]
        L.lora_cache_num_resident.restype = _i32
        L.lora_cache_admit.argtypes = [_vp, _i64, _i32, _vp, P(_i32), _vp, _i32, P(_i32)]
        L.lora_cache_set_pinned.argtypes = [_vp, _i64, _i32]
        L.lora_cache_release.argtypes = [_vp, _i64]
        L.lora_cache_lookup.argtypes = [_vp, _i64, _vp, _i32, P(_i32)]
        L.lora_upload_pages.argtypes = [P(lora_pool_t), _vp, _vp, _i32, _vp]
        for name in ("lora_segments_init", "lora_build_segments", "lora_shrink", "lora_expand",
                     "lora_apply", "lora_apply_noalloc", "lora_validate_tables", "lora_cache_create", "lora_cache_admit",
                     "lora_cache_set_pinned", "lora_cache_release", "lora_cache_lookup", "lora_upload_pages"):
            getattr(L, name).restype = _i32
        _lib = L
    return _lib


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise LoraError(fn, st)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else _vp(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return _vp(stream.cuda_stream)


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return LORA_DTYPE_BF16
    if dt == torch.float32:
        return LORA_DTYPE_F32
    raise ValueError(f"unsupported dtype {dt}")


# ------------------------------------------------------------------ wrappers
class Adapters:
    """rank (int32) and alpha (float32) device tensors, one entry per adapter."""

    def __init__(self, rank: torch.Tensor, alpha: torch.Tensor):
        assert rank.dtype == torch.int32 and alpha.dtype == torch.float32
        assert rank.is_contiguous() and alpha.is_contiguous() and rank.numel() == alpha.numel()
        self.rank, self.alpha = rank, alpha
        self.c = lora_adapters_t(rank.data_ptr(), alpha.data_ptr(), rank.numel())

    @property
    def num_adapters(self) -> int:
        return self.rank.numel()


class Pool:
    """Page pool tensor of shape (num_pages, 16*page_width), bf16 or fp32."""

    def __init__(self, base: torch.Tensor, page_width: int):
        assert base.dim() == 2 and base.shape[1] == 16 * page_width and base.is_contiguous()
        self.base, self.page_width = base, page_width
        self.c = lora_pool_t(base.data_ptr(), base.shape[0], page_width, dtype_code(base.dtype))


class Proj:
    """One projection: X (T, d_in), Y_base and Y (T, d_out) and its page tables."""

    def __init__(self, X: torch.Tensor, Y_base: torch.Tensor, Y: torch.Tensor, a_indptr: torch.Tensor,
                 a_pages: torch.Tensor, b_indptr: torch.Tensor, b_pages: torch.Tensor,
                 d_in: Optional[int] = None, d_out: Optional[int] = None):
        for t in (a_indptr, a_pages, b_indptr, b_pages):
            assert t.dtype == torch.int32 and t.is_contiguous()
        for t in (X, Y_base, Y):
            assert t.dim() == 2 and t.stride(1) == 1
        self.keep = (X, Y_base, Y, a_indptr, a_pages, b_indptr, b_pages)
        d_in = X.shape[1] if d_in is None else d_in
        d_out = Y.shape[1] if d_out is None else d_out
        self.c = lora_proj_t(X.data_ptr(), X.stride(0), Y_base.data_ptr(), Y_base.stride(0), Y.data_ptr(),
                             Y.stride(0), d_in, d_out, a_indptr.data_ptr(), a_pages.data_ptr(),
                             b_indptr.data_ptr(), b_pages.data_ptr())


class Segments:
    """Device buffer for the segments of a T-token batch over N adapters."""

    def __init__(self, T: int, num_adapters: int, device="cuda"):
        L = lib()
        nbytes = L.lora_segments_size(T, num_adapters)
        if nbytes == 0:
            raise ValueError("bad segment capacity")
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.c = lora_segments_t()
        _check("lora_segments_init", L.lora_segments_init(_ptr(self.buf), nbytes, T, num_adapters,
                                                          ctypes.byref(self.c)))
        self.T, self.num_adapters = T, num_adapters

    def _view(self, field: str, n: int) -> torch.Tensor:
        off = getattr(self.c, field) - self.buf.data_ptr()
        return self.buf[off:off + 4 * n].view(torch.int32)

    def counts(self) -> torch.Tensor:
        return self._view("counts", N_COUNTS)

    def arrays(self) -> dict:
        """Host copies of the segment arrays (synchronises)."""
        c = self.counts().cpu()
        S = int(c[COUNT_S])
        return dict(perm=self._view("perm", self.T).cpu().numpy(),
                    seg_indptr=self._view("seg_indptr", S + 1).cpu().numpy(),
                    seg_adapter=self._view("seg_adapter", S).cpu().numpy(),
                    v_indptr=self._view("v_indptr", S + 1).cpu().numpy(),
                    S=S, n_invalid=int(c[COUNT_INVALID]), T_valid=int(c[COUNT_T_VALID]),
                    V_total=int(c[COUNT_V_TOTAL]), flags=int(c[COUNT_FLAGS]))


def workspace(T: int, num_adapters: int, n_projs: int, max_d_in: int, device="cuda") -> torch.Tensor:
    n = lib().lora_workspace_size(T, num_adapters, n_projs, max_d_in)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


# ------------------------------------------------------- the C entry points
def lora_status_string(status: int) -> str:
    return lib().lora_status_string(status).decode()


def lora_v_slices(d_in: int) -> int:
    return int(lib().lora_v_slices(d_in))


def lora_workspace_size(T: int, num_adapters: int, n_projs: int, max_d_in: int) -> int:
    return int(lib().lora_workspace_size(T, num_adapters, n_projs, max_d_in))


def lora_build_segments(ids: torch.Tensor, adapters: Adapters, segs: Segments, ws: torch.Tensor,
                        stream=None) -> None:
    assert ids.dtype == torch.int32 and ids.is_contiguous()
    _check("lora_build_segments", lib().lora_build_segments(
        _ptr(ids), ids.numel(), ctypes.byref(adapters.c), ctypes.byref(segs.c), _ptr(ws), ws.numel(),
        _stream(stream)))


def _proj_group(projs, v):
    if isinstance(projs, Proj):
        projs = [projs]
    if isinstance(v, torch.Tensor):
        v = [v]
    projs, v = list(projs), list(v)
    if len(projs) != len(v):
        raise ValueError("one v buffer per projection")
    for t in v:
        if t.dtype != torch.float32:
            raise TypeError("v must be float32")
    arr = (lora_proj_t * max(len(projs), 1))(*[p.c for p in projs])
    vp = (_vp * max(len(v), 1))(*[_ptr(t) for t in v])
    return arr, len(projs), vp


def lora_shrink(projs, adapters: Adapters, segs: Segments, pool: Pool, v, v_stride: int, stream=None) -> None:
    """projs: a Proj or a sequence of them; v: one fp32 tensor per projection."""
    arr, n, vp = _proj_group(projs, v)
    _check("lora_shrink", lib().lora_shrink(arr, n, ctypes.byref(adapters.c), ctypes.byref(segs.c),
                                            ctypes.byref(pool.c), vp, v_stride, _stream(stream)))


def lora_expand(projs, adapters: Adapters, segs: Segments, pool: Pool, v, v_slices: int, v_stride: int,
                stream=None) -> None:
    """v_slices: 0 = each projection's lora_v_slices(d_in), k >= 1 = k slices for all."""
    arr, n, vp = _proj_group(projs, v)
    _check("lora_expand", lib().lora_expand(arr, n, ctypes.byref(adapters.c), ctypes.byref(segs.c),
                                            ctypes.byref(pool.c), vp, v_slices, v_stride, _stream(stream)))


def lora_apply(ids: Optional[torch.Tensor], segs: Optional[Segments], T: int, projs: Sequence[Proj],
               adapters: Adapters, pool: Pool, ws: torch.Tensor, stream=None) -> None:
    arr = (lora_proj_t * max(len(projs), 1))(*[p.c for p in projs])
    _check("lora_apply", lib().lora_apply(
        _ptr(ids), ctypes.byref(segs.c) if segs is not None else None, T, arr, len(projs),
        ctypes.byref(adapters.c), ctypes.byref(pool.c), _ptr(ws), ws.numel(), _stream(stream)))


def lora_apply_noalloc(ids: Optional[torch.Tensor], segs: Optional[Segments], T: int, projs: Sequence[Proj],
                       adapters: Adapters, pool: Pool, stream=None) -> None:
    """lora_apply on the library's own fixed device array (no workspace)."""
    arr = (lora_proj_t * max(len(projs), 1))(*[p.c for p in projs])
    _check("lora_apply_noalloc", lib().lora_apply_noalloc(
        _ptr(ids), ctypes.byref(segs.c) if segs is not None else None, T, arr, len(projs),
        ctypes.byref(adapters.c), ctypes.byref(pool.c), _stream(stream)))


def lora_set_wait_limit(ns: int) -> None:
    """Bound on lora_apply's internal phase wait (0: default; < 0: give up after |ns|, for tests)."""
    lib().lora_set_wait_limit(int(ns))


def lora_set_launch_mode(mode: int) -> None:
    """LORA_LAUNCH_AUTO / _SINGLE / _TWO for lora_apply (process-wide)."""
    _check("lora_set_launch_mode", lib().lora_set_launch_mode(int(mode)))


def lora_validate_tables(rank, d_in: int, d_out: int, page_width: int, num_pages: int,
                         a_indptr, a_pages, b_indptr, b_pages) -> int:
    """Host-array validation (numpy int32 arrays); returns the status code."""
    import numpy as np
    arrs = [np.ascontiguousarray(x, np.int32) for x in (rank, a_indptr, a_pages, b_indptr, b_pages)]
    p = [a.ctypes.data_as(_vp) for a in arrs]
    return int(lib().lora_validate_tables(len(arrs[0]), p[0], d_in, d_out, page_width, num_pages,
                                          p[1], p[2], p[3], p[4]))


# ------------------------------------------------- pool manager (lora_pool.h)
class PageCache:
    """Resident adapters of a page pool: page allocation and LRU eviction.
    Host state only; not thread-safe."""

    def __init__(self, num_pages: int):
        h = _vp()
        _check("lora_cache_create", lib().lora_cache_create(num_pages, ctypes.byref(h)))
        self.h, self.num_pages = h, num_pages

    def __del__(self):
        h, self.h = getattr(self, "h", None), None
        if h and _lib is not None:
            _lib.lora_cache_destroy(h)

    @property
    def free_pages(self) -> int:
        return int(lib().lora_cache_free_pages(self.h))

    @property
    def num_resident(self) -> int:
        return int(lib().lora_cache_num_resident(self.h))

    def admit(self, key: int, n_pages: int, max_evicted: Optional[int] = None):
        """Returns (hit, pages (int32 numpy), evicted keys (int64 numpy, oldest first))."""
        import numpy as np
        max_evicted = self.num_pages if max_evicted is None else max_evicted
        pages = np.empty(max(n_pages, 1), np.int32)
        ev = np.empty(max(max_evicted, 1), np.int64)
        hit, nev = _i32(), _i32()
        _check("lora_cache_admit", lib().lora_cache_admit(
            self.h, key, n_pages, pages.ctypes.data_as(_vp), ctypes.byref(hit), ev.ctypes.data_as(_vp),
            max_evicted, ctypes.byref(nev)))
        return bool(hit.value), pages[:n_pages], ev[:nev.value]

    def lookup(self, key: int):
        """Pages of a resident adapter (int32 numpy; empty if not resident),
        without touching the recency order."""
        import numpy as np
        n = _i32()
        _check("lora_cache_lookup", lib().lora_cache_lookup(self.h, key, None, 0, ctypes.byref(n)))
        pages = np.empty(max(n.value, 1), np.int32)
        _check("lora_cache_lookup", lib().lora_cache_lookup(self.h, key, pages.ctypes.data_as(_vp), n.value,
                                                            ctypes.byref(n)))
        return pages[:n.value]

    def set_pinned(self, key: int, pinned: bool = True) -> None:
        _check("lora_cache_set_pinned", lib().lora_cache_set_pinned(self.h, key, int(bool(pinned))))

    def release(self, key: int) -> None:
        _check("lora_cache_release", lib().lora_cache_release(self.h, key))


def lora_upload_pages(pool: Pool, host_src: torch.Tensor, pages, stream=None) -> None:
    """Copy host_src (n_pages, 16*page_width) into the pool pages listed in
    ``pages`` (host int32 array), asynchronously on the stream.  host_src
    should be pinned and must stay alive until the stream has passed the copy."""
    import numpy as np
    pg = np.ascontiguousarray(pages, np.int32)
    if host_src.device.type != "cpu" or not host_src.is_contiguous() or host_src.dtype != pool.base.dtype:
        raise ValueError("host_src must be a contiguous CPU tensor of the pool's dtype")
    if host_src.dim() != 2 or host_src.shape[0] != len(pg) or host_src.shape[1] != pool.base.shape[1]:
        raise ValueError("host_src must hold one pool page per page id")
    _check("lora_upload_pages", lib().lora_upload_pages(ctypes.byref(pool.c), _ptr(host_src),
                                                        pg.ctypes.data_as(_vp), len(pg), _stream(stream)))


def hip_runtimes_mapped() -> list:
    """Paths of every libamdhip64 mapped in this process."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(line.split()[-1])
    return sorted(paths)
