"""Device residency of a synthetic batch: copies a host workload (ids, ranks,
alphas, page tables, pool, activations) into device tensors and wraps them
in the binding's descriptors.  Plumbing only; no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import lora


def host_to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """fp32 values or bf16 bit patterns (uint16) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def device_to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> fp32 values or bf16 bit patterns (uint16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@dataclass
class DeviceBatch:
    T: int
    dtype: str
    ids: torch.Tensor
    adapters: lora.Adapters
    pool: lora.Pool
    tables: List[tuple]
    X: List[torch.Tensor]
    Y_base: List[torch.Tensor]
    Y: List[torch.Tensor]
    projs: List[lora.Proj] = field(default_factory=list)

    def proj(self, p: int, in_place: bool = False) -> lora.Proj:
        a_ip, a_pg, b_ip, b_pg = self.tables[p]
        Y = self.Y_base[p] if in_place else self.Y[p]
        return lora.Proj(self.X[p], self.Y_base[p], Y, a_ip, a_pg, b_ip, b_pg)


def to_device(w, device="cuda", pool: Optional[torch.Tensor] = None) -> DeviceBatch:
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)
    ids = i32(w.ids)
    adapters = lora.Adapters(i32(w.ranks), torch.from_numpy(np.ascontiguousarray(w.alpha, np.float32)).to(device))
    if pool is None:
        pool = host_to_device(w.pool, w.dtype, device)
    pl = lora.Pool(pool, w.page_width)
    tables = [(i32(t.a_indptr), i32(t.a_pages), i32(t.b_indptr), i32(t.b_pages)) for t in w.tables]
    X = [host_to_device(x, w.dtype, device) for x in w.X]
    Yb = [host_to_device(y, w.dtype, device) for y in w.Y_base]
    Y = [torch.empty_like(y) for y in Yb]
    b = DeviceBatch(w.T, w.dtype, ids, adapters, pl, tables, X, Yb, Y)
    b.projs = [b.proj(p) for p in range(len(tables))]
    return b
