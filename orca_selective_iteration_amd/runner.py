"""Device-side setup around the C ABI: allocates the weights, the K/V pool and
workspace with PyTorch (device memory only), reserves each request's slots
through the library's K/V manager and calls orca_iteration.  No arithmetic
of the method happens here; every step of the iteration runs in liborca.so.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

from . import lib as L
from .synth import HostInputs, Workload, device_normal_, device_param_tensors


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def orca_dtype(dtype: str) -> int:
    return L.ORCA_BF16 if dtype == "bf16" else L.ORCA_F32


class DeviceModel:
    """Weights + K/V pool + engine context for one workload on one GPU.

    kv_capacity: token slots per layer/head (default: every request's
    kv_len + q_len plus `slack` slots each).
    """

    def __init__(self, work: Workload, host: Optional[HostInputs] = None, device: str = "cuda",
                 seed: int = 0, kv_capacity: Optional[int] = None, slack: int = 0,
                 max_rows: Optional[int] = None, max_reqs: Optional[int] = None,
                 use_kv_manager: bool = True, fill_caches: bool = True, log=None):
        import torch
        log = log or (lambda *a: None)
        self.work = work
        self.device = device
        self.tdt = torch_dtype(work.dtype)
        self.odt = orca_dtype(work.dtype)
        d = work.head_dim
        need = [kv + q + slack for kv, q in zip(work.kv_len, work.q_len)]
        self.cap = int(kv_capacity if kv_capacity is not None else max(sum(need), 1))
        # weights
        if host is not None:
            self.weights = [{k: torch.from_numpy(np.ascontiguousarray(v)).to(device=device, dtype=self.tdt)
                             for k, v in p.items()} for p in host.params]
        else:
            self.weights = []
            for l in range(work.layers):
                self.weights.append(device_param_tensors(work, seed * 1000003 + l, device,
                                                         self.tdt))
                if l % 10 == 9:
                    log(f"weights: {l + 1}/{work.layers} layers drawn")
        # one pool [layers][heads][cap][2][d]: each slot's key row, then its
        # value row; k_pool and v_pool are the two [layers][heads][cap][d] views
        self.kv_pool = torch.empty((work.layers, work.heads, self.cap, 2, d), dtype=self.tdt,
                                   device=device)
        self.k_pool = self.kv_pool[:, :, :, 0]
        self.v_pool = self.kv_pool[:, :, :, 1]
        # reservations, in batch order
        self.kv = L.orca_kv_create(self.cap) if use_kv_manager else None
        self.bases: List[int] = []
        off = 0
        for n in need:
            if self.kv is not None:
                self.bases.append(L.orca_kv_alloc(self.kv, max(n, 1)))
            else:
                self.bases.append(off)
                off += n
        if fill_caches:
            if host is not None:
                self.load_host_caches(host.caches)
            else:
                log(f"filling the K/V pool: {self.kv_pool.numel() * self.kv_pool.element_size() / 1e9:.1f} GB")
                self.fill_device_caches(seed)
                log("K/V pool filled")
        self.max_rows = int(max_rows or max(work.rows, 1))
        self.max_reqs = int(max_reqs or max(work.n_reqs, 1))
        self.ctx = L.orca_create(work.layers, work.hidden, work.heads, work.ffn, self.odt,
                                 work.eps, self.cap, self.weights, self.kv_pool,
                                 self.kv, self.max_rows, self.max_reqs)
        self.ws_bytes = L.orca_workspace_bytes(self.ctx)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        assert self.ws.data_ptr() % 256 == 0

    # ------------------------------------------------------------- caches
    def load_host_caches(self, caches):
        import torch
        w = self.work
        for l in range(w.layers):
            for i, (k, v) in enumerate(caches[l]):
                kv = k.shape[0]
                if kv == 0:
                    continue
                b = self.bases[i]
                kt = torch.from_numpy(k).to(self.device, self.tdt).view(kv, w.heads, w.head_dim)
                vt = torch.from_numpy(v).to(self.device, self.tdt).view(kv, w.heads, w.head_dim)
                self.k_pool[l, :, b:b + kv] = kt.permute(1, 0, 2)
                self.v_pool[l, :, b:b + kv] = vt.permute(1, 0, 2)

    def fill_device_caches(self, seed: int):
        """Seeded N(0,1) in every key and value row of the pool (cached and
        free slots)."""
        device_normal_(self.kv_pool, seed * 7919 + 1)

    def cache_rows(self, layer: int, req: int, lo: int, hi: int):
        """K, V entries lo..hi-1 of request `req` at `layer` as [n, H] fp32 host arrays."""
        w = self.work
        b = self.bases[req]
        k = self.k_pool[layer, :, b + lo:b + hi].permute(1, 0, 2).reshape(hi - lo, w.hidden)
        v = self.v_pool[layer, :, b + lo:b + hi].permute(1, 0, 2).reshape(hi - lo, w.hidden)
        return k.float().cpu().numpy(), v.float().cpu().numpy()

    # ---------------------------------------------------------- iteration
    def descriptors(self, q_len: Sequence[int] = None, kv_len: Sequence[int] = None,
                    reqs: Sequence[int] = None):
        """Descriptor tuples for requests `reqs` (default all, batch order)."""
        w = self.work
        idx = list(range(w.n_reqs)) if reqs is None else list(reqs)
        q_len = q_len or [w.q_len[i] for i in idx]
        kv_len = kv_len or [w.kv_len[i] for i in idx]
        out, off = [], 0
        for i, q, kv in zip(idx, q_len, kv_len):
            # one new token over a cache: increment; otherwise a prompt or a
            # prompt chunk over the tokens earlier chunks cached
            phase = L.ORCA_INCREMENT if (kv > 0 and q == 1) else L.ORCA_INITIATION
            out.append((off, q, kv, phase, self.bases[i]))
            off += q
        return out

    def iteration(self, reqs, x, y, stream=None):
        L.orca_iteration(self.ctx, reqs, x, y, self.ws, self.ws_bytes, stream)

    def close(self):
        if getattr(self, "ctx", None):
            L.orca_destroy(self.ctx)
            self.ctx = None
        if getattr(self, "kv", None):
            L.orca_kv_destroy(self.kv)
            self.kv = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
