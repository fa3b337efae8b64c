"""Device-resident MoE layer: weights packed into an HBM slot pool, forward = the four libmoe calls.

Marshalling only: packing happens in libmoe (moe_pack_expert), compute in its kernels.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import (combine, expert_ffn_grouped, pack_expert, permute_workspace, route_permute, slot_bytes, workspace_bytes,
               y_perm_dtype, WDT)
from ._lib import MOE_BF16, MOE_F32


def _to_device(a: np.ndarray, dtype: str, device):
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    raise ValueError(dtype)


def _expert_arrays(ew):
    return (ew.wg, ew.wu, ew.wd, getattr(ew, "sg", None), getattr(ew, "su", None), getattr(ew, "sd", None))


def pack_pool(experts, slot_of_expert, n_slots: int, d: int, f: int, wdt: str) -> np.ndarray:
    """Host image of a slot pool: expert e packed into slot slot_of_expert[e]."""
    stride = slot_bytes(d, f, wdt)
    pool = np.zeros((n_slots, stride), dtype=np.uint8)
    for e, ew in enumerate(experts):
        s = int(slot_of_expert[e])
        if s >= 0:
            pack_expert(wdt, d, f, *_expert_arrays(ew), out=pool[s])
    return pool


class DeviceLayer:
    """One MoE layer whose routed experts sit in HBM slots (all resident)."""

    def __init__(self, d, f, E, k, act: str, wdt: str, w_router, bias, experts, shared=None,
                 slot_of_expert=None, n_slots: Optional[int] = None, device="cuda"):
        import torch

        self.d, self.f, self.E, self.k, self.act, self.wdt = d, f, E, k, act, wdt
        self.device = device
        self.stride = slot_bytes(d, f, wdt)
        if slot_of_expert is None:
            slot_of_expert = np.arange(E, dtype=np.int32)
        self.n_slots = int(n_slots if n_slots is not None else max(int(np.max(slot_of_expert)) + 1, 1))
        host = pack_pool(experts, slot_of_expert, self.n_slots, d, f, wdt)
        self.pool = torch.from_numpy(host.reshape(-1)).to(device)
        del host
        self.slot_of_expert = torch.from_numpy(np.ascontiguousarray(slot_of_expert, dtype=np.int32)).to(device)
        self.w_router = _to_device(w_router, act, device)
        self.bias = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(device)
        self.shared = None
        if shared is not None:
            img = pack_expert(wdt, d, f, *_expert_arrays(shared))
            self.shared = torch.from_numpy(img).to(device)
        self.act_code = MOE_BF16 if act == "bf16" else MOE_F32

    @classmethod
    def from_inputs(cls, li, device="cuda", n_slots=None):
        wl = li.wl
        return cls(wl.d, wl.f, wl.E, wl.k, wl.act, wl.wdt, li.w_router, li.bias, li.experts, li.shared,
                   li.slot_of_expert, n_slots=n_slots, device=device)

    def x_to_device(self, x: np.ndarray):
        return _to_device(x, self.act, self.device)

    def workspace(self, T: int):
        import torch

        n = workspace_bytes(T, self.d, self.f, self.E, self.k, self.shared is not None, self.act_code, WDT[self.wdt])
        return torch.zeros(n, dtype=torch.uint8, device=self.device)

    def buffers(self, T: int):
        """Outputs of a T-token forward allocated once (a serving loop's buffers): forward(...,
        bufs=...) writes into them, so each call overwrites the previous call's results."""
        import torch

        dev, k, E, d = self.device, self.k, self.E, self.d
        rows = T * k + (T if self.shared is not None else 0)
        act = torch.bfloat16 if self.act == "bf16" else torch.float32
        i32 = dict(dtype=torch.int32, device=dev)
        return dict(
            route=(torch.empty((T, k), **i32), torch.empty((T, k), dtype=torch.float32, device=dev),
                   torch.empty((T, E), dtype=torch.float32, device=dev), torch.empty(E, **i32),
                   torch.empty(E + 1, **i32), torch.empty(T * k, **i32), torch.empty(T * k, **i32)),
            y_perm=torch.empty((rows, d), dtype=y_perm_dtype(act, T), device=dev),
            y=torch.empty((T, d), dtype=act, device=dev),
            ws=self.workspace(T), pws=permute_workspace(T, k, E, dev))

    def forward(self, x, forced_idx=None, ws=None, stream=None, slot_of_expert=None, bufs=None):
        """x: device tensor [T, d].  Returns a dict of every intermediate and y [T, d].  With
        `bufs` (from buffers(T)) the outputs are written there instead of new tensors."""
        T = x.shape[0]
        b = bufs or {}
        pws = b["pws"] if "pws" in b else permute_workspace(T, self.k, self.E, x.device)
        idx, w, logits, counts, offsets, perm, inv = route_permute(x, self.w_router, self.bias, self.k,
                                                                  forced_idx=forced_idx, out=b.get("route"),
                                                                  stream=stream, ws=pws)
        if ws is None:
            ws = b["ws"] if "ws" in b else self.workspace(T)
        soe = self.slot_of_expert if slot_of_expert is None else slot_of_expert
        y_perm, ws = expert_ffn_grouped(x, perm, offsets, counts, soe, self.pool, self.n_slots, self.stride,
                                        self.wdt, self.f, self.k, shared_w=self.shared, y_perm=b.get("y_perm"),
                                        y_dtype=y_perm_dtype(x.dtype, T),
                                        ws=ws, stream=stream)
        y = combine(y_perm, w, inv, self.k, self.shared is not None, x.dtype, y=b.get("y"), stream=stream)
        return dict(y=y, topk_idx=idx, topk_w=w, logits=logits, counts=counts, offsets=offsets, perm=perm,
                    inv_perm=inv, y_perm=y_perm, ws=ws)
