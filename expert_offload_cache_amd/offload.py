"""Offloaded MoE stack: routed experts in a pinned host pool, one LRU slot cache in HBM shared by
all layers, decode with a per-layer device->host id read-back, prefill that double-buffers the
next layer's experts (FreeToken linux guide, "MoE memory handling" and its mechanism table;
FreeToken GGUF page, offload backend; FreeToken RTX 5090 page, memory hierarchy and prefill).

Marshalling and orchestration only: every step runs in libmoe (moe_route, moe_permute,
moe_expert_ffn_grouped, moe_combine, moe_cache_*), on two HIP streams (compute, copy).

Pool contents: `n_images` distinct seeded expert images are packed once and key (layer, expert)
holds image (layer * E + expert) % n_images.  Every key still has its own bytes in the pinned pool
and its own slot, copy and LRU entry; only the weight values repeat, which changes neither the
traffic nor the cache decisions.
"""
from __future__ import annotations

import ctypes
import time
from typing import Optional

import numpy as np

from . import (MoeError, SlotCache, combine, expert_ffn_grouped, pack_expert, permute, pinned_alloc, pinned_free,
               route, slot_bytes, workspace_bytes, WDT)
from ._lib import MOE_BF16, MOE_F32
from .layer import _expert_arrays, _to_device


class OffloadStack:
    """L stacked MoE layers whose routed experts live in a pinned host pool behind an LRU slot cache."""

    def __init__(self, wl, n_layers: int, n_slots: int, seed: int = 0, n_images: Optional[int] = None,
                 x_bank: int = 8, prefill_tokens: int = 0, device="cuda", log=None):
        import torch
        import synth

        self.wl, self.L, self.E, self.k, self.d, self.f = wl, n_layers, wl.E, wl.k, wl.d, wl.f
        self.seed, self.device, self.log = seed, device, log or (lambda *a: None)
        self.stride = slot_bytes(wl.d, wl.f, wl.wdt)
        L, E = self.L, self.E
        self.n_images = int(n_images or E)
        self.act_code = MOE_BF16 if wl.act == "bf16" else MOE_F32

        # distinct routed images, packed once
        t0 = time.perf_counter()
        imgs = np.empty((self.n_images, self.stride), dtype=np.uint8)
        for i in range(self.n_images):
            ew = synth.expert_weights(wl, seed, i // E, i % E)
            pack_expert(wl.wdt, wl.d, wl.f, *_expert_arrays(ew), out=imgs[i])
        self.log(f"packed {self.n_images} expert images in {time.perf_counter() - t0:.1f} s")

        # pinned host pool, one stride per key
        t0 = time.perf_counter()
        self.pool_bytes = L * E * self.stride
        self.pinned = pinned_alloc(self.pool_bytes)
        try:
            view = np.ctypeslib.as_array((ctypes.c_uint8 * self.pool_bytes).from_address(self.pinned))
            for key in range(L * E):
                view[key * self.stride:(key + 1) * self.stride] = imgs[key % self.n_images]
            del view
        except Exception:
            pinned_free(self.pinned)
            raise
        self.log(f"pinned pool {self.pool_bytes / 2**30:.1f} GiB filled in {time.perf_counter() - t0:.1f} s")
        del imgs
        host_ptrs = [self.pinned + key * self.stride for key in range(L * E)]

        # HBM slots and the slot table the kernels read
        self.n_slots = int(n_slots)
        self.slot_pool = torch.empty(self.n_slots * self.stride, dtype=torch.uint8, device=device)
        self.slot_table = torch.empty(L * E, dtype=torch.int32, device=device)
        self.cache = SlotCache(L, E, self.n_slots, self.stride, self.slot_pool, self.slot_table, host_ptrs)

        # resident per-layer state: router, bias, shared expert, activation banks
        self.w_router, self.bias, self.shared, self.x_dec, self.x_pre = [], [], [], [], []
        for l in range(L):
            li = synth.layer_inputs(wl, x_bank, seed, layer=l, batch=1, with_experts=False)
            self.w_router.append(_to_device(li.w_router, wl.act, device))
            self.bias.append(None if li.bias is None else torch.from_numpy(li.bias).to(device))
            self.x_dec.append(_to_device(li.x, wl.act, device))
            if wl.shared:
                sh = synth.expert_weights(wl, seed, self.shared_layer_of(l), 0, shared=True)
                self.shared.append(torch.from_numpy(pack_expert(wl.wdt, wl.d, wl.f, *_expert_arrays(sh))).to(device))
            else:
                self.shared.append(None)
            if prefill_tokens:
                xp = synth.layer_inputs(wl, prefill_tokens, seed, layer=l, batch=0, with_experts=False).x
                self.x_pre.append(_to_device(xp, wl.act, device))
        self.compute = torch.cuda.Stream(device=device)
        self.copy = torch.cuda.Stream(device=device)
        self._ws = {}

    # ------------------------------------------------------------------------------------------
    def image_of(self, layer: int, expert: int) -> int:
        """Image held by key (layer, expert); image i is synth.expert_weights(wl, seed, i // E, i % E)."""
        return (layer * self.E + expert) % self.n_images

    def shared_layer_of(self, layer: int) -> int:
        """The shared expert of `layer` is synth.expert_weights(wl, seed, this, 0, shared=True)."""
        return layer % max(1, self.n_images // self.E)

    def _workspace(self, T: int):
        import torch

        if T not in self._ws:
            n = workspace_bytes(T, self.d, self.f, self.E, self.k, self.wl.shared, self.act_code, WDT[self.wl.wdt])
            self._ws[T] = torch.zeros(n, dtype=torch.uint8, device=self.device)
        return self._ws[T]

    def _layer_kernels(self, l: int, x, idx, w, counts, offsets, perm, inv, y=None, y_perm=None):
        """Grouped experts through layer l's slot-table row, then the combine (compute stream)."""
        E = self.E
        table = self.slot_table[l * E:(l + 1) * E]
        y_perm, _ = expert_ffn_grouped(x, perm, offsets, counts, table, self.slot_pool, self.n_slots, self.stride,
                                       self.wl.wdt, self.f, self.k, shared_w=self.shared[l], y_perm=y_perm,
                                       ws=self._workspace(x.shape[0]), stream=self.compute)
        return combine(y_perm, w, inv, self.k, self.shared[l] is not None, x.dtype, y=y, stream=self.compute)

    # ------------------------------------------------------------------------------------------
    def prefill(self, T: Optional[int] = None, keep_outputs: bool = False):
        """All L layers over the prefill batch; layer l+1's experts stream in while layer l computes.

        Returns wall seconds (and the per-layer outputs when keep_outputs)."""
        import torch

        outs = []
        T = T or self.x_pre[0].shape[0]
        self._workspace(T)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.cache.prefetch_layer(0, self.copy, self.compute)
        with torch.cuda.stream(self.compute):
            for l in range(self.L):
                x = self.x_pre[l][:T]
                idx, w, _ = route(x, self.w_router[l], self.bias[l], self.k, stream=self.compute)
                counts, offsets, perm, inv = permute(idx, self.E, stream=self.compute)
                y = self._layer_kernels(l, x, idx, w, counts, offsets, perm, inv)
                if keep_outputs:
                    outs.append((idx, y))
                if l + 1 < self.L:
                    self.cache.prefetch_layer(l + 1, self.copy, self.compute)
                self.cache.mark_read(l, self.compute)
        self.compute.synchronize()
        el = time.perf_counter() - t0
        return (el, outs) if keep_outputs else el

    def decode(self, trace: np.ndarray, keep_outputs: bool = False, steps: Optional[int] = None):
        """Batch-1 decode over a routing trace [steps, L, k]: each layer's ids are forced from the
        trace (gates are the renormalised softmax of the router logits at those ids); per layer
        route -> ids back to the host -> cache lookup + fill -> permute/GEMV/combine.

        Returns wall seconds (and outputs [(step, layer, y)] when keep_outputs)."""
        import torch

        steps = steps or trace.shape[0]
        L, E, k = self.L, self.E, self.k
        forced = torch.from_numpy(np.ascontiguousarray(trace[:steps], dtype=np.int32)).to(self.device)
        host_idx = torch.empty((1, k), dtype=torch.int32, pin_memory=True)
        done = torch.cuda.Event()
        dev = self.device
        rbuf = (torch.empty((1, k), dtype=torch.int32, device=dev), torch.empty((1, k), dtype=torch.float32, device=dev),
                torch.empty((1, E), dtype=torch.float32, device=dev))
        pbuf = (torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
                torch.empty(k, dtype=torch.int32, device=dev), torch.empty(k, dtype=torch.int32, device=dev))
        y_perm = torch.empty((k + (1 if self.wl.shared else 0), self.d), dtype=torch.float32, device=dev)
        y_buf = torch.empty((1, self.d), dtype=self.x_dec[0].dtype, device=dev)
        outs = []
        nb = self.x_dec[0].shape[0]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(self.compute):
            for s in range(steps):
                for l in range(L):
                    x = self.x_dec[l][s % nb:s % nb + 1]
                    idx, w, _ = route(x, self.w_router[l], self.bias[l], k, forced_idx=forced[s, l:l + 1],
                                      out=rbuf, stream=self.compute)
                    counts, offsets, perm, inv = permute(idx, E, out=pbuf, stream=self.compute)
                    host_idx.copy_(idx, non_blocking=True)
                    done.record(self.compute)
                    done.synchronize()  # the ids cross to the host: the cache decides there
                    ids = np.unique(host_idx.numpy())
                    self.cache.lookup(l, ids)
                    self.cache.fill(self.copy, self.compute)
                    y = self._layer_kernels(l, x, idx, w, counts, offsets, perm, inv, y=y_buf, y_perm=y_perm)
                    self.cache.mark_read(l, self.compute)
                    if keep_outputs:
                        outs.append((s, l, y.clone()))
        self.compute.synchronize()
        el = time.perf_counter() - t0
        return (el, outs) if keep_outputs else el

    def close(self):
        import torch

        if getattr(self, "cache", None) is not None:
            torch.cuda.synchronize()
            self.cache.close()
            self.cache = None
        if getattr(self, "pinned", None):
            pinned_free(self.pinned)
            self.pinned = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
