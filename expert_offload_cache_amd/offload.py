"""Offloaded MoE stack: routed experts in a pinned host pool, one LRU slot cache in HBM shared by
all layers, decode with a per-layer device->host id read-back, prefill that double-buffers the
next layer's experts (FreeToken linux guide, "MoE memory handling" and its mechanism table;
FreeToken GGUF page, offload backend; FreeToken RTX 5090 page, memory hierarchy and prefill).

Marshalling and orchestration only: every step runs in libmoe (moe_route_permute,
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

from . import (MoeError, SlotCache, combine, expert_ffn_grouped, hybrid_split, pack_expert, permute_workspace,
               pinned_alloc, pinned_free, route_permute, slot_bytes, workspace_bytes, y_perm_dtype, WDT)
from ._lib import MOE_BF16, MOE_F32
from .layer import _expert_arrays, _to_device


def _hybrid_args(hybrid):
    """hybrid = (cpu_rate, pcie_rate[, copy_too[, host_fixed_s]]) -> the four values."""
    cpu, pcie = float(hybrid[0]), float(hybrid[1])
    copy_too = bool(hybrid[2]) if len(hybrid) > 2 else True
    fixed = float(hybrid[3]) if len(hybrid) > 3 else 0.0
    return cpu, pcie, copy_too, fixed


class OffloadStack:
    """L stacked MoE layers whose routed experts live in a pinned host pool behind an LRU slot cache.

    Every device buffer is allocated before the pool is pinned: on the hosts this runs on, device
    allocations made after a large pinned allocation can be refused."""

    def __init__(self, wl, n_layers: int, n_slots: int, seed: int = 0, n_images: Optional[int] = None,
                 x_bank: int = 8, prefill_tokens: int = 0, device="cuda", log=None, slot_pool=None,
                 min_layers: Optional[int] = None):
        import torch
        import synth

        self.wl, self.L, self.E, self.k, self.d, self.f = wl, n_layers, wl.E, wl.k, wl.d, wl.f
        self.seed, self.device, self.log = seed, device, log or (lambda *a: None)
        self.stride = slot_bytes(wl.d, wl.f, wl.wdt)
        L, E, k, d = self.L, self.E, self.k, self.d
        self.n_images = int(n_images or E)
        self.act_code = MOE_BF16 if wl.act == "bf16" else MOE_F32
        self.n_slots = int(n_slots)
        self.pinned = []
        self.cache = None

        # ---- device memory: slots, slot table, per-layer state, call buffers ----
        if slot_pool is None:
            slot_pool = torch.empty(self.n_slots * self.stride, dtype=torch.uint8, device=device)
        if slot_pool.numel() < self.n_slots * self.stride:
            raise ValueError("slot_pool is smaller than n_slots * slot stride")
        self.slot_pool = slot_pool
        self.slot_table = torch.empty(L * E, dtype=torch.int32, device=device)
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
        self._ws = {}
        self._bufs = {}
        self.cpu_experts = 0
        for T in ({1, prefill_tokens} - {0}):
            self._workspace(T)
            self._buffers(T)
        self.compute = torch.cuda.Stream(device=device)
        self.copy = torch.cuda.Stream(device=device)
        self._host_idx = torch.empty((1, k), dtype=torch.int32, pin_memory=True)

        # ---- distinct routed images, packed once ----
        t0 = time.perf_counter()
        imgs = np.empty((self.n_images, self.stride), dtype=np.uint8)
        for i in range(self.n_images):
            ew = synth.expert_weights(wl, seed, i // E, i % E)
            pack_expert(wl.wdt, wl.d, wl.f, *_expert_arrays(ew), out=imgs[i])
        self.log(f"packed {self.n_images} expert images in {time.perf_counter() - t0:.1f} s")

        # ---- pinned host pool: one stride per key, one block (a refused attempt pins nothing) ----
        t0 = time.perf_counter()
        self.layer_bytes = E * self.stride
        try:
            self.pinned = [pinned_alloc(L * self.layer_bytes)]
        except MoeError as err:
            if min_layers is None or min_layers >= L:
                raise
            self.log(f"pinning {L} layers failed ({err}); running {min_layers} layers")
            self.L = L = min_layers
            self.pinned = [pinned_alloc(L * self.layer_bytes)]
            for lst in (self.w_router, self.bias, self.shared, self.x_dec, self.x_pre):
                del lst[L:]
        view = np.ctypeslib.as_array((ctypes.c_uint8 * (L * self.layer_bytes)).from_address(self.pinned[0]))
        for key in range(L * E):
            view[key * self.stride:(key + 1) * self.stride] = imgs[self.image_of(key // E, key % E)]
        del view, imgs
        self.pool_bytes = L * self.layer_bytes
        self.log(f"pinned pool {self.pool_bytes / 2**30:.1f} GiB filled in {time.perf_counter() - t0:.1f} s")
        self.new_cache(self.n_slots)

    # ------------------------------------------------------------------------------------------
    def new_cache(self, n_slots: int):
        """A fresh, empty LRU cache of n_slots slots over this stack's pool and slot memory."""
        if n_slots * self.stride > self.slot_pool.numel():
            raise ValueError("not enough slot memory")
        if self.cache is not None:
            self.cache.close()
        self.n_slots = int(n_slots)
        self.cache = SlotCache(self.L, self.E, self.n_slots, self.stride, self.slot_pool, self.slot_table,
                               self.host_ptrs())

    def resize(self, n_slots: int):
        """Change the cache capacity between layers (a safe point); moves run on the copy stream."""
        if n_slots * self.stride > self.slot_pool.numel():
            raise ValueError("not enough slot memory")
        self.cache.resize(n_slots, self.copy, self.compute)
        self.n_slots = int(n_slots)

    def host_ptrs(self):
        """Pinned address of every key (layer * E + expert)."""
        return [self.pinned[0] + key * self.stride for key in range(self.L * self.E)]

    def _free_pinned(self):
        for p in self.pinned:
            pinned_free(p)
        self.pinned = []

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

    def _buffers(self, T: int):
        """Outputs of route, permute, the grouped experts and the combine for a T-token call."""
        import torch

        if T not in self._bufs:
            dev, k, E, d = self.device, self.k, self.E, self.d
            rows = T * k + (T if self.wl.shared else 0)
            act = torch.bfloat16 if self.wl.act == "bf16" else torch.float32
            self._bufs[T] = dict(
                route=(torch.empty((T, k), dtype=torch.int32, device=dev),
                       torch.empty((T, k), dtype=torch.float32, device=dev),
                       torch.empty((T, E), dtype=torch.float32, device=dev)),
                perm=(torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
                      torch.empty(T * k, dtype=torch.int32, device=dev),
                      torch.empty(T * k, dtype=torch.int32, device=dev)),
                y_perm=torch.empty((rows, d), dtype=y_perm_dtype(act, T), device=dev),
                y=torch.empty((T, d), dtype=act, device=dev),
                pws=permute_workspace(T, k, E, dev))
        return self._bufs[T]

    def _layer(self, l: int, x, forced=None):
        """One layer on the compute stream up to the grouped experts' inputs: route + permute."""
        T = x.shape[0]
        b = self._buffers(T)
        idx, w, _, *perm = route_permute(x, self.w_router[l], self.bias[l], self.k, forced_idx=forced,
                                         out=b["route"] + b["perm"], stream=self.compute, ws=b["pws"])
        return idx, w, tuple(perm)

    def _experts(self, l: int, x, w, perm, table=None, do_combine: bool = True, with_shared: bool = True):
        """Grouped experts through layer l's slot-table row (or `table`), then the combine (compute
        stream).  Without the combine it returns y_perm."""
        T, E = x.shape[0], self.E
        b = self._buffers(T)
        counts, offsets, p, inv = perm
        if table is None:
            table = self.slot_table[l * E:(l + 1) * E]
        y_perm, _ = expert_ffn_grouped(x, p, offsets, counts, table, self.slot_pool, self.n_slots, self.stride,
                                       self.wl.wdt, self.f, self.k,
                                       shared_w=self.shared[l] if with_shared else None, y_perm=b["y_perm"],
                                       ws=self._workspace(T), stream=self.compute)
        if not do_combine:
            return y_perm
        return combine(y_perm, w, inv, self.k, self.shared[l] is not None, x.dtype, y=b["y"], stream=self.compute)

    # ------------------------------------------------------------------------------------------
    def prefill(self, keep_outputs: bool = False):
        """All L layers over the prefill batch; layer l+1's experts stream in on the copy stream
        while layer l computes (when the cache holds two layers, else layer by layer).
        Returns wall seconds (and per-layer (ids, y) when keep_outputs)."""
        import torch

        outs = []
        # double buffering needs room for two layers (the one read and the one copied in)
        double = self.n_slots >= 2 * self.E
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if double:
            self.cache.prefetch_layer(0, self.copy, self.compute)
        with torch.cuda.stream(self.compute):
            for l in range(self.L):
                if not double:
                    self.cache.prefetch_layer(l, self.copy, self.compute)
                x = self.x_pre[l]
                idx, w, perm = self._layer(l, x)
                y = self._experts(l, x, w, perm)
                if keep_outputs:
                    outs.append((idx.clone(), y.clone()))
                if double and l + 1 < self.L:
                    self.cache.prefetch_layer(l + 1, self.copy, self.compute)
                self.cache.mark_read(l, self.compute)
        self.compute.synchronize()
        el = time.perf_counter() - t0
        return (el, outs) if keep_outputs else el

    def decode(self, trace: np.ndarray, keep_outputs: bool = False, steps: Optional[int] = None, first_step: int = 0,
               hybrid: Optional[tuple] = None, split_launch: bool = False, native: bool = True):
        """Batch-1 decode over a routing trace [steps, L, k]: each layer's ids are forced from the
        trace (gates are the renormalised softmax of the router logits at those ids); per layer
        route + permute -> ids back to the host -> cache lookup + fill -> GEMV/combine.

        `first_step` numbers the trace's first row (it selects the activations), so a trace can be
        replayed in pieces, e.g. around a resize.

        `native`: each step is one moe_decode_step (moe_decode_step_hybrid,
        moe_decode_step_split) call, which makes the same library calls per layer without the
        Python marshalling between them; native=False runs the same calls from this loop.

        `split_launch`: a layer with misses runs its hit experts before waiting for the copies (the
        misses marked as produced elsewhere), then the missed experts after them, then the combine.

        `hybrid` = (cpu_rate, pcie_rate[, copy_too[, host_fixed_s]]) turns on hybrid miss handling:
        each layer's misses are split by the library's rule (moe_hybrid_split); the host runs its
        share (moe_cpu_expert_ffn on the pinned images) while the rest is copied and run on the GPU,
        and the host's rows are copied into y_perm before the combine.  With copy_too (default) the host's misses are also inserted
        and copied after the others, off this layer's critical path (the cache then sees every
        request in full); without it they stay out of the cache.  The number of host-run experts
        is added to self.cpu_experts.

        Returns wall seconds (and outputs [(step, layer, y)] when keep_outputs)."""
        import torch

        steps = steps or trace.shape[0]
        L, E, k = self.L, self.E, self.k
        forced = self._forced(trace[:steps])
        host_idx = self._host_idx
        done = torch.cuda.Event()
        outs = []
        nb = self.x_dec[0].shape[0]
        if native and not (hybrid and split_launch):
            return self._decode_native(forced, steps, first_step, keep_outputs, hybrid, split_launch)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if hybrid or split_launch:
            tabs = [torch.full((E,), -1, dtype=torch.int32, pin_memory=True) for _ in range(2)]
            dtabs = [torch.empty(E, dtype=torch.int32, device=self.device) for _ in range(2)]
        if hybrid:
            from . import cpu_expert_ffn

            dev, d = self.device, self.d
            host_x = torch.empty((1, d), dtype=torch.int16, pin_memory=True)
            host_tab = torch.full((E,), -1, dtype=torch.int32, pin_memory=True)
            dev_tab = torch.empty(E, dtype=torch.int32, device=dev)
            host_y = torch.empty((k, d), dtype=torch.float32, pin_memory=True)
            y_perm_buf = self._buffers(1)["y_perm"]
        with torch.cuda.stream(self.compute):
            for s in range(steps):
                for l in range(L):
                    xb = (first_step + s) % nb
                    x = self.x_dec[l][xb:xb + 1]
                    idx, w, perm = self._layer(l, x, forced[s, l:l + 1])
                    host_idx.copy_(idx, non_blocking=True)
                    if hybrid:
                        host_x.copy_(x.view(torch.int16), non_blocking=True)
                    done.record(self.compute)
                    done.synchronize()  # the ids cross to the host: the cache decides there
                    ids = np.unique(host_idx.numpy())
                    if not hybrid and split_launch:
                        missed = {int(e) for e in ids if self.cache.slot_of(l, int(e)) < 0}
                        slots, _ = self.cache.lookup(l, ids)
                        if not missed:
                            self.cache.fill(self.copy, self.compute)
                            y = self._experts(l, x, w, perm)
                        else:
                            a, b_ = tabs[0].numpy(), tabs[1].numpy()
                            a[:], b_[:] = -1, -1
                            for e, sl in zip(ids, slots):
                                e = int(e)
                                a[e], b_[e] = (-2, sl) if e in missed else (sl, -2)
                            dtabs[0].copy_(tabs[0], non_blocking=True)
                            dtabs[1].copy_(tabs[1], non_blocking=True)
                            # the resident experts run while the misses are copied in
                            self._experts(l, x, w, perm, table=dtabs[0], do_combine=False)
                            self.cache.fill(self.copy, self.compute)
                            y_perm = self._experts(l, x, w, perm, table=dtabs[1], do_combine=False,
                                                   with_shared=False)
                            y = combine(y_perm, w, perm[3], k, self.shared[l] is not None, x.dtype,
                                        y=self._buffers(1)["y"], stream=self.compute)
                    elif not hybrid:
                        self.cache.lookup(l, ids)
                        self.cache.fill(self.copy, self.compute)
                        y = self._experts(l, x, w, perm)
                    else:
                        cpu_rate, pcie_rate, copy_too, fixed_s = _hybrid_args(hybrid)
                        miss = [int(e) for e in ids if self.cache.slot_of(l, int(e)) < 0]
                        n_cpu = hybrid_split(len(miss), cpu_rate, pcie_rate, fixed_s)
                        on_cpu = miss[len(miss) - n_cpu:] if n_cpu else []
                        gpu_ids = [int(e) for e in ids if copy_too or int(e) not in on_cpu]
                        slots, _ = self.cache.lookup(l, gpu_ids)
                        if copy_too:
                            self.cache.fill_split(on_cpu, self.copy, self.compute)
                        else:
                            self.cache.fill(self.copy, self.compute)
                        tab = host_tab.numpy()
                        for e, sl in zip(gpu_ids, slots):
                            tab[e] = sl
                        for e in on_cpu:
                            tab[e] = -2  # rows produced on the host
                        dev_tab.copy_(host_tab, non_blocking=True)
                        self._experts(l, x, w, perm, table=dev_tab, do_combine=False)
                        # the host's experts, while the copies and the GPU experts run
                        rank = {int(e): j for j, e in enumerate(ids)}  # one token: row = rank of the id
                        hy = host_y.numpy()
                        for e in on_cpu:
                            key = l * E + e
                            cpu_expert_ffn(self.pinned[0] + key * self.stride, self.wl.wdt, self.d, self.f,
                                           host_x.numpy().view(np.uint16), y=hy[rank[e]:rank[e] + 1])
                            y_perm_buf[rank[e]:rank[e] + 1].copy_(host_y[rank[e]:rank[e] + 1], non_blocking=True)
                        self.cpu_experts += len(on_cpu)
                        # the combine reads the host rows: it runs once they are in place
                        y = combine(y_perm_buf, w, perm[3], k, self.shared[l] is not None, x.dtype,
                                    y=self._buffers(1)["y"], stream=self.compute)
                    self.cache.mark_read(l, self.compute)
                    if keep_outputs:
                        outs.append((first_step + s, l, y.clone()))
        self.compute.synchronize()
        el = time.perf_counter() - t0
        return (el, outs) if keep_outputs else el

    def _decode_native(self, forced, steps: int, first_step: int, keep_outputs: bool, hybrid=None,
                       split_launch: bool = False):
        """decode() in the plain, hybrid or split-launch mode, one native call per step."""
        import torch
        from . import DECODE_LAYER, decode_step, decode_step_hybrid, decode_step_split

        L, E, k, d = self.L, self.E, self.k, self.d
        nb = self.x_dec[0].shape[0]
        esz = 2 if self.wl.act == "bf16" else 4
        b = self._buffers(1)
        ws = self._workspace(1)
        ys = ([torch.empty_like(b["y"]) for _ in range(L)] if keep_outputs else [b["y"]] * L)
        # every step's layer descriptors, built before the timed loop
        xb = (first_step + np.arange(steps)) % nb
        arr = np.zeros((steps, L), dtype=DECODE_LAYER)
        x0 = np.array([self.x_dec[l].data_ptr() for l in range(L)], dtype=np.uint64)
        arr["x"] = x0[None, :] + (xb[:, None] * d * esz).astype(np.uint64)
        arr["w_router"] = np.array([w.data_ptr() for w in self.w_router], dtype=np.uint64)[None, :]
        arr["bias"] = np.array([0 if bb is None else bb.data_ptr() for bb in self.bias], dtype=np.uint64)[None, :]
        arr["shared_w"] = np.array([0 if sw is None else sw.data_ptr() for sw in self.shared], dtype=np.uint64)[None, :]
        arr["forced"] = forced.data_ptr() + (np.arange(steps * L, dtype=np.uint64) * (k * 4)).reshape(steps, L)
        arr["y"] = np.array([y.data_ptr() for y in ys], dtype=np.uint64)[None, :]
        arr["layer"] = np.arange(L, dtype=np.int32)[None, :]
        outs = []
        if hybrid:
            host_x = torch.empty((1, d), dtype=torch.int16, pin_memory=True)
            host_y = torch.empty((k, d), dtype=torch.float32, pin_memory=True)
            host_tab = torch.full((E,), -1, dtype=torch.int32, pin_memory=True)
            dev_tab = torch.empty(E, dtype=torch.int32, device=self.device)
            cpu_rate, pcie_rate, copy_too, fixed_s = _hybrid_args(hybrid)
        if split_launch:
            host_tabs = torch.full((2, E), -1, dtype=torch.int32, pin_memory=True)
            dev_tabs = torch.empty((2, E), dtype=torch.int32, device=self.device)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(self.compute):
            for s in range(steps):
                if hybrid:
                    self.cpu_experts += decode_step_hybrid(
                        self.cache, arr[s], d, self.f, E, k, self.act_code, self.wl.wdt, self.slot_pool, self.n_slots,
                        self.stride, self.slot_table, b["route"], b["perm"], b["y_perm"], ws, self._host_idx, host_x,
                        host_y, host_tab, dev_tab, cpu_rate, pcie_rate, copy_too, self.compute, self.copy,
                        host_fixed_s=fixed_s)
                elif split_launch:
                    decode_step_split(self.cache, arr[s], 1, d, self.f, E, k, self.act_code, self.wl.wdt,
                                      self.slot_pool, self.n_slots, self.stride, self.slot_table, b["route"], b["perm"],
                                      b["y_perm"], ws, self._host_idx, host_tabs, dev_tabs, self.compute, self.copy)
                else:
                    decode_step(self.cache, arr[s], 1, d, self.f, E, k, self.act_code, self.wl.wdt, self.slot_pool,
                                self.n_slots, self.stride, self.slot_table, b["route"], b["perm"], b["y_perm"], ws,
                                self._host_idx, self.compute, self.copy)
                if keep_outputs:
                    outs += [(first_step + s, l, ys[l].clone()) for l in range(L)]
        self.compute.synchronize()
        el = time.perf_counter() - t0
        return (el, outs) if keep_outputs else el

    def _forced(self, trace):
        """The routing trace on the device (its buffer is reused between calls of the same length)."""
        import torch

        t = np.ascontiguousarray(trace, dtype=np.int32)
        key = ("forced",) + t.shape
        if key not in self._bufs:
            self._bufs[key] = torch.empty(t.shape, dtype=torch.int32, device=self.device)
        buf = self._bufs[key]
        buf.copy_(torch.from_numpy(t))
        return buf

    def close(self):
        import torch

        if getattr(self, "cache", None) is not None:
            torch.cuda.synchronize()
            self.cache.close()
            self.cache = None
        if getattr(self, "pinned", None):
            self._free_pinned()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def pinned_h2d_GBps(nbytes: int = 1 << 29, reps: int = 4) -> float:
    """Plain pinned host -> device copy rate, the ceiling the cache fills are compared with."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    return nbytes * reps / (time.perf_counter() - t0) / 1e9


def host_expert_rate(stack, reps: int = 5) -> float:
    """Expert images per second the host kernel runs for one token (threads: the whole pool)."""
    from . import cpu_expert_ffn

    x = np.zeros((1, stack.d), dtype=np.uint16)
    x[0, ::7] = 0x3F80  # some ones
    cpu_expert_ffn(stack.pinned[0], stack.wl.wdt, stack.d, stack.f, x)
    t0 = time.perf_counter()
    for i in range(reps):
        cpu_expert_ffn(stack.pinned[0] + i * stack.stride, stack.wl.wdt, stack.d, stack.f, x)
    return reps / (time.perf_counter() - t0)


def hybrid_rates(wl, seed: int = 0, n: int = 8, reps: int = 20, device="cuda") -> dict:
    """The inputs of the hybrid split, measured on this machine (FreeToken RTX 5090 page, miss split:
    host and PCIe bandwidths are to be measured on the actual computer).

    Both paths read host memory, so each rate is measured while the other path is busy: `n` slot
    images copied pinned -> device on one stream while the host kernel runs `n` other pinned slot
    images.  The fixed host-path cost is the round trip a layer pays once the host takes any expert:
    the activation row to the host and one output row back, each waited for (averaged over `reps`).
    Runs before the stack's pool is pinned, on buffers of its own (freed on return).
    -> dict(cpu_rate, pcie_rate (expert images per second, under contention), host_fixed_s, and the
    two rates measured alone)."""
    import torch
    import synth
    from . import cpu_expert_ffn

    d, f = wl.d, wl.f
    stride = slot_bytes(d, f, wl.wdt)
    img = pack_expert(wl.wdt, d, f, *_expert_arrays(synth.expert_weights(wl, seed, 0, 0)))
    src = torch.empty((n, stride), dtype=torch.uint8, pin_memory=True)       # what the copies read
    host = torch.empty((n, stride), dtype=torch.uint8, pin_memory=True)      # what the host kernel reads
    src.numpy()[:] = img
    host.numpy()[:] = img
    dst = torch.empty((n, stride), dtype=torch.uint8, device=device)
    st = torch.cuda.Stream(device=device)
    x = np.zeros((1, d), dtype=np.uint16)
    x[0, ::7] = 0x3F80
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hbase = host.data_ptr()

    def copies():
        with torch.cuda.stream(st):
            e0.record(st)
            for i in range(n):
                dst[i].copy_(src[i], non_blocking=True)
            e1.record(st)

    def run_host():
        t0 = time.perf_counter()
        for i in range(n):
            cpu_expert_ffn(hbase + i * stride, wl.wdt, d, f, x)
        return time.perf_counter() - t0

    run_host()  # warm the host threads and pages
    copies()
    e1.synchronize()
    copies()
    e1.synchronize()
    pcie_alone = n / (e0.elapsed_time(e1) * 1e-3)
    cpu_alone = n / run_host()
    copies()
    t_host = run_host()
    e1.synchronize()
    pcie_busy = n / (e0.elapsed_time(e1) * 1e-3)
    cpu_busy = n / t_host
    # fixed cost of the host path: activation row down, an output row up, each waited for
    hx = torch.empty((1, d), dtype=torch.int16, pin_memory=True)
    hy = torch.zeros((1, d), dtype=torch.float32, pin_memory=True)
    xd = torch.zeros((1, d), dtype=torch.int16, device=device)
    yd = torch.empty((1, d), dtype=torch.float32, device=device)
    ev = torch.cuda.Event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(st):
        for _ in range(reps):
            hx.copy_(xd, non_blocking=True)
            ev.record(st)
            ev.synchronize()
            yd.copy_(hy, non_blocking=True)
            ev.record(st)
            ev.synchronize()
    fixed = (time.perf_counter() - t0) / reps
    torch.cuda.synchronize()
    del src, host, dst, hx, hy, xd, yd
    torch.cuda.empty_cache()
    return dict(cpu_rate=cpu_busy, pcie_rate=pcie_busy, host_fixed_s=fixed, cpu_rate_alone=cpu_alone,
                pcie_rate_alone=pcie_alone)


def run_trace(wl, layers: int, capacity_fracs=(0.40, 0.58), steps: int = 2048, prefill_tokens: int = 2048,
              seed: int = 0, n_images: Optional[int] = None, log=None, min_layers: Optional[int] = 12):
    """The offload workload: a prefill of `prefill_tokens`, then a `steps`-step batch-1 decode over a
    seeded routing trace, once per cache capacity (fraction of all L*E routed experts).  When the
    host cannot pin L layers, `min_layers` layers run instead (and the capacities scale with them).

    Returns a dict of the measured figures per capacity (tokens/s, miss rates, H2D traffic)."""
    import torch
    import synth

    log = log or (lambda *a: None)
    pcie = pinned_h2d_GBps()  # before the pool is pinned
    hr = hybrid_rates(wl, seed)
    n_caps = [int(round(fr * layers * wl.E)) for fr in capacity_fracs]
    stack = OffloadStack(wl, layers, max(n_caps), seed=seed, n_images=n_images, prefill_tokens=prefill_tokens,
                         log=log, min_layers=min_layers)
    requested, layers = layers, stack.L
    trace = synth.routing_trace(seed, steps, layers, wl.E, wl.k)
    caps = [int(round(fr * layers * wl.E)) for fr in capacity_fracs]
    out = {"layers": layers, "layers_requested": requested, "experts_per_layer": wl.E, "slot_bytes": stack.stride,
           "pool_GiB": stack.pool_bytes / 2**30, "steps": steps, "prefill_tokens": prefill_tokens,
           "pcie_h2d_GBps": pcie, "host_expert_GBps": hr["cpu_rate_alone"] * stack.stride / 1e9,
           "hybrid_split_inputs": {"host_GBps_while_copying": hr["cpu_rate"] * stack.stride / 1e9,
                                   "pcie_GBps_while_host_runs": hr["pcie_rate"] * stack.stride / 1e9,
                                   "host_GBps_alone": hr["cpu_rate_alone"] * stack.stride / 1e9,
                                   "pcie_GBps_alone": hr["pcie_rate_alone"] * stack.stride / 1e9,
                                   "host_fixed_us": hr["host_fixed_s"] * 1e6},
           "runs": []}
    # the host's share is also copied in, after the layer's own copies (the cache sees every request
    # in full); the variant that keeps it out of the cache (direct CPU execution only) is measured
    # beside it
    rates = (hr["cpu_rate"], hr["pcie_rate"], True, hr["host_fixed_s"])
    try:
        for fr, C in zip(capacity_fracs, caps):
            stack.new_cache(C)
            t_pre = stack.prefill()
            st0 = stack.cache.stats()
            t_dec = stack.decode(trace)
            st = stack.cache.stats()
            dec_bytes = st["bytes_h2d"] - st0["bytes_h2d"]
            r = {"capacity_frac": fr, "slots": C,
                 "prefill_s": t_pre, "prefill_tokens_per_s": prefill_tokens / t_pre,
                 "prefill_miss_rate": st["pre_miss"] / max(1, st["pre_acc"]),
                 "prefill_h2d_GBps": st0["bytes_h2d"] / t_pre / 1e9,
                 "decode_s": t_dec, "decode_tokens_per_s": steps / t_dec,
                 "decode_miss_rate": st["dec_miss"] / max(1, st["dec_acc"]),
                 "decode_h2d_GBps": dec_bytes / t_dec / 1e9,
                 "decode_h2d_MB_per_token": dec_bytes / steps / 1e6}
            # the same trace through the per-layer Python loop (the loop hybrid and split use)
            stack.new_cache(C)
            stack.prefill()
            r["python_loop_decode_tokens_per_s"] = steps / stack.decode(trace, native=False)
            # the same trace with hybrid miss handling: the host runs part of each layer's misses
            stack.new_cache(C)
            stack.prefill()
            stack.cpu_experts = 0
            t_hyb = stack.decode(trace, hybrid=rates)
            sth = stack.cache.stats()
            r["hybrid_decode_tokens_per_s"] = steps / t_hyb
            r["hybrid_gpu_miss_rate"] = sth["dec_miss"] / max(1, sth["dec_acc"] + stack.cpu_experts)
            r["hybrid_host_experts_per_token"] = stack.cpu_experts / steps
            # the same split with the host's misses kept out of the cache (run on the host each time)
            stack.new_cache(C)
            stack.prefill()
            stack.cpu_experts = 0
            r["hybrid_uncached_decode_tokens_per_s"] = steps / stack.decode(trace, hybrid=rates[:2] + (False,) + rates[3:])
            r["hybrid_uncached_host_experts_per_token"] = stack.cpu_experts / steps
            # the same trace with split launches: resident experts overlap the miss copies
            stack.new_cache(C)
            stack.prefill()
            r["split_decode_tokens_per_s"] = steps / stack.decode(trace, split_launch=True)
            log(f"capacity {fr:.0%} ({C} slots): " + ", ".join(f"{k}={v:.4g}" for k, v in r.items()
                                                              if isinstance(v, float)))
            out["runs"].append(r)
        if len(caps) >= 2:
            # elastic capacity: start at the largest cache, shrink to the next one half way
            hi, lo = sorted(caps)[-1], sorted(caps)[-2]
            stack.new_cache(hi)
            stack.prefill()
            half = steps // 2
            t1 = stack.decode(trace[:half])
            n_log = len(stack.cache.copy_log())
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            stack.resize(lo)
            torch.cuda.synchronize()
            t_resize = time.perf_counter() - t0
            moves = int((stack.cache.copy_log()[n_log:, 2] <= -2).sum())
            st0 = stack.cache.stats()
            t2 = stack.decode(trace[half:], first_step=half)
            st = stack.cache.stats()
            out["elastic"] = {"from_slots": hi, "to_slots": lo, "at_step": half, "resize_ms": t_resize * 1e3,
                              "moved_slots": moves, "decode_tokens_per_s_before": half / t1,
                              "decode_tokens_per_s_after": (steps - half) / t2,
                              "decode_miss_rate_after": (st["dec_miss"] - st0["dec_miss"]) /
                                                        max(1, st["dec_acc"] - st0["dec_acc"])}
            log("elastic: " + ", ".join(f"{k}={v:.4g}" for k, v in out["elastic"].items()))
    finally:
        stack.close()
        torch.cuda.empty_cache()
    return out
