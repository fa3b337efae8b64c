"""Routed-expert MoE layer behind an HBM expert-slot cache, on MI355X (gfx950).

Thin Python binding of libmoe (include/moe.h): argument marshalling only.  Every step
of the layer runs in the library's HIP kernels; device memory and streams come from
PyTorch.  There is no CPU fallback: calls fail when libmoe.so is missing.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from ._lib import (MOE_BF16, MOE_F32, MOE_INT4_G128, MoeError, check, lib)

__all__ = ["route", "permute", "permute_workspace", "permute_workspace_bytes", "route_permute", "expert_ffn_grouped", "expert_ffn_grouped_noalloc", "combine",
           "slot_bytes", "pack_expert", "workspace_bytes", "hybrid_split", "SlotCache", "pinned_alloc", "pinned_free", "profile_enable",
           "profile_collect", "profile_results", "profile_reset", "MoeError", "WDT", "lib"]

WDT = {"f32": MOE_F32, "bf16": MOE_BF16, "int4": MOE_INT4_G128}


def _torch():
    import torch

    return torch


def _act(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {t.dtype}")


def _y_code(t) -> int:
    """Element type code of a y_perm tensor (float32 or bfloat16)."""
    torch = _torch()
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"y_perm must be float32 or bfloat16, got {t.dtype}")


def y_perm_dtype(act_dtype, T: int):
    """The y_perm element type the layer orchestration uses: bfloat16 for bf16 prefill (more than 64
    tokens, the matrix-core path), where the intermediate rows may be bf16; float32 otherwise."""
    torch = _torch()
    return torch.bfloat16 if act_dtype == torch.bfloat16 and T > 64 else torch.float32


def _p(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _s(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors passed to libmoe must be contiguous")


# ---------------------------------------------------------------------------------------------
# hot-path calls
# ---------------------------------------------------------------------------------------------
def route(x, w_router, bias, k: int, forced_idx=None, out=None, stream=None):
    """-> (topk_idx int32 [T,k], topk_w f32 [T,k], logits f32 [T,E])."""
    torch = _torch()
    _contig(x, w_router, bias, forced_idx)
    T, d = x.shape
    E = w_router.shape[0]
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=x.device),
               torch.empty((T, k), dtype=torch.float32, device=x.device),
               torch.empty((T, E), dtype=torch.float32, device=x.device))
    idx, w, logits = out
    check(lib().moe_route(_p(x), _act(x), T, d, _p(w_router), _p(bias), E, k, _p(forced_idx), _p(idx), _p(w),
                          _p(logits), _s(stream)))
    return idx, w, logits


def permute_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(lib().moe_permute_workspace_bytes(T, k, E))


def permute_workspace(T: int, k: int, E: int, device):
    """Device scratch for a split sort of T*k pairs (None when one workgroup sorts)."""
    n = permute_workspace_bytes(T, k, E)
    return _torch().empty(n, dtype=_torch().uint8, device=device) if n else None


def permute(topk_idx, E: int, out=None, stream=None, ws=None):
    """-> (counts [E], offsets [E+1], perm [T*k], inv_perm [T*k]) int32.  ws: permute_workspace or None."""
    torch = _torch()
    _contig(topk_idx)
    T, k = topk_idx.shape
    if out is None:
        dev = topk_idx.device
        out = (torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev), torch.empty(T * k, dtype=torch.int32, device=dev))
    c, o, p, ip = out
    check(lib().moe_permute(_p(topk_idx), T, k, E, _p(c), _p(o), _p(p), _p(ip), _p(ws),
                            0 if ws is None else ws.numel(), _s(stream)))
    return c, o, p, ip


def route_permute(x, w_router, bias, k: int, forced_idx=None, out=None, stream=None, ws=None):
    """route then permute as one call -> (topk_idx, topk_w, logits, counts, offsets, perm, inv_perm).
    ws: permute_workspace(T, k, E) or None (then a large batch sorts in one workgroup)."""
    torch = _torch()
    _contig(x, w_router, bias, forced_idx)
    T, d = x.shape
    E = w_router.shape[0]
    if out is None:
        dev = x.device
        out = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((T, E), dtype=torch.float32, device=dev), torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev), torch.empty(T * k, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev))
    idx, w, logits, c, o, p, ip = out
    check(lib().moe_route_permute(_p(x), _act(x), T, d, _p(w_router), _p(bias), E, k, _p(forced_idx), _p(idx),
                                  _p(w), _p(logits), _p(c), _p(o), _p(p), _p(ip), _p(ws),
                                  0 if ws is None else ws.numel(), _s(stream)))
    return out


def workspace_bytes(T, d, f, E, k, has_shared, act: int, wdt: int) -> int:
    return int(lib().moe_workspace_bytes(T, d, f, E, k, int(bool(has_shared)), act, wdt))


def expert_ffn_grouped(x, perm, offsets, counts, slot_of_expert, slot_pool, n_slots: int, slot_stride: int,
                       wdt: str, f: int, k: int, shared_w=None, y_perm=None, ws=None, stream=None, y_dtype=None):
    """Grouped SwiGLU experts through the slot table. -> (y_perm [T*k (+T), d], ws).  y_perm's element
    type is that of the given tensor (float32, or bfloat16 with bf16 activations), else y_dtype
    (a torch dtype, default float32)."""
    torch = _torch()
    _contig(x, perm, offsets, counts, slot_of_expert)
    T, d = x.shape
    E = counts.shape[0]
    act = _act(x)
    rows = T * k + (T if shared_w is not None else 0)
    if y_perm is None:
        y_perm = torch.empty((rows, d), dtype=y_dtype or torch.float32, device=x.device)
    if ws is None:
        need = workspace_bytes(T, d, f, E, k, shared_w is not None, act, WDT[wdt])
        ws = torch.zeros(need, dtype=torch.uint8, device=x.device)
    check(lib().moe_expert_ffn_grouped(_p(x), act, T, d, f, E, k, _p(perm), _p(offsets), _p(counts),
                                       _p(slot_of_expert), n_slots, _p(slot_pool), slot_stride, WDT[wdt],
                                       _p(shared_w), _p(y_perm), _y_code(y_perm), _p(ws), ws.numel(), _s(stream)))
    return y_perm, ws


def expert_ffn_grouped_noalloc(x, perm, offsets, counts, slot_of_expert, slot_pool, n_slots: int,
                               slot_stride: int, wdt: str, f: int, k: int, y_perm, shared_w=None, status=None,
                               stream=None):
    """expert_ffn_grouped through moe_expert_ffn_grouped_noalloc: no workspace, the library's
    per-GPU scratch instead; y_perm must be given.  status: device int32 tensor or None."""
    _contig(x, perm, offsets, counts, slot_of_expert, y_perm)
    T, d = x.shape
    E = counts.shape[0]
    check(lib().moe_expert_ffn_grouped_noalloc(_p(x), _act(x), T, d, f, E, k, _p(perm), _p(offsets), _p(counts),
                                               _p(slot_of_expert), n_slots, _p(slot_pool), slot_stride, WDT[wdt],
                                               _p(shared_w), _p(y_perm), _y_code(y_perm), _p(status), _s(stream)))
    return y_perm


def combine(y_perm, topk_w, inv_perm, k: int, has_shared: bool, out_dtype, y=None, stream=None):
    torch = _torch()
    _contig(y_perm, topk_w, inv_perm)
    T = topk_w.shape[0]
    d = y_perm.shape[1]
    if y is None:
        y = torch.empty((T, d), dtype=out_dtype, device=y_perm.device)
    code = MOE_BF16 if y.dtype == torch.bfloat16 else MOE_F32
    check(lib().moe_combine(_p(y_perm), _y_code(y_perm), _p(topk_w), _p(inv_perm), T, k, d, int(bool(has_shared)),
                            _p(y), code, _s(stream)))
    return y


# ---------------------------------------------------------------------------------------------
# slots
# ---------------------------------------------------------------------------------------------
def slot_bytes(d: int, f: int, wdt: str) -> int:
    return int(lib().moe_slot_bytes(d, f, WDT[wdt]))


def _np_ptr(a):
    return None if a is None else np.ascontiguousarray(a).ctypes.data


def pack_expert(wdt: str, d: int, f: int, wg, wu, wd, sg=None, su=None, sd=None, out=None) -> np.ndarray:
    """Canonical expert weights (numpy) -> slot image (numpy uint8, or written into ``out``)."""
    n = slot_bytes(d, f, wdt)
    if n == 0:
        raise MoeError(-2, f"unsupported slot shape d={d} f={f} {wdt}")
    if out is None:
        out = np.empty(n, dtype=np.uint8)
    arrs = [np.ascontiguousarray(a) if a is not None else None for a in (wg, wu, wd, sg, su, sd)]
    optr = out.ctypes.data if isinstance(out, np.ndarray) else int(out)
    check(lib().moe_pack_expert(WDT[wdt], d, f, *[_np_ptr(a) for a in arrs], optr))
    return out


def cpu_expert_ffn(slot_image, wdt: str, d: int, f: int, x_bf16: np.ndarray, y: Optional[np.ndarray] = None,
                   threads: int = 0) -> np.ndarray:
    """One expert on the host from its packed slot image (numpy uint8 array or a host address).
    x_bf16: bf16 bits (uint16) [n, d].  -> y float32 [n, d]."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    n = x.shape[0]
    if y is None:
        y = np.empty((n, d), dtype=np.float32)
    img = slot_image.ctypes.data if isinstance(slot_image, np.ndarray) else int(slot_image)
    check(lib().moe_cpu_expert_ffn(img, WDT[wdt], d, f, x.ctypes.data, n, y.ctypes.data, threads))
    return y


# moe_decode_layer (include/moe.h): six pointers, then layer and a reserved int32
DECODE_LAYER = np.dtype([("x", "<u8"), ("w_router", "<u8"), ("bias", "<u8"), ("forced", "<u8"),
                         ("shared_w", "<u8"), ("y", "<u8"), ("layer", "<i4"), ("reserved", "<i4")])


def _f32_rows(y_perm, fn: str):
    """The decode steps keep y_perm in binary32 (their C signature takes float rows)."""
    if _y_code(y_perm) != MOE_F32:
        raise TypeError(f"{fn}: y_perm must be float32, got {y_perm.dtype}")


def decode_step(cache, layers: np.ndarray, T: int, d: int, f: int, E: int, k: int, act: int, wdt: str, slot_pool,
                n_slots: int, slot_stride: int, slot_table, route_bufs, perm_bufs, y_perm, ws, host_idx, compute,
                copy):
    """One decode step of every layer in `layers` (a DECODE_LAYER array) through moe_decode_step."""
    _f32_rows(y_perm, "decode_step")
    idx, w, logits = route_bufs
    c, o, p, ip = perm_bufs
    check(lib().moe_decode_step(cache.h, len(layers), layers.ctypes.data, T, d, f, E, k, act, WDT[wdt],
                                _p(slot_pool), n_slots, slot_stride, _p(slot_table), _p(idx), _p(w), _p(logits),
                                _p(c), _p(o), _p(p), _p(ip), _p(y_perm), _p(ws), ws.numel(), host_idx.data_ptr(),
                                _s(compute), _s(copy)))



def decode_step_split(cache, layers: np.ndarray, T: int, d: int, f: int, E: int, k: int, act: int, wdt: str,
                      slot_pool, n_slots: int, slot_stride: int, slot_table, route_bufs, perm_bufs, y_perm, ws,
                      host_idx, host_tables, dev_tables, compute, copy):
    """One decode step of every layer in `layers` with split launches (moe_decode_step_split).
    host_tables: pinned int32 [2, E]; dev_tables: device int32 [2, E]."""
    _f32_rows(y_perm, "decode_step_split")
    idx, w, logits = route_bufs
    c, o, p, ip = perm_bufs
    check(lib().moe_decode_step_split(cache.h, len(layers), layers.ctypes.data, T, d, f, E, k, act, WDT[wdt],
                                      _p(slot_pool), n_slots, slot_stride, _p(slot_table), _p(idx), _p(w),
                                      _p(logits), _p(c), _p(o), _p(p), _p(ip), _p(y_perm), _p(ws), ws.numel(),
                                      host_idx.data_ptr(), host_tables.data_ptr(), _p(dev_tables), _s(compute),
                                      _s(copy)))

def decode_step_hybrid(cache, layers: np.ndarray, d: int, f: int, E: int, k: int, act: int, wdt: str, slot_pool,
                       n_slots: int, slot_stride: int, slot_table, route_bufs, perm_bufs, y_perm, ws, host_idx,
                       host_x, host_y, host_table, dev_table, cpu_rate: float, pcie_rate: float, copy_too: bool,
                       compute, copy, cpu_threads: int = 0, host_fixed_s: float = 0.0) -> int:
    """One batch-1 decode step of every layer in `layers` with hybrid miss handling
    (moe_decode_step_hybrid).  host_idx/host_x/host_y/host_table: pinned host tensors; dev_table:
    device int32 [E].  -> number of experts run on the host."""
    _f32_rows(y_perm, "decode_step_hybrid")
    idx, w, logits = route_bufs
    c, o, p, ip = perm_bufs
    n_cpu = ctypes.c_int64(0)
    check(lib().moe_decode_step_hybrid(cache.h, len(layers), layers.ctypes.data, d, f, E, k, act, WDT[wdt],
                                       _p(slot_pool), n_slots, slot_stride, _p(slot_table), _p(idx), _p(w),
                                       _p(logits), _p(c), _p(o), _p(p), _p(ip), _p(y_perm), _p(ws), ws.numel(),
                                       host_idx.data_ptr(), host_x.data_ptr(), host_y.data_ptr(),
                                       host_table.data_ptr(), _p(dev_table), float(cpu_rate), float(pcie_rate),
                                       float(host_fixed_s), int(bool(copy_too)), cpu_threads, ctypes.byref(n_cpu),
                                       _s(compute), _s(copy)))
    return n_cpu.value


def hybrid_split(m: int, cpu_rate: float, pcie_rate: float, host_fixed_s: float = 0.0) -> int:
    """Misses of a layer the host runs (moe_hybrid_split): of m misses, the n minimising
    max((m - n) / pcie_rate, host_fixed_s + n / cpu_rate) (m / pcie_rate for n = 0), ties to fewer."""
    n = ctypes.c_int32()
    check(lib().moe_hybrid_split(int(m), float(cpu_rate), float(pcie_rate), float(host_fixed_s), ctypes.byref(n)))
    return n.value

# ---------------------------------------------------------------------------------------------
# expert-slot cache
# ---------------------------------------------------------------------------------------------
class SlotCache:
    """LRU expert-slot cache shared by all layers (wraps moe_cache_*)."""

    def __init__(self, L: int, E: int, n_slots: int, slot_stride: int = 0, slot_pool=None, slot_table=None,
                 host_ptrs=None):
        self.L, self.E, self.C = L, E, n_slots
        self._host = None
        hp = None
        if host_ptrs is not None:
            self._host = (ctypes.c_void_p * (L * E))(*[int(p) for p in host_ptrs])
            hp = ctypes.cast(self._host, ctypes.c_void_p)
        h = ctypes.c_void_p()
        check(lib().moe_cache_create(L, E, n_slots, slot_stride, _p(slot_pool), _p(slot_table), hp,
                                     ctypes.byref(h)))
        self.h = h

    def lookup(self, layer: int, ids):
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        slots = np.empty(len(ids), dtype=np.int32)
        nm = ctypes.c_int32()
        check(lib().moe_cache_lookup(self.h, layer, ids.ctypes.data, len(ids), slots.ctypes.data, ctypes.byref(nm)))
        return slots, nm.value

    def fill(self, copy_stream=None, compute_stream=None):
        check(lib().moe_cache_fill(self.h, _s(copy_stream), _s(compute_stream)))

    def fill_split(self, later, copy_stream=None, compute_stream=None):
        """fill(), with the copies of the experts in `later` deferred (compute does not wait)."""
        ids = np.ascontiguousarray(np.asarray(later, dtype=np.int32))
        check(lib().moe_cache_fill_split(self.h, ids.ctypes.data if len(ids) else None, len(ids),
                                         _s(copy_stream), _s(compute_stream)))

    def policy_fill_split(self, later):
        ids = np.ascontiguousarray(np.asarray(later, dtype=np.int32))
        check(lib().moe_cache_fill_split(self.h, ids.ctypes.data if len(ids) else None, len(ids), None, None))

    def prefetch_layer(self, layer: int, copy_stream=None, compute_stream=None):
        check(lib().moe_cache_prefetch_layer(self.h, layer, _s(copy_stream), _s(compute_stream)))

    def mark_read(self, layer: int, compute_stream=None):
        check(lib().moe_cache_mark_read(self.h, layer, _s(compute_stream)))

    def resize(self, n_slots: int, copy_stream=None, compute_stream=None):
        """Change the capacity at a safe point (every layer marked read, no fill pending)."""
        check(lib().moe_cache_resize(self.h, n_slots, _s(copy_stream), _s(compute_stream)))
        self.C = n_slots

    def policy_resize(self, n_slots: int):
        """resize() of a policy-only cache (no streams involved)."""
        check(lib().moe_cache_resize(self.h, n_slots, None, None))
        self.C = n_slots

    def policy_fill(self):
        """fill() of a policy-only cache (no streams involved)."""
        check(lib().moe_cache_fill(self.h, None, None))

    def policy_prefetch(self, layer: int):
        """prefetch_layer() of a policy-only cache (no streams involved)."""
        check(lib().moe_cache_prefetch_layer(self.h, layer, None, None))

    def policy_mark_read(self, layer: int):
        check(lib().moe_cache_mark_read(self.h, layer, None))

    def stats(self):
        out = np.zeros(6, dtype=np.int64)
        check(lib().moe_cache_stats(self.h, out.ctypes.data))
        keys = ("dec_acc", "dec_hit", "dec_miss", "pre_acc", "pre_miss", "bytes_h2d")
        return dict(zip(keys, (int(v) for v in out)))

    def trace(self):
        n = ctypes.c_int64()
        check(lib().moe_cache_trace(self.h, None, 0, ctypes.byref(n)))
        buf = np.empty(n.value, dtype=np.uint8)
        if n.value:
            check(lib().moe_cache_trace(self.h, buf.ctypes.data, n.value, ctypes.byref(n)))
        return buf

    def copy_log(self):
        n = ctypes.c_int64()
        check(lib().moe_cache_copy_log(self.h, None, 0, ctypes.byref(n)))
        buf = np.empty((n.value, 3), dtype=np.int64)
        if n.value:
            check(lib().moe_cache_copy_log(self.h, buf.ctypes.data, n.value, ctypes.byref(n)))
        return buf

    def inject_copy_failures(self, n: int):
        check(lib().moe_cache_inject_copy_failures(self.h, n))

    def slot_of(self, layer: int, expert: int) -> int:
        s = ctypes.c_int32()
        check(lib().moe_cache_slot_of(self.h, layer, expert, ctypes.byref(s)))
        return s.value

    def close(self):
        if self.h:
            lib().moe_cache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def pinned_alloc(nbytes: int) -> int:
    p = ctypes.c_void_p()
    check(lib().moe_pinned_alloc(nbytes, ctypes.byref(p)))
    return p.value


def pinned_free(ptr: int):
    lib().moe_pinned_free(ptr)


# ---------------------------------------------------------------------------------------------
# kernel timing
# ---------------------------------------------------------------------------------------------
def profile_enable(on: bool = True):
    lib().moe_profile_enable(int(on))


def profile_collect():
    check(lib().moe_profile_collect())


def profile_results() -> dict:
    """{kernel name: (total ms, launches)} accumulated since the last reset."""
    out = {}
    i = 0
    name = ctypes.create_string_buffer(128)
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    while lib().moe_profile_get(i, name, 128, ctypes.byref(ms), ctypes.byref(n)) == 0:
        out[name.value.decode()] = (ms.value, n.value)
        i += 1
    return out


def profile_reset():
    lib().moe_profile_reset()
