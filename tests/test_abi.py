"""The C-ABI library: it loads, exports every declared symbol, rejects bad arguments on the host,
and packs experts into the slot layout the header documents.  No GPU needed."""
import ctypes
import inspect
import os
import re

import numpy as np
import pytest

import synth
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def moe():
    import expert_offload_cache_amd as m
    from expert_offload_cache_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        from expert_offload_cache_amd import build as b

        b.build()
    return m


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(moe):
    names = declared_symbols()
    assert len(names) >= 25
    lib = ctypes.CDLL(moe._lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    # and the binding declares each one
    assert set(names) == set(moe._lib.SIGNATURES)


def test_version_and_slot_sizes(moe):
    assert b"gfx950" in moe.lib().moe_version()
    # 3*d*f elements; int4: 1.5 d f bytes + bf16 scale per 128 inputs (3 d f / 64 bytes)
    assert moe.slot_bytes(64, 128, "f32") == 3 * 64 * 128 * 4 == 98304
    assert moe.slot_bytes(2048, 768, "bf16") == 9437184
    assert moe.slot_bytes(4096, 2048, "bf16") == 50331648
    assert moe.slot_bytes(4096, 2048, "int4") == 12976128
    assert moe.slot_bytes(100, 128, "bf16") == 0
    assert moe.slot_bytes(4096, 2000, "int4") == 0


def test_host_validation_needs_no_gpu(moe):
    L = moe.lib()
    vp = ctypes.c_void_p(16)
    # bad shapes / dtypes are refused before anything touches a device
    assert L.moe_route(vp, 1, 4, 100, vp, None, 8, 2, None, vp, vp, vp, None) == moe._lib.MOE_ESHAPE
    assert L.moe_route(vp, 1, 4, 128, vp, None, 8, 9, None, vp, vp, vp, None) == moe._lib.MOE_ESHAPE
    assert L.moe_route(vp, 7, 4, 128, vp, None, 8, 2, None, vp, vp, vp, None) == moe._lib.MOE_EDTYPE
    assert L.moe_route(None, 1, 4, 128, vp, None, 8, 2, None, vp, vp, vp, None) == moe._lib.MOE_EINVAL
    assert b"NULL" in L.moe_last_error()
    assert L.moe_permute(vp, 4, 2, 2000, vp, vp, vp, vp, None, 0, None) == moe._lib.MOE_ESHAPE
    # prefill experts with few tokens run on the decode kernels: a threshold per weight type
    assert 0 <= L.moe_prefill_gemv_tokens(2) < 1000 and L.moe_prefill_gemv_tokens(0) == 0
    # the split sort's scratch: none for few pairs, one int32 per (workgroup, expert) for many
    assert L.moe_permute_workspace_bytes(64, 8, 128) == 0
    assert L.moe_permute_workspace_bytes(8192, 6, 256) == 24 * 256 * 4
    assert L.moe_permute_workspace_bytes(8192, 6, 2000) == 0
    # route + permute in one call: the route checks, then the permute buffers
    rp = L.moe_route_permute
    assert rp(vp, 1, -1, 128, vp, None, 8, 2, None, vp, vp, vp, vp, vp, vp, vp, None, 0, None) == moe._lib.MOE_ESHAPE
    assert rp(vp, 1, 4, 100, vp, None, 8, 2, None, vp, vp, vp, vp, vp, vp, vp, None, 0, None) == moe._lib.MOE_ESHAPE
    assert rp(vp, 1, 4, 128, vp, None, 8, 9, None, vp, vp, vp, vp, vp, vp, vp, None, 0, None) == moe._lib.MOE_ESHAPE
    assert rp(vp, 7, 4, 128, vp, None, 8, 2, None, vp, vp, vp, vp, vp, vp, vp, None, 0, None) == moe._lib.MOE_EDTYPE
    assert rp(vp, 1, 4, 128, None, None, 8, 2, None, vp, vp, vp, vp, vp, vp, vp, None, 0, None) == moe._lib.MOE_EINVAL
    assert rp(vp, 1, 4, 128, vp, None, 8, 2, None, vp, vp, vp, vp, vp, None, vp, None, 0, None) == moe._lib.MOE_EINVAL
    assert b"moe_route_permute" in L.moe_last_error()
    assert rp(vp, 1, 4, 128, vp, None, 8, 2, None, vp, vp, vp, vp, vp, vp, None, None, 0, None) == moe._lib.MOE_EINVAL
    assert rp(vp, 1, 0, 128, vp, None, 2000, 2, None, vp, vp, vp, vp, vp, vp, vp, None, 0, None) == moe._lib.MOE_ESHAPE
    assert L.moe_combine(vp, 0, vp, vp, 4, 2, 6, 0, vp, 1, None) == moe._lib.MOE_ESHAPE
    # y_perm element type: F32 or BF16 only
    assert L.moe_combine(vp, 2, vp, vp, 4, 2, 8, 0, vp, 1, None) == moe._lib.MOE_EDTYPE
    a = ctypes.c_void_p(256)
    # int4 weights need bf16 activations; dense weights must match the activation dtype
    assert L.moe_expert_ffn_grouped(a, 0, 4, 2048, 768, 128, 8, a, a, a, a, 128, a, 9437184, 2, None, a, 0,
                                    a, 1 << 30, None) == moe._lib.MOE_EDTYPE
    assert L.moe_expert_ffn_grouped(a, 0, 4, 2048, 768, 128, 8, a, a, a, a, 128, a, 9437184, 1, None, a, 0,
                                    a, 1 << 30, None) == moe._lib.MOE_EDTYPE
    # bf16 y_perm needs bf16 activations; other y_perm types are refused
    assert L.moe_expert_ffn_grouped(a, 0, 4, 2048, 768, 128, 8, a, a, a, a, 128, a, 9437184 * 2, 0, None, a, 1,
                                    a, 1 << 30, None) == moe._lib.MOE_EDTYPE
    assert L.moe_expert_ffn_grouped(a, 1, 4, 2048, 768, 128, 8, a, a, a, a, 128, a, 9437184, 1, None, a, 2,
                                    a, 1 << 30, None) == moe._lib.MOE_EDTYPE
    # stride smaller than a slot
    assert L.moe_expert_ffn_grouped(a, 1, 4, 2048, 768, 128, 8, a, a, a, a, 128, a, 4096, 1, None, a, 0,
                                    a, 1 << 30, None) == moe._lib.MOE_EINVAL
    # T == 0 is a no-op
    assert L.moe_route(None, 1, 0, 128, None, None, 8, 2, None, None, None, None, None) == 0
    # workspace too small
    ws_need = moe.workspace_bytes(4, 2048, 768, 128, 8, False, 1, 1)
    assert L.moe_expert_ffn_grouped(ctypes.c_void_p(256), 1, 4, 2048, 768, 128, 8, vp, vp, vp, vp, 128,
                                    ctypes.c_void_p(256), 9437184, 1, None, ctypes.c_void_p(256), 1,
                                    ctypes.c_void_p(256), ws_need - 1, None) == moe._lib.MOE_ENOMEM
    # the decode step checks its arguments before any call: no cache, no layers, bad shapes
    # (after slot_table: topk_idx .. ws = 9 buffers, ws_bytes, host_idx, compute, copy)
    bufs = [None] * 9

    def step(cache, n, layers, k, host_idx):
        return L.moe_decode_step(cache, n, layers, 1, 256, 128, 8, k, 1, 1, vp, 4, 4096, vp, *bufs, 0, host_idx,
                                 None, None)

    assert step(None, 1, vp, 2, vp) == moe._lib.MOE_EINVAL
    c = moe.SlotCache(2, 8, 4)  # policy-only cache: a real handle, no device memory
    try:
        assert step(c.h, 1, None, 2, vp) == moe._lib.MOE_EINVAL
        layers = np.zeros(1, dtype=moe.DECODE_LAYER)
        assert moe.DECODE_LAYER.itemsize == 6 * 8 + 2 * 4  # moe_decode_layer: six pointers, two int32
        assert step(c.h, 1, layers.ctypes.data, 9, vp) == moe._lib.MOE_ESHAPE  # k > E
        # a layer without its input is refused before anything is enqueued
        assert step(c.h, 1, layers.ctypes.data, 2, vp) == moe._lib.MOE_EINVAL
        assert step(c.h, 0, layers.ctypes.data, 2, vp) == 0  # zero layers: nothing to do

        # the hybrid step: (after slot_table) 9 buffers, ws_bytes, host_idx, host_x, host_y,
        # host_table, dev_table, cpu_rate, pcie_rate, host_fixed_s, copy_too, threads, n_cpu_out,
        # compute, copy
        def hstep(n, k, act, host, pcie=1.0, fixed=0.0):
            return L.moe_decode_step_hybrid(c.h, n, layers.ctypes.data, 256, 128, 8, k, act, 1, vp, 4, 4096, vp,
                                            *bufs, 0, host, host, host, host, host, 1.0, pcie, fixed, 1, 0, None,
                                            None, None)

        assert hstep(1, 2, 1, None) == moe._lib.MOE_EINVAL  # no pinned staging buffers
        assert hstep(1, 2, 1, vp, pcie=0.0) == moe._lib.MOE_EINVAL  # no PCIe rate
        assert hstep(1, 2, 1, vp, fixed=-1.0) == moe._lib.MOE_EINVAL  # negative fixed cost
        n = ctypes.c_int32(-5)
        assert L.moe_hybrid_split(3, 1.0, 0.0, 0.0, ctypes.byref(n)) == moe._lib.MOE_EINVAL
        assert L.moe_hybrid_split(-1, 1.0, 1.0, 0.0, ctypes.byref(n)) == moe._lib.MOE_EINVAL
        assert L.moe_hybrid_split(3, 1.0, 1.0, 0.0, None) == moe._lib.MOE_EINVAL
        assert L.moe_hybrid_split(3, 1.0, 1.0, 0.0, ctypes.byref(n)) == 0 and n.value == 1
        assert hstep(1, 2, 0, vp) == moe._lib.MOE_ESHAPE  # f32 activations
        assert hstep(1, 9, 1, vp) == moe._lib.MOE_ESHAPE  # k > E
        assert hstep(1, 2, 1, vp) == moe._lib.MOE_EINVAL  # a layer without its input
        assert hstep(0, 2, 1, vp) == 0

        # the split-launch step: (after slot_table) 9 buffers, ws_bytes, host_idx, host_tables,
        # dev_tables, compute, copy
        def sstep(n, k, host):
            return L.moe_decode_step_split(c.h, n, layers.ctypes.data, 1, 256, 128, 8, k, 1, 1, vp, 4, 4096, vp,
                                           *bufs, 0, host, host, host, None, None)

        assert sstep(1, 2, None) == moe._lib.MOE_EINVAL  # no staging buffers
        assert sstep(1, 9, vp) == moe._lib.MOE_ESHAPE  # k > E
        assert sstep(1, 2, vp) == moe._lib.MOE_EINVAL  # a layer without its input
        assert sstep(0, 2, vp) == 0
    finally:
        c.close()


def _unpack_dense(img, R, K, dt):
    # inverse of the documented layout: fragment (rb, kb), lane l <- row 16rb + l%16,
    # inputs 32kb + 8(l/16) .. +7 at element offset 8l
    out = np.empty((R, K), dtype=dt)
    v = img.view(dt)
    for rb in range(R // 16):
        for kb in range(K // 32):
            frag = v[(rb * 16 * K + kb * 512):(rb * 16 * K + kb * 512 + 512)].reshape(64, 8)
            for l in range(64):
                out[rb * 16 + l % 16, kb * 32 + 8 * (l // 16): kb * 32 + 8 * (l // 16) + 8] = frag[l]
    return out


def _unpack_int4(img, R, K):
    G = K // 128
    rbb = 8 * K + 32 * G
    q = np.empty((R, K), dtype=np.uint8)
    sc = np.empty((R, G), dtype=np.uint16)
    for rb in range(R // 16):
        blk = img[rb * rbb:(rb + 1) * rbb]
        for g in range(G):
            words = blk[g * 1024:(g + 1) * 1024].view(np.uint32).reshape(64, 4)
            for l in range(64):
                r, qq = rb * 16 + l % 16, l // 16
                for s in range(4):
                    w = int(words[l, s])
                    k0 = g * 128 + 32 * s + 8 * qq
                    for p in range(4):
                        q[r, k0 + 2 * p] = (w >> (4 * p)) & 0xF
                        q[r, k0 + 2 * p + 1] = (w >> (16 + 4 * p)) & 0xF
        sc[rb * 16:(rb + 1) * 16] = blk[G * 1024:G * 1024 + 32 * G].view(np.uint16).reshape(16, G)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, sc


@pytest.mark.parametrize("wdt,d,f", [("bf16", 64, 96), ("f32", 64, 128), ("int4", 256, 128)])
def test_pack_expert_layout_roundtrip(moe, wdt, d, f):
    wl = synth.Workload("t", d=d, E=1, k=1, f=f, act="bf16" if wdt != "f32" else "f32", wdt=wdt, T_list=(1,))
    ew = synth.expert_weights(wl, 3, 0, 0)
    img = moe.pack_expert(wdt, d, f, ew.wg, ew.wu, ew.wd, ew.sg, ew.su, ew.sd)
    assert img.nbytes == moe.slot_bytes(d, f, wdt)
    if wdt == "int4":
        rbd = 8 * d + 32 * (d // 128)
        gate = np.concatenate([img[(2 * b) * rbd:(2 * b + 1) * rbd] for b in range(f // 16)])
        up = np.concatenate([img[(2 * b + 1) * rbd:(2 * b + 2) * rbd] for b in range(f // 16)])
        down = img[2 * (f // 16) * rbd:]
        for blk, (pq, ps), R, K in ((gate, (ew.wg, ew.sg), f, d), (up, (ew.wu, ew.su), f, d),
                                    (down, (ew.wd, ew.sd), d, f)):
            uq, us = _unpack_int4(blk[:(R // 16) * (8 * K + 32 * (K // 128))], R, K)
            assert np.array_equal(uq, pq) and np.array_equal(us, ps)
    else:
        dt = np.uint16 if wdt == "bf16" else np.float32
        esz = np.dtype(dt).itemsize
        rbd = 16 * d * esz
        gate = np.concatenate([img[(2 * b) * rbd:(2 * b + 1) * rbd] for b in range(f // 16)])
        up = np.concatenate([img[(2 * b + 1) * rbd:(2 * b + 2) * rbd] for b in range(f // 16)])
        down = img[2 * (f // 16) * rbd:2 * (f // 16) * rbd + d * f * esz]
        assert np.array_equal(_unpack_dense(gate, f, d, dt), ew.wg)
        assert np.array_equal(_unpack_dense(up, f, d, dt), ew.wu)
        assert np.array_equal(_unpack_dense(down, d, f, dt), ew.wd)


def test_y_perm_element_types_in_the_binding(moe):
    """y_perm's element type goes to the library from the tensor (float32 or bfloat16, nothing
    else); the layer orchestration keeps bf16 rows for bf16 prefill only; the decode steps, whose C
    signature takes float rows, refuse anything but float32 before calling the library."""
    import torch

    assert moe._y_code(torch.empty(1, dtype=torch.float32)) == moe._lib.MOE_F32
    assert moe._y_code(torch.empty(1, dtype=torch.bfloat16)) == moe._lib.MOE_BF16
    with pytest.raises(TypeError):
        moe._y_code(torch.empty(1, dtype=torch.float16))
    assert moe.y_perm_dtype(torch.bfloat16, 65) == torch.bfloat16
    assert moe.y_perm_dtype(torch.bfloat16, 64) == torch.float32
    assert moe.y_perm_dtype(torch.float32, 4096) == torch.float32
    y16 = torch.empty((4, 8), dtype=torch.bfloat16)
    for fn, nargs in ((moe.decode_step, 20), (moe.decode_step_split, 22), (moe.decode_step_hybrid, 26)):
        args = [None] * nargs
        pos = list(inspect.signature(fn).parameters).index("y_perm")
        args[pos] = y16
        with pytest.raises(TypeError, match="y_perm must be float32"):
            fn(*args)
