"""moe_expert_ffn_grouped_noalloc (the library's own per-GPU scratch instead of a caller workspace)
against moe_expert_ffn_grouped on the same inputs: y_perm bitwise equal (binary32 and bf16 rows), on two calls in a row
with the second smaller, on the decode GEMV and prefill MFMA paths; plus the size limit (refused
on the host, nothing launched) and the status word of an absent slot."""
import numpy as np
import pytest

import synth
from gpu_util import need_gpu, small_workload

pytestmark = pytest.mark.gpu


def _layer_and_routes(wl, Ts, seed=0):
    import torch
    from expert_offload_cache_amd.layer import DeviceLayer

    li = synth.layer_inputs(wl, max(Ts), seed=seed)
    layer = DeviceLayer.from_inputs(li, device="cuda")
    routes = []
    for T in Ts:
        x = layer.x_to_device(synth.layer_inputs(wl, T, seed=seed, batch=1, with_experts=False).x)
        out = layer.forward(x)
        routes.append((x, out))
    torch.cuda.synchronize()
    return layer, routes


def _both(moe, layer, x, out, soe=None, y_dtype=None):
    """y_perm (as bit patterns) and status from the workspace entry point and from the no-alloc one."""
    import torch

    soe = layer.slot_of_expert if soe is None else soe
    args = (x, out["perm"], out["offsets"], out["counts"], soe, layer.pool, layer.n_slots, layer.stride,
            layer.wdt, layer.f, layer.k)
    y_ws, ws = moe.expert_ffn_grouped(*args, shared_w=layer.shared, y_dtype=y_dtype)
    y_na = torch.full_like(y_ws, float("nan"))
    status = torch.zeros(1, dtype=torch.int32, device=x.device)
    moe.expert_ffn_grouped_noalloc(*args, y_perm=y_na, shared_w=layer.shared, status=status)
    torch.cuda.synchronize()
    st_ws = int(ws[:4].view(torch.int32).item())
    bits = torch.int16 if y_ws.dtype == torch.bfloat16 else torch.int32
    return y_ws.view(bits).cpu().numpy(), y_na.view(bits).cpu().numpy(), st_ws, int(status.item())


CASES = [
    # (name, workload, token counts of the two calls: the second smaller, y_perm rows in bf16)
    ("qwen_a3b_bf16_decode", synth.WORKLOADS["qwen_a3b_decode_bf16"], (64, 4), False),
    ("int4_decode", small_workload("bf16", "int4", 512, 512, 8, 2, shared=True), (20, 5), False),
    ("bf16_prefill_mfma", small_workload("bf16", "bf16", 512, 256, 16, 4, shared=True), (300, 100), False),
    ("bf16_prefill_mfma_bf16_rows", small_workload("bf16", "bf16", 512, 256, 16, 4, shared=True), (300, 100), True),
    ("int4_prefill_bf16_rows", small_workload("bf16", "int4", 512, 256, 6, 2, shared=True), (300, 120), True),
    ("f32_decode", small_workload("f32", "f32", 128, 64, 5, 3), (70, 3), False),
]


@pytest.mark.parametrize("name,wl,Ts,y16", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_workspace_call(name, wl, Ts, y16):
    need_gpu()
    import torch
    import expert_offload_cache_amd as moe

    print(f"no-alloc {name} T={Ts}", flush=True)
    layer, routes = _layer_and_routes(wl, Ts)
    for x, out in routes:  # two calls in a row into the same scratch, the second smaller
        y_ws, y_na, st_ws, st_na = _both(moe, layer, x, out, y_dtype=torch.bfloat16 if y16 else None)
        assert np.array_equal(y_ws, y_na), name
        assert st_ws == 0 and st_na == 0


def test_noalloc_reports_an_absent_slot_like_the_workspace_call():
    need_gpu()
    import torch
    import expert_offload_cache_amd as moe

    wl = small_workload("bf16", "bf16", 256, 96, 16, 4)
    layer, routes = _layer_and_routes(wl, (9,))
    x, out = routes[0]
    counts = out["counts"].cpu().numpy()
    soe = layer.slot_of_expert.clone()
    soe[int(np.argmax(counts))] = -1  # the busiest expert is absent
    y_ws, y_na, st_ws, st_na = _both(moe, layer, x, out, soe=soe)
    assert st_ws == 1 and st_na == 1
    assert np.array_equal(y_ws, y_na)
    # without a status pointer the call still runs and gives the same rows
    y2 = torch.full((y_ws.shape[0], y_ws.shape[1]), float("nan"), device="cuda")
    moe.expert_ffn_grouped_noalloc(x, out["perm"], out["offsets"], out["counts"], soe, layer.pool, layer.n_slots,
                                   layer.stride, layer.wdt, layer.f, layer.k, y_perm=y2)
    torch.cuda.synchronize()
    assert np.array_equal(y2.view(torch.int32).cpu().numpy(), y_ws)


def test_noalloc_refuses_calls_beyond_its_scratch():
    """A call needing more scratch than the library holds is refused on the host (nothing runs)."""
    need_gpu()
    import torch
    import expert_offload_cache_amd as moe
    from expert_offload_cache_amd._lib import MOE_BF16, MOE_ENOMEM

    wl = synth.WORKLOADS["qwen_a3b_decode_bf16"]
    T = 2048
    need = moe.workspace_bytes(T, wl.d, wl.f, wl.E, wl.k, False, MOE_BF16, moe.WDT["bf16"])
    assert need > (16 << 20)
    dev = "cuda"
    x = torch.zeros((T, wl.d), dtype=torch.bfloat16, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    perm, counts, offsets = torch.zeros(T * wl.k, **i32), torch.zeros(wl.E, **i32), torch.zeros(wl.E + 1, **i32)
    soe = torch.arange(wl.E, **i32)
    stride = moe.slot_bytes(wl.d, wl.f, "bf16")
    pool = torch.empty(stride, dtype=torch.uint8, device=dev)
    y = torch.empty((T * wl.k, wl.d), dtype=torch.float32, device=dev)
    with pytest.raises(moe.MoeError) as err:
        moe.expert_ffn_grouped_noalloc(x, perm, offsets, counts, soe, pool, 1, stride, "bf16", wl.f, wl.k, y_perm=y)
    assert err.value.status == MOE_ENOMEM
