"""A decode layer captured in a HIP graph (torch.cuda.CUDAGraph around the C-ABI calls) and
replayed: every replay gives bitwise the outputs of the eager call on the same input, with eager
work and synchronisations between the replays.  The captured calls enqueue kernel launches only
(no memset or copy nodes)."""
import gc

import numpy as np
import pytest

import synth
from gpu_util import need_gpu

pytestmark = pytest.mark.gpu

KEYS = ("y", "topk_idx", "topk_w", "logits", "counts", "offsets", "perm", "inv_perm", "y_perm")


def _bits(t):
    import torch

    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    elif t.dtype == torch.float32:
        t = t.view(torch.int32)
    return t.cpu().numpy().copy()


def _check(out, ref, what):
    for key in KEYS:
        assert np.array_equal(_bits(out[key]), ref[key]), f"{what}: {key} differs"


@pytest.mark.parametrize("name,T", [("qwen_a3b_decode_bf16", 1), ("qwen_a3b_decode_bf16", 64),
                                    ("dsv4_decode_int4", 1), ("dsv4_decode_int4", 8)])
def test_graph_replays_match_eager(name, T):
    need_gpu()
    import torch

    from expert_offload_cache_amd.layer import DeviceLayer

    print(f"graph {name} T={T}", flush=True)
    wl = synth.WORKLOADS[name]
    layer = DeviceLayer.from_inputs(synth.layer_inputs(wl, T, seed=0))
    xs = [layer.x_to_device(synth.layer_inputs(wl, T, seed=0, batch=b, with_experts=False).x) for b in (1, 2)]
    ws = layer.workspace(T)
    refs = []
    for x in xs:
        o = layer.forward(x, ws=ws)
        refs.append({key: _bits(o[key]) for key in KEYS})
    assert not np.array_equal(refs[0]["y"], refs[1]["y"])

    x_static = xs[0].clone()
    ws_static = layer.workspace(T)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x_static, ws=ws_static)  # warm-up off the default stream, as torch asks
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = layer.forward(x_static, ws=ws_static)
    torch.cuda.synchronize()

    for rep, b in enumerate((0, 0, 1, 0, 1)):
        x_static.copy_(xs[b])
        g.replay()
        torch.cuda.synchronize()
        _check(out, refs[b], f"replay {rep} (input {b})")
        eager = layer.forward(xs[1 - b], ws=ws)  # the program's own work between replays
        torch.cuda.synchronize()
        _check(eager, refs[1 - b], f"eager call after replay {rep}")
    del g, out, layer
    gc.collect()
