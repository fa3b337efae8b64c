"""MoE-layer throughput on one MI355X.

Workload: the Qwen3.6-35B-A3B shaped decode layer (d_model 2048, 128 routed experts, top-8,
SwiGLU d_ff 768, bf16, Zipf(1.1) router bias, experts in HBM slots in a seeded order).  A step
is one whole layer forward -- route, permute, slot-indirected grouped SwiGLU, combine -- on one
batch of T tokens (default 64).  Steps rotate over R distinct HBM copies of the layer's weights
and R distinct input batches so that the 256 MB last-level cache cannot hold the working set.

Prints one JSON line: tokens/s, the HBM roofline of the dominant kernel (algorithmic bytes per
launch over its event-timed duration), and the oracle timed on the host cores as a baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--tokens", type=int, default=64)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--sweep", default="1,4,16,64", help="extra token counts timed for the sweep field")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def algorithmic_bytes(counts: np.ndarray, T: int, d: int, f: int, k: int, E: int, act_bytes=2, w_bytes=2):
    """Bytes the layer must move: touched experts' weights, router weights, x in, y out,
    plus the gate/up kernel's own share (its weights, its x rows, its h rows)."""
    U = int((counts > 0).sum())
    gateup = U * 2 * f * d * w_bytes + T * k * d * act_bytes + T * k * f * act_bytes
    down = U * d * f * w_bytes + T * k * f * act_bytes + T * k * d * 4
    layer = U * 3 * d * f * w_bytes + E * d * act_bytes + 2 * T * d * act_bytes
    return dict(U=U, gateup=gateup, down=down, layer=layer)


def cpu_baseline(wl, li, T, budget_s):
    """The oracle as it stands, on the host cores, on a bounded number of layer calls."""
    import synth
    from oracle.layer import moe_layer

    try:
        from threadpoolctl import threadpool_info

        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = 1
    cores = max(blas, int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
    calls, t0 = 0, time.perf_counter()
    while True:
        xb = synth.layer_inputs(wl, T, seed=0, batch=calls, with_experts=False).x
        moe_layer(xb, li.w_router, li.bias, wl.act, wl.k, wl.E, li.experts)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= 50:
            break
    return {"value": calls * T / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{calls} layer calls of {T} tokens (float64 numpy/BLAS oracle, {el:.1f} s)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import expert_offload_cache_amd as moe
    import synth
    from expert_offload_cache_amd.layer import DeviceLayer

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS["qwen_a3b_decode_bf16"]
    Tmain = args.tokens
    R = args.replicas
    tlist = sorted({Tmain, *[int(t) for t in args.sweep.split(",") if t]})
    Tmax = max(tlist)

    print(f"[bench] generating {wl.name} weights", file=sys.stderr, flush=True)
    li = synth.layer_inputs(wl, Tmax, seed=0)
    base = DeviceLayer.from_inputs(li, device=dev)
    layers = [base]
    for r in range(1, R):  # distinct HBM copies of the same layer (same slot order)
        cp = DeviceLayer.__new__(DeviceLayer)
        cp.__dict__.update(base.__dict__)
        cp.pool = base.pool.clone()
        layers.append(cp)
    stream = torch.cuda.Stream()

    def run_T(T, steps, warmup, profile=False):
        xs = [base.x_to_device(synth.layer_inputs(wl, T, seed=0, batch=b, with_experts=False).x) for b in range(R)]
        wss = [base.workspace(T) for _ in range(R)]
        outs = []
        with torch.cuda.stream(stream):
            for i in range(warmup):
                layers[i % R].forward(xs[i % R], ws=wss[i % R], stream=stream)
            stream.synchronize()
            if profile:
                moe.profile_reset()
                moe.profile_enable(True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                o = layers[i % R].forward(xs[i % R], ws=wss[i % R], stream=stream)
                if i < R:
                    outs.append(o["counts"])
            stream.synchronize()
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            if profile:
                moe.profile_collect()
                moe.profile_enable(False)
        counts = [c.cpu().numpy() for c in outs]
        return el, counts

    res = {}
    for T in tlist:
        steps = args.steps if T == Tmain else max(20, args.steps // 4)
        print(f"[bench] T={T}: {steps} timed steps", file=sys.stderr, flush=True)
        el, counts = run_T(T, steps, args.warmup)
        _, _ = run_T(T, steps, 2, profile=True)
        prof = moe.profile_results()
        byts = [algorithmic_bytes(c, T, wl.d, wl.f, wl.k, wl.E) for c in counts]
        avg = {key: float(np.mean([b[key] for b in byts])) for key in ("U", "gateup", "down", "layer")}
        kern = {name: ms / n * 1e3 for name, (ms, n) in prof.items()}  # average us per launch
        res[T] = dict(el=el, steps=steps, avg=avg, kern=kern)

    def kname(kern, part):
        names = [n for n in kern if n.startswith("ffn_") and part in n]
        return names[0] if names else None

    m = res[Tmain]
    ms_per_step = m["el"] / m["steps"] * 1e3
    gu_name = kname(m["kern"], "gateup")
    gu_us = m["kern"].get(gu_name)
    achieved = m["avg"]["gateup"] / (gu_us * 1e-6) / 1e9 if gu_us else None
    roofline = {"bound": "hbm", "kernel": gu_name, "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": (achieved / HBM_PEAK_GBS) if achieved else None, "traffic": None,
                "bytes_per_launch": m["avg"]["gateup"], "avg_launch_us": gu_us}
    sweep = {}
    for T, r in res.items():
        gu = r["kern"].get(kname(r["kern"], "gateup"))
        dn = r["kern"].get(kname(r["kern"], "down"))
        ffn_us = (gu or 0) + (dn or 0)
        sweep[str(T)] = {
            "tokens_per_s": T * r["steps"] / r["el"], "layer_us": r["el"] / r["steps"] * 1e6,
            "touched_experts": r["avg"]["U"],
            "gateup_us": gu, "down_us": dn,
            "gateup_GBps": r["avg"]["gateup"] / (gu * 1e-6) / 1e9 if gu else None,
            "ffn_GBps": (r["avg"]["gateup"] + r["avg"]["down"]) / (ffn_us * 1e-6) / 1e9 if ffn_us else None,
            "layer_GBps": r["avg"]["layer"] / (r["el"] / r["steps"]) / 1e9,
            "kernels_us": r["kern"],
        }
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host cores", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, li, Tmain, args.cpu_seconds)
    line = {
        "metric": "MoE-layer tokens/s (decode, grouped GEMV HBM roofline)",
        "value": Tmain * m["steps"] / m["el"], "unit": "tokens/s", "n_gpus": 1, "steps": m["steps"],
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3.6-35b-a3b shaped decode MoE layer", "tokens": Tmain, "d_model": wl.d,
                   "experts": wl.E, "top_k": wl.k, "d_ff": wl.f, "weights": "bf16", "router_bias": "zipf(1.1)",
                   "hbm_replicas": R, "parallelism": "single gpu"},
        "roofline": roofline, "cpu_baseline": cpu, "sweep": sweep,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
