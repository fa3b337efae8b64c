"""Helpers shared by the GPU parity tests (marshalling and comparison only)."""
import numpy as np
import pytest

import synth


def need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def to_dev(a, dt):
    import torch

    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    if dt == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    if dt == "i32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    raise ValueError(dt)


def y_to_f64(y):
    import torch

    if y.dtype == torch.bfloat16:
        bits = y.view(torch.int16).cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return y.float().cpu().numpy().astype(np.float64)


def rel_err_per_token(y, ref):
    num = np.linalg.norm(y - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return num / np.maximum(den, 1e-300)


def tol_for(wl):
    return 1e-4 if (wl.act == "f32" and wl.wdt == "f32") else 2e-2


def small_workload(act, wdt, d, f, E, k, shared=False, bias=1.1):
    return synth.Workload(f"small_{act}_{wdt}_{d}_{f}_{E}_{k}", d=d, E=E, k=k, f=f, act=act, wdt=wdt,
                          T_list=(1,), shared=shared, zipf_bias=bias)
