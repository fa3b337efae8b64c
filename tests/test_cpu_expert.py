"""Host expert kernel (the CPU side of hybrid miss handling) against the oracle's SwiGLU expert on
the identically decoded weights (no GPU: the kernel makes no HIP call)."""
import numpy as np
import pytest

import synth
from gpu_util import rel_err_per_token, small_workload
from oracle.ffn import swiglu_expert
from oracle.numerics import bf16_to_f64, expert_to_f64


@pytest.mark.parametrize("wdt,d,f,n", [("int4", 256, 128, 1), ("int4", 512, 384, 3), ("bf16", 256, 96, 2),
                                       ("int4", 4096, 2048, 1)])
def test_cpu_expert_matches_oracle(wdt, d, f, n):
    import expert_offload_cache_amd as moe

    wl = small_workload("bf16", wdt, d, f, 4, 2)
    ew = synth.expert_weights(wl, 0, 0, 1)
    img = moe.pack_expert(wdt, d, f, ew.wg, ew.wu, ew.wd, ew.sg, ew.su, ew.sd)
    x = synth.normal_bf16(0, synth.stream_id(synth.KIND_X, 0, 9), (n, d), 1.0)
    y = moe.cpu_expert_ffn(img, wdt, d, f, x)
    ref = swiglu_expert(bf16_to_f64(x), *expert_to_f64(ew))
    err = rel_err_per_token(y.astype(np.float64), ref)
    assert err.max() <= 2e-2, err
    y1 = moe.cpu_expert_ffn(img, wdt, d, f, x, threads=1)
    assert np.array_equal(y, y1)  # thread count does not change the bits


def test_cpu_expert_rejects_bad_arguments():
    import expert_offload_cache_amd as moe

    img = np.zeros(moe.slot_bytes(256, 128, "int4"), dtype=np.uint8)
    with pytest.raises(moe.MoeError):
        moe.cpu_expert_ffn(img, "int4", 256, 100, np.zeros((1, 256), np.uint16))
    with pytest.raises(moe.MoeError):
        moe.cpu_expert_ffn(img, "f32", 256, 128, np.zeros((1, 256), np.uint16))
