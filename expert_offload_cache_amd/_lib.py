"""ctypes declarations of libmoe (include/moe.h).  Loading fails loudly when the library is missing."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH selects another build of the same library (the host-sanitizer build of the tests)
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_EDTYPE, MOE_ENOMEM, MOE_EHIP, MOE_ECAPACITY, MOE_ESTATE = 0, -1, -2, -3, -4, -5, -6, -7
MOE_F32, MOE_BF16, MOE_INT4_G128 = 0, 1, 2
STATUS_NAMES = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_ESHAPE", -3: "MOE_EDTYPE", -4: "MOE_ENOMEM",
                -5: "MOE_EHIP", -6: "MOE_ECAPACITY", -7: "MOE_ESTATE"}

# every function the header declares: name -> (restype, argtypes)
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
_st = ctypes.c_int32
SIGNATURES = {
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_version": (ctypes.c_char_p, []),
    "moe_slot_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_pack_expert": (_st, [_i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_route": (_st, [_vp, _i32, _i32, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "moe_permute": (_st, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_route_permute": (_st, [_vp, _i32, _i32, _i32, _vp, _vp, _i32, _i32] + [_vp] * 8 + [_vp, _sz, _vp]),
    "moe_permute_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "moe_expert_ffn_grouped": (_st, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _sz,
                                     _i32, _vp, _vp, _i32, _vp, _sz, _vp]),
    "moe_expert_ffn_grouped_noalloc": (_st, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32,
                                             _vp, _sz, _i32, _vp, _vp, _i32, _vp, _vp]),
    "moe_prefill_gemv_tokens": (_i32, [_i32]),
    "moe_combine": (_st, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp]),
    "moe_decode_step": (_st, [_vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _sz, _vp, _vp, _vp,
                              _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp, _vp]),
    "moe_decode_step_split": (_st, [_vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _sz, _vp,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp, _vp, _vp, _vp]),
    "moe_decode_step_hybrid": (_st, [_vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _sz, _vp, _vp,
                                     _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp, _vp, _vp, _vp,
                                     ctypes.c_double, ctypes.c_double, ctypes.c_double, _i32, _i32, _vp, _vp,
                                     _vp]),
    "moe_hybrid_split": (_st, [_i32, ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.POINTER(_st)]),
    "moe_cache_create": (_st, [_i32, _i32, _i32, _sz, _vp, _vp, _vp, ctypes.POINTER(_vp)]),
    "moe_cache_lookup": (_st, [_vp, _i32, _vp, _i32, _vp, _vp]),
    "moe_cache_fill": (_st, [_vp, _vp, _vp]),
    "moe_cache_prefetch_layer": (_st, [_vp, _i32, _vp, _vp]),
    "moe_cache_mark_read": (_st, [_vp, _i32, _vp]),
    "moe_cache_resize": (_st, [_vp, _i32, _vp, _vp]),
    "moe_cache_fill_split": (_st, [_vp, _vp, _i32, _vp, _vp]),
    "moe_cpu_expert_ffn": (_st, [_vp, _i32, _i32, _i32, _vp, _i32, _vp, _i32]),
    "moe_cache_stats": (_st, [_vp, _vp]),
    "moe_cache_trace": (_st, [_vp, _vp, _i64, _vp]),
    "moe_cache_copy_log": (_st, [_vp, _vp, _i64, _vp]),
    "moe_cache_inject_copy_failures": (_st, [_vp, _i32]),
    "moe_cache_slot_of": (_st, [_vp, _i32, _i32, _vp]),
    "moe_cache_destroy": (None, [_vp]),
    "moe_pinned_alloc": (_st, [_sz, ctypes.POINTER(_vp)]),
    "moe_pinned_free": (None, [_vp]),
    "moe_profile_enable": (None, [_i32]),
    "moe_profile_collect": (_st, []),
    "moe_profile_get": (_st, [_i32, ctypes.c_char_p, _i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
    "moe_profile_reset": (None, []),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def lib():
    """The loaded libmoe.  Raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(the HIP library is the only implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())
    return status
