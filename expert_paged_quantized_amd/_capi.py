"""ctypes declarations of the C ABI in include/strata_moe.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

c_i32, c_u64, c_vp = ctypes.c_int32, ctypes.c_uint64, ctypes.c_void_p

OK, E_INVALID, E_UNSUPPORTED, E_BAD_SCALE, E_NOMEM, E_HIP, E_POISONED = range(7)
STATUS_NAMES = ["OK", "E_INVALID", "E_UNSUPPORTED", "E_BAD_SCALE", "E_NOMEM", "E_HIP", "E_POISONED"]
Q_INT4_G64, Q_MXFP4_G32, Q_INT4_G128, Q_NVFP4_G16 = 1, 2, 3, 4
R_SOFTMAX, R_SIGMOID = 1, 2
P_LRU, P_LFU, P_WARM = 1, 2, 3
PAGER_AUTO, PAGER_KERNEL, PAGER_DMA = 0, 1, 2
KERNEL_CLASSES = ["router", "group", "decode_gate_up", "decode_down", "prefill_gate_up",
                  "prefill_down", "combine"]


class QMat(ctypes.Structure):
    _fields_ = [("codes", c_vp), ("scales", c_vp), ("biases", c_vp), ("global_scale", c_vp)]


class Desc(ctypes.Structure):
    _fields_ = [("hidden", c_i32), ("ffn", c_i32), ("num_experts", c_i32), ("top_k", c_i32),
                ("num_shared", c_i32), ("quant", c_i32), ("router", c_i32), ("policy", c_i32),
                ("expert_budget", c_i32), ("max_tokens", c_i32), ("device", c_i32),
                ("decay_shift", c_i32), ("prefetch", c_i32), ("pager", c_i32), ("expert_profile", c_vp),
                ("router_w", c_vp), ("router_bias", c_vp),
                ("gate", QMat), ("up", QMat), ("down", QMat),
                ("sh_gate", QMat), ("sh_up", QMat), ("sh_down", QMat), ("shared_gate_w", c_vp),
                ("hybrid", c_i32), ("host_threads", c_i32), ("hybrid_rows", c_i32)]


class RouteDbg(ctypes.Structure):
    _fields_ = [("logits", c_vp), ("topk_idx", c_vp), ("topk_w", c_vp), ("counts", c_vp),
                ("offsets", c_vp), ("perm", c_vp)]


class CacheStats(ctypes.Structure):
    _fields_ = [("forwards", c_u64), ("hits", c_u64), ("misses", c_u64), ("evictions", c_u64),
                ("bytes_h2d", c_u64), ("waves", c_u64), ("budget", c_i32), ("resident", c_i32),
                ("policy", c_i32), ("decay_shift", c_i32), ("resident_bytes", c_u64),
                ("expert_bytes", c_u64), ("prefetched", c_u64), ("prefetch_hits", c_u64),
                ("prefetch", c_i32), ("pager", c_i32), ("host_experts", c_u64), ("host_ns", c_u64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class MemoryInfo(ctypes.Structure):
    _fields_ = [("slot_pool", c_u64), ("shared", c_u64), ("router", c_u64), ("workspace", c_u64),
                ("device_total", c_u64), ("host_store", c_u64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class Timing(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * 7), ("launches", c_u64 * 7)]


EXPORTS = {
    "strata_moe_create": (c_i32, [ctypes.POINTER(Desc), ctypes.POINTER(c_vp)]),
    "strata_moe_forward": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_vp, ctypes.POINTER(RouteDbg)]),
    "strata_moe_forward_noalloc": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_vp, ctypes.POINTER(RouteDbg)]),
    "strata_expert_cache_stats": (c_i32, [c_vp, ctypes.POINTER(CacheStats)]),
    "strata_moe_memory": (c_i32, [c_vp, ctypes.POINTER(MemoryInfo)]),
    "strata_moe_set_timing": (c_i32, [c_vp, c_i32]),
    "strata_moe_timing": (c_i32, [c_vp, ctypes.POINTER(Timing)]),
    "strata_moe_destroy": (None, [c_vp]),
    "strata_last_error": (ctypes.c_char_p, []),
    "strata_measure_h2d": (c_i32, [c_i32, c_u64, c_i32, ctypes.POINTER(ctypes.c_double)]),
    "strata_measure_hbm_read": (c_i32, [c_i32, c_u64, c_i32, ctypes.POINTER(ctypes.c_double)]),
    "strata_expert_profile_save": (c_i32, [c_vp, c_vp, c_i32]),
    "strata_expert_profile_load": (c_i32, [c_vp, c_vp, c_i32]),
    "strata_residency_replay": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_u64, c_i32,
                                        c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp,
                                        ctypes.POINTER(CacheStats)]),
}

_lib = None


def lib():
    """The loaded HIP library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m expert_paged_quantized_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class StrataError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES[status] if 0 <= status < 7 else status}: {message}")


def check(status: int):
    if status != OK:
        raise StrataError(status, lib().strata_last_error().decode(errors="replace"))
