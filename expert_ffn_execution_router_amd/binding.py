"""ctypes binding of libmoe.so: the C ABI of include/moe.h under the same names.

Argument marshalling only: every step of the MoE layer runs in the library's
HIP kernels and host C++.  Pointers are passed as integers (device pointers
from torch tensors' data_ptr(), streams from torch.cuda.Stream.cuda_stream).
Raises RuntimeError when the library is missing; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_E_INVAL = -1
MOE_E_HIP = -2
MOE_E_NOSLOTS = -3
MOE_E_PIN = -4
MOE_E_NOT_RESIDENT = -5
MOE_E_UNSUPPORTED = -6
MOE_I_FALLBACK_ONDEMAND = 1
MOE_I_SINGLE_BUFFER = 2

MOE_W_BF16, MOE_W_FP8_E4M3_B128, MOE_W_MXFP4, MOE_W_NVFP4 = 0, 1, 2, 3
MOE_ACT_DEFAULT, MOE_ACT_MXFP6 = 0, 1
MOE_QUANT_MXFP6 = 64
MOE_POLICY_OFFLOAD, MOE_POLICY_HOST, MOE_POLICY_HYBRID = 0, 1, 2


class moe_config(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int), ("E", ctypes.c_int), ("k", ctypes.c_int), ("H", ctypes.c_int),
                ("I", ctypes.c_int), ("wfmt", ctypes.c_int), ("n_slots", ctypes.c_int),
                ("max_tokens", ctypes.c_int), ("host_threads", ctypes.c_int)]


class moe_plan_totals(ctypes.Structure):
    _fields_ = [(f, ctypes.c_longlong) for f in ("calls", "n_unique", "n_hit", "m", "q", "n_host", "n_evict")] + \
        [("host_ms", ctypes.c_double)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class moe_calibration(ctypes.Structure):
    _fields_ = [(f, ctypes.c_double) for f in ("B_P", "B_P_min", "B_P_max", "B_H", "host_alone", "host_alone_min",
                                               "host_alone_max", "host_conc", "host_conc_min", "host_conc_max")] + \
        [(f, ctypes.c_int) for f in ("n_copy", "n_host_alone", "n_host_conc")] + \
        [(f, ctypes.c_double) for f in ("host_alone_1", "host_conc_1", "host_t0_us", "B_R")]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class moe_plan_info(ctypes.Structure):
    _fields_ = [("n_unique", ctypes.c_int), ("n_hit", ctypes.c_int), ("m", ctypes.c_int), ("q", ctypes.c_int),
                ("n_host", ctypes.c_int), ("n_evict", ctypes.c_int), ("t_fill_pred_us", ctypes.c_double),
                ("t_host_pred_us", ctypes.c_double)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


MOE_N_STAGES = 12
STAGES = ["route", "topk", "group", "quant_x", "gemm1", "quant_a", "gemm2", "combine", "plan", "fixup", "fill",
          "tail"]


class moe_profile(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int * MOE_N_STAGES), ("ms", ctypes.c_double * MOE_N_STAGES),
                ("dropped", ctypes.c_int)]

    def as_dict(self):
        return {name: {"launches": self.launches[i], "ms": self.ms[i]} for i, name in enumerate(STAGES)}


_vp, _i, _sz, _d = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
_P = ctypes.POINTER

# name -> (restype, argtypes), in the order of include/moe.h
SIGNATURES = {
    "moe_expert_bytes": (_sz, [_P(moe_config)]),
    "moe_workspace_bytes": (_sz, [_P(moe_config)]),
    "moe_create": (_i, [_P(moe_config), _vp, _sz, _vp, _sz, _vp, _sz, _P(_vp)]),
    "moe_destroy": (_i, [_vp]),
    "moe_last_error": (ctypes.c_char_p, [_vp]),
    "moe_host_alloc": (_i, [_sz, _P(_vp)]),
    "moe_host_free": (_i, [_vp]),
    "moe_set_policy": (_i, [_vp, _i, _d, _d]),
    "moe_set_activations": (_i, [_vp, _i]),
    "moe_calibrate_ex": (_i, [_vp, _i, _P(moe_calibration)]),
    "moe_calibrate": (_i, [_vp, _P(_d), _P(_d)]),
    "moe_slot_table": (_vp, [_vp]),
    "moe_reset_cache": (_i, [_vp, _vp]),
    "moe_route": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _vp, _vp]),
    "moe_route_from_logits": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_quantize": (_i, [_i, _i, _vp, _i, _i, _vp, _vp, _vp, _vp]),
    "moe_plan": (_i, [_vp, _i, _vp, _i, _vp, _P(moe_plan_info), _vp, _vp, _vp]),
    "slot_pool_fill": (_i, [_vp, _i, _vp, _vp, _i, _vp]),
    "slot_pool_admit": (_i, [_vp, _i, _vp, _i, _vp]),
    "slot_pool_evict": (_i, [_vp, _i, _vp, _i]),
    "moe_host_partial": (_i, [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp]),
    "moe_host_ffn": (_i, [_P(moe_config), _vp, _i, _vp, _vp, _vp, _i, _vp, _vp]),
    "moe_layer_forward": (_i, [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp]),
    "moe_layer_forward_noalloc": (_i, [_P(moe_config), _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp]),
    "moe_decode_layer": (_i, [_vp, _i, _vp, _vp, _vp, _i, _vp, _P(moe_plan_info), _vp, _vp]),
    "moe_decode_layer_async": (_i, [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp]),
    "moe_plan_stats": (_i, [_vp, _P(moe_plan_totals), _i]),
    "slot_pool_resize": (_i, [_vp, _vp, ctypes.c_size_t, _i, _vp]),
    "prefill_stream_layer": (_i, [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i]),
    "moe_check_device_error": (_i, [_vp]),
    "moe_profile_begin": (_i, [_vp, _i, ctypes.c_uint]),
    "moe_profile_end": (_i, [_vp, _P(moe_profile)]),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libmoe error {code}: {msg}")
        self.code = code


def lib():
    """Load libmoe.so from the package directory (built by build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with expert_ffn_execution_router_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error(ctx=None) -> str:
    s = lib().moe_last_error(ctx)
    return s.decode() if s else ""


def check(rc, ctx=None):
    if rc < 0:
        raise MoeError(rc, last_error(ctx))
    return rc


def _fn(name):
    def call(*args):
        return getattr(lib(), name)(*args)
    call.__name__ = name
    return call


# the C functions under their own names (raw return codes)
moe_expert_bytes = _fn("moe_expert_bytes")
moe_workspace_bytes = _fn("moe_workspace_bytes")
moe_create = _fn("moe_create")
moe_destroy = _fn("moe_destroy")
moe_host_alloc = _fn("moe_host_alloc")
moe_host_free = _fn("moe_host_free")
moe_set_policy = _fn("moe_set_policy")
moe_set_activations = _fn("moe_set_activations")
moe_calibrate_ex = _fn("moe_calibrate_ex")
moe_calibrate = _fn("moe_calibrate")
moe_slot_table = _fn("moe_slot_table")
moe_reset_cache = _fn("moe_reset_cache")
moe_route = _fn("moe_route")
moe_route_from_logits = _fn("moe_route_from_logits")
moe_quantize = _fn("moe_quantize")
moe_plan = _fn("moe_plan")
slot_pool_fill = _fn("slot_pool_fill")
slot_pool_admit = _fn("slot_pool_admit")
slot_pool_evict = _fn("slot_pool_evict")
moe_host_partial = _fn("moe_host_partial")
moe_host_ffn = _fn("moe_host_ffn")
moe_layer_forward = _fn("moe_layer_forward")
moe_layer_forward_noalloc = _fn("moe_layer_forward_noalloc")
moe_decode_layer = _fn("moe_decode_layer")
moe_decode_layer_async = _fn("moe_decode_layer_async")
moe_plan_stats = _fn("moe_plan_stats")
slot_pool_resize = _fn("slot_pool_resize")
prefill_stream_layer = _fn("prefill_stream_layer")
moe_check_device_error = _fn("moe_check_device_error")
moe_profile_begin = _fn("moe_profile_begin")
moe_profile_end = _fn("moe_profile_end")


def make_config(L, E, k, H, I, wfmt, n_slots, max_tokens, host_threads=0) -> moe_config:
    return moe_config(L, E, k, H, I, wfmt, n_slots, max_tokens, host_threads)
