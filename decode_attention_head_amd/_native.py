"""ctypes view of libdah.so: the C ABI of include/dah.h, function by function.

Loading fails loudly when the library has not been built; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdah.so")
PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdah_probe.so")

DAH_F32 = 0
DAH_BF16 = 1

STATUS_NAMES = {
    0: "DAH_OK", 1: "DAH_ERR_NULL", 2: "DAH_ERR_SHAPE", 3: "DAH_ERR_DTYPE",
    4: "DAH_ERR_ALIGN", 5: "DAH_ERR_WORKSPACE", 6: "DAH_ERR_HIP",
}

_c_int, _c_float, _c_i64, _c_size, _vp = (ctypes.c_int, ctypes.c_float, ctypes.c_int64,
                                           ctypes.c_size_t, ctypes.c_void_p)

# name -> (restype, argtypes), in the order of include/dah.h
SIGNATURES = {
    "qk_norm_rope_append": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_float, _c_float, _vp, _vp, _c_int,
                                     _c_i64, _vp, _c_int, _vp, _c_int, _vp, _vp]),
    "paged_decode_gqa": (_c_int, [_vp, _vp, _vp, _c_int, _c_i64, _vp, _c_int, _vp, _c_int, _c_int,
                                  _c_int, _vp, _vp, _c_size, _vp]),
    "decode_attn_step": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_float, _c_float, _vp, _vp, _c_int,
                                  _c_i64, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp,
                                  _c_size, _vp]),
    "dah_plan_decode": (_c_int, [_c_int, _c_int, _c_int, _c_int, ctypes.c_void_p]),
    "dah_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int]),
    "dah_workspace_bytes_for": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "qk_norm_rope_append_ex": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_float, _c_float, _vp, _vp,
                                        _c_int, _c_i64, _vp, _c_int, _vp, _c_int, _c_int, _vp, _vp]),
    "paged_decode_gqa_ex": (_c_int, [_vp, _vp, _vp, _c_int, _c_i64, _vp, _c_int, _vp, _c_int,
                                     _c_int, _c_int, _c_int, _vp, _vp, _c_size, _vp]),
    "decode_attn_step_ex": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_float, _c_float, _vp, _vp, _c_int,
                                     _c_i64, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _c_int, _vp,
                                     _vp, _vp, _c_size, _vp]),
    "decode_attn_step_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_float, _c_float, _vp,
                                          _vp, _c_int, _c_i64, _vp, _c_int, _vp, _c_int, _c_int,
                                          _c_int, _c_int, _vp, _vp, _vp]),
    "dah_plan_decode_ex": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    ctypes.c_void_p]),
    "dah_workspace_bytes_ex": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "chunk_attn_step": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_float, _c_float, _vp, _vp, _c_int,
                                 _c_i64, _vp, _c_int, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                 _c_int, _vp, _vp, _vp]),
    "dah_linear": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _vp, _vp]),
    "attn_qkv_proj": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp]),
    "attn_o_proj": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _vp, _vp]),
    "dah_linear_residual": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp]),
    "dah_linear_kernel": (_c_int, [_c_int, _c_int, _c_int]),
    "dah_linear_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int]),
    "dah_linear_ws": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _c_size, _vp]),
    "attn_o_proj_ws": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _c_size, _vp]),
    "dah_linear_ws_kernel": (_c_int, [_c_int, _c_int, _c_int, _vp]),
    "dah_rmsnorm_linear": (_c_int, [_vp, _vp, _c_float, _vp, _c_int, _c_int, _c_int, _vp, _vp]),
    "dah_rmsnorm_swiglu": (_c_int, [_vp, _vp, _c_float, _vp, _c_int, _c_int, _c_int, _vp, _vp]),
    "dah_rmsnorm": (_c_int, [_vp, _vp, _c_float, _c_int, _c_int, _vp, _vp]),
    "dah_silu_mul": (_c_int, [_vp, _c_int, _c_int, _vp, _vp]),
    "dah_layer_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                            _c_int]),
    "decoder_layer_step": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_float, _c_float, _vp,
                                    _vp, _c_int, _c_i64, _vp, _c_int, _vp, _c_int, _c_int, _c_int,
                                    _vp, _vp, _c_size, _vp]),
    "dah_status_string": (ctypes.c_char_p, [_c_int]),
    "dah_last_error": (ctypes.c_char_p, []),
}

# include/dah_probe.h (benchmark probes, separate library)
PROBE_SIGNATURES = {
    "dah_probe_copy": (_c_int, [_vp, _vp, _c_size, _vp]),
    "dah_probe_read": (_c_int, [_vp, _c_size, _vp, _c_int, _vp]),
    "dah_probe_paged_read": (_c_int, [_vp, _vp, _c_int, _c_i64, _vp, _c_int, _vp, _c_int, _c_int,
                                      _vp, _vp]),
}

_LIB = None
_PROBE_LIB = None

PLAN_MODES = {0: "per_sequence", 1: "split", 2: "balanced"}


class DecodePlan(ctypes.Structure):
    """dah_decode_plan of include/dah.h."""
    _fields_ = [("mode", ctypes.c_int), ("splits", ctypes.c_int),
                ("pages_per_split", ctypes.c_int), ("workgroups", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t), ("kernel", ctypes.c_int)]


class LayerWeights(ctypes.Structure):
    """dah_layer_weights of include/dah.h."""
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("w_in", "w_qkv", "q_gain", "k_gain", "w_o", "w_post", "w_gate_up", "w_down")]


class DahError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {detail}")


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m decode_attention_head_amd.build` "
                "(hipcc, gfx950). There is no fallback implementation.")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def probe_lib() -> ctypes.CDLL:
    """The benchmark's memory-probe library (loaded once)."""
    global _PROBE_LIB
    if _PROBE_LIB is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with "
                              "`python -m decode_attention_head_amd.build`")
        handle = ctypes.CDLL(PROBE_LIB_PATH)
        for name, (res, args) in PROBE_SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _PROBE_LIB = handle
    return _PROBE_LIB


def check(status: int, where: str) -> None:
    if status != 0:
        detail = lib().dah_last_error().decode(errors="replace")
        raise DahError(status, where, detail)
