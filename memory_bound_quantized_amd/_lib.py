"""ctypes loader for libmbq.so (the C ABI declared in include/mbq.h).

The library is loaded from this package directory.  There is no fallback:
if the shared object is missing, importing the binding raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmbq.so")

OK, EINVAL, EALIGN, EUNSUPPORTED, EHIP = 0, -1, -2, -3, -4
BF16, Q45, Q65, Q25 = 0, 1, 2, 3

# Every symbol include/mbq.h declares, in declaration order.
EXPORTS = (
    "mbq_format_info", "mbq_plane_sizes", "mbq_pack", "mbq_unpack", "mbq_gemv_q",
    "mbq_gemv_q_gather", "mbq_gemv_fused", "mbq_decode_workspace_bytes", "mbq_decode_step",
    "mbq_decode_kv_workspace_bytes", "mbq_decode_step_kv", "mbq_decode_step_noalloc", "mbq_decode_prepare", "mbq_decode_step_persistent",
    "mbq_xq_bytes", "mbq_stage_x", "mbq_gemv_xq", "mbq_gemv_xq_workspace_bytes", "mbq_gemv_xq_ws",
    "mbq_rmsnorm_xq",
    "mbq_silu_mul_xq", "mbq_rmsnorm", "mbq_layernorm", "mbq_silu_mul", "mbq_dequant_f32",
    "mbq_unpack_codes", "mbq_quantize", "mbq_attention_workspace_bytes", "mbq_attention_decode",
    "mbq_attention_decode_append", "mbq_probe_read", "mbq_probe_copy", "mbq_probe_mixed", "mbq_probe_chase_init",
    "mbq_probe_chase", "mbq_probe_peak", "mbq_status_str",
    "mbq_last_error", "mbq_version",
)


class QWeightDesc(ctypes.Structure):
    """struct mbq_qweight."""
    _fields_ = [("fmt", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("codes_hi", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("super_scales", ctypes.c_void_p)]


class DecodeLayerDesc(ctypes.Structure):
    """struct mbq_decode_layer."""
    _fields_ = [("qkv", QWeightDesc), ("o", QWeightDesc), ("gate_up", QWeightDesc),
                ("down", QWeightDesc), ("gamma1", ctypes.c_void_p), ("gamma2", ctypes.c_void_p)]


class DecodeModelDesc(ctypes.Structure):
    """struct mbq_decode_model."""
    _fields_ = [("n_layers", ctypes.c_int32), ("eps", ctypes.c_float),
                ("d", ctypes.c_int64), ("dq", ctypes.c_int64), ("dkv", ctypes.c_int64),
                ("f", ctypes.c_int64), ("vocab", ctypes.c_int64),
                ("layers", ctypes.POINTER(DecodeLayerDesc)), ("gamma_f", ctypes.c_void_p),
                ("lm_head", QWeightDesc)]


class MbqError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s (%s)" % (detail, _status_name(status)))
        self.status = status


def _status_name(s):
    return {OK: "MBQ_OK", EINVAL: "MBQ_EINVAL", EALIGN: "MBQ_EALIGN",
            EUNSUPPORTED: "MBQ_EUNSUPPORTED", EHIP: "MBQ_EHIP"}.get(s, str(s))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmbq.so is not built at %s; run "
                          "`python memory_bound_quantized_amd/build.py` first" % LIB_PATH)
    # torch supplies device memory and streams, so libmbq must run on torch's
    # HIP runtime.  torch bundles its own libamdhip64 with the same SONAME
    # (libamdhip64.so.7); once torch is loaded, libmbq's dependency resolves
    # to that copy instead of loading a second runtime into the process.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    sz = ctypes.c_size_t
    sig = {
        "mbq_format_info": (i32, [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]),
        "mbq_plane_sizes": (i32, [i32, i64, i64, ctypes.POINTER(sz)]),
        "mbq_pack": (i32, [i32, i64, i64, vp, vp, vp, ctypes.POINTER(vp)]),
        "mbq_unpack": (i32, [i32, i64, i64, ctypes.POINTER(vp), vp, vp, vp]),
        "mbq_gemv_q": (i32, [ctypes.POINTER(QWeightDesc), vp, i64, i64, vp, i64, i32, vp]),
        "mbq_gemv_q_gather": (i32, [ctypes.POINTER(QWeightDesc), i64, vp, i64, vp, vp, vp]),
        "mbq_gemv_fused": (i32, [ctypes.POINTER(QWeightDesc), vp, vp, f32, i32, vp, vp]),
        "mbq_decode_workspace_bytes": (i32, [ctypes.POINTER(DecodeModelDesc), ctypes.POINTER(sz)]),
        "mbq_decode_step": (i32, [ctypes.POINTER(DecodeModelDesc), vp, vp, vp, sz, vp]),
        "mbq_decode_kv_workspace_bytes": (i32, [ctypes.POINTER(DecodeModelDesc), i64, ctypes.POINTER(sz)]),
        "mbq_decode_step_kv": (i32, [ctypes.POINTER(DecodeModelDesc), vp, vp, ctypes.POINTER(vp),
                                     ctypes.POINTER(vp), i64, i64, vp, sz, vp]),
        "mbq_decode_step_noalloc": (i32, [ctypes.POINTER(DecodeModelDesc), vp, vp, vp]),
        "mbq_decode_prepare": (i32, [ctypes.POINTER(DecodeModelDesc), vp, sz, vp]),
        "mbq_decode_step_persistent": (i32, [ctypes.POINTER(DecodeModelDesc), vp, vp, vp, sz, vp]),
        "mbq_xq_bytes": (i32, [i32, i64, i64, ctypes.POINTER(sz)]),
        "mbq_stage_x": (i32, [i32, vp, i64, i64, i64, vp, vp]),
        "mbq_gemv_xq": (i32, [ctypes.POINTER(QWeightDesc), vp, i64, vp, i64, i32, vp]),
        "mbq_gemv_xq_workspace_bytes": (i32, [ctypes.POINTER(QWeightDesc), i64, ctypes.POINTER(sz)]),
        "mbq_gemv_xq_ws": (i32, [ctypes.POINTER(QWeightDesc), vp, i64, vp, i64, i32, vp, sz, vp]),
        "mbq_rmsnorm_xq": (i32, [vp, vp, f32, i64, vp, i32, vp, vp]),
        "mbq_silu_mul_xq": (i32, [vp, vp, i64, i32, vp, vp]),
        "mbq_rmsnorm": (i32, [vp, vp, f32, i64, i64, vp, vp]),
        "mbq_layernorm": (i32, [vp, vp, vp, f32, i64, i64, vp, vp]),
        "mbq_silu_mul": (i32, [vp, vp, i64, vp, vp]),
        "mbq_dequant_f32": (i32, [ctypes.POINTER(QWeightDesc), vp, vp]),
        "mbq_unpack_codes": (i32, [ctypes.POINTER(QWeightDesc), vp, vp]),
        "mbq_quantize": (i32, [i32, vp, i64, i64, i64, ctypes.POINTER(vp), vp]),
        "mbq_attention_workspace_bytes": (i32, [i64, i32, i32, i32, ctypes.POINTER(sz)]),
        "mbq_attention_decode": (i32, [vp, vp, vp, i64, i64, i32, i32, i32, vp, vp, sz, vp]),
        "mbq_attention_decode_append": (i32, [vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, vp, vp, sz, vp]),
        "mbq_probe_mixed": (i32, [vp, sz, vp, sz, i32, i32, vp, vp]),
        "mbq_probe_read": (i32, [vp, sz, vp, vp]),
        "mbq_probe_copy": (i32, [vp, vp, sz, vp]),
        "mbq_probe_chase_init": (i32, [vp, sz, ctypes.POINTER(ctypes.c_uint32), vp]),
        "mbq_probe_chase": (i32, [vp, ctypes.c_uint32, i64, vp, vp]),
        "mbq_probe_peak": (i32, [i32, i64, vp, ctypes.POINTER(ctypes.c_int64), vp]),
        "mbq_status_str": (ctypes.c_char_p, [i32]),
        "mbq_last_error": (ctypes.c_char_p, []),
        "mbq_version": (i32, []),
    }
    for name in EXPORTS:
        f = getattr(L, name)
        f.restype, f.argtypes = sig[name]
    return L


lib = _load()


def check(status: int) -> int:
    if status != OK:
        raise MbqError(status, lib.mbq_last_error().decode() or lib.mbq_status_str(status).decode())
    return status
