"""ctypes loader for libqlora.so: argument marshalling only.

The library is required: there is no fallback implementation, and loading
fails loudly when it has not been built.
"""

from __future__ import annotations

import ctypes
import os
import threading

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libqlora.so")

c_i64 = ctypes.c_int64
c_i32 = ctypes.c_int32
c_f32 = ctypes.c_float
c_vp = ctypes.c_void_p
c_sz = ctypes.c_size_t


class LinearLayer(ctypes.Structure):
    """qlora_linear_layer: one layer of a grouped forward (host struct)."""
    _fields_ = [("n", c_i64), ("m", c_i64), ("r", c_i32), ("s", c_f32),
                ("x", c_vp), ("codes", c_vp), ("absmax8", c_vp), ("c2", c_vp),
                ("A", c_vp), ("B", c_vp), ("h", c_vp), ("u_out", c_vp)]


class QuantWeight(ctypes.Structure):
    """qlora_quant_weight: one weight of a grouped quantization (host struct)."""
    _fields_ = [("W", c_vp), ("m", c_i64), ("n", c_i64), ("codes", c_vp), ("absmax8", c_vp), ("c2", c_vp)]


class Dropout(ctypes.Structure):
    """qlora_dropout: dropout on the adapter input (host struct)."""
    _fields_ = [("p", c_f32), ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64)]


class AdamTensor(ctypes.Structure):
    """qlora_adam_tensor: one adapter tensor of an optimizer step (host struct)."""
    _fields_ = [("count", c_i64), ("param", c_vp), ("param_bf16", c_vp), ("grad", c_vp),
                ("exp_avg", c_vp), ("exp_avg_sq", c_vp)]


# name -> (restype, argtypes); mirrors include/qlora.h
PROTOTYPES = {
    "qlora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qlora_version": (ctypes.c_int, []),
    "qlora_nf4_table": (None, [c_vp, c_vp]),
    "qlora_quantize_nf4_dq": (ctypes.c_int, [c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp]),
    "qlora_dequant_nf4_dq": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp]),
    "qlora_level_table": (ctypes.c_int, [c_i32, c_vp, c_vp]),
    "qlora_quantize_dq": (ctypes.c_int, [c_i32, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp]),
    "qlora_quantize_dq_grouped": (ctypes.c_int, [c_i32, c_i32, ctypes.POINTER(QuantWeight), c_vp]),
    "qlora_dequant_dq": (ctypes.c_int, [c_i32, c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp]),
    "qlora_adam_step": (ctypes.c_int, [ctypes.POINTER(AdamTensor), c_i32, c_f32, c_f32, c_f32, c_f32, c_f32, c_i64,
                                       c_vp]),
    "qlora_merge_adapter": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp]),
    "qlora_workspace_bytes": (c_sz, [ctypes.c_int, c_i64, c_i64, c_i64, c_i32]),
    "qlora_linear_fwd": (ctypes.c_int, [c_i64, c_i64, c_i64, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, c_vp, c_vp, c_sz, c_vp]),
    "qlora_linear_fwd_static": (ctypes.c_int, [c_i64, c_i64, c_i64, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_vp,
                                               c_vp, c_vp, c_vp, c_vp]),
    "qlora_grouped_workspace_bytes": (c_sz, [c_i64, c_i32, ctypes.POINTER(LinearLayer)]),
    "qlora_linear_fwd_grouped": (ctypes.c_int, [c_i64, c_i32, ctypes.POINTER(LinearLayer), c_vp, c_sz, c_vp]),
    "qlora_linear_bwd": (ctypes.c_int, [c_i64, c_i64, c_i64, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "qlora_linear_fwd_ex": (ctypes.c_int, [c_i64, c_i64, c_i64, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                           c_vp, c_vp, ctypes.POINTER(Dropout), c_vp, c_sz, c_vp]),
    "qlora_linear_bwd_ex": (ctypes.c_int, [c_i64, c_i64, c_i64, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                           c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.POINTER(Dropout), c_vp, c_sz,
                                           c_vp]),
    "qlora_linear_check": (ctypes.c_int, [ctypes.c_int, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp]),
    "qlora_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "qlora_profile_query": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(c_i64), ctypes.POINTER(ctypes.c_double)]),
}

_lock = threading.Lock()
_lib = None


class QloraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def load() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m bit_quantized_fine_qlora_amd.build`; "
                    "there is no fallback implementation")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in PROTOTYPES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().qlora_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != 0:
        raise QloraError(status, where)
