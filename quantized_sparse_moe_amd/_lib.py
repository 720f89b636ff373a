"""ctypes binding of libqsmoe.so: struct mirrors and raw entry points.

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library. Loading fails loudly when the library is not built.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_int64, POINTER, Structure, c_char_p, c_float, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqsmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_ALIGNMENT = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5

MOE_FMT_AFFINE = 0
MOE_FMT_MXFP4 = 1
MOE_FMT_MXFP8 = 2
MOE_ROUTE_TOPK = 0
MOE_ROUTE_HASH = 1
MOE_OUT_BF16 = 0
MOE_OUT_F32 = 1

MOE_DEVERR_TOKEN_ID = 1
MOE_DEVERR_HASH_ID = 2
MOE_DEVERR_EXPERT_ID = 4
MOE_DEVERR_QUANT_INPUT = 8


class QTensorC(Structure):
    _fields_ = [("format", c_int32), ("bits", c_int32), ("group_size", c_int32), ("rows", c_int32),
                ("cols", c_int32), ("num_experts", c_int32), ("codes", c_void_p), ("scales", c_void_p),
                ("biases", c_void_p)]


class ExpertsC(Structure):
    _fields_ = [("gate", QTensorC), ("up", QTensorC), ("down", QTensorC)]


class RouterC(Structure):
    _fields_ = [("mode", c_int32), ("num_experts", c_int32), ("top_k", c_int32), ("hidden", c_int32),
                ("vocab", c_int32), ("weight", c_void_p), ("bias", c_void_p), ("tid2eid", c_void_p),
                ("routed_scale", c_float)]


class LayerC(Structure):
    _fields_ = [("router", RouterC), ("routed", ExpertsC), ("shared", POINTER(ExpertsC))]


class WsLayoutC(Structure):
    _fields_ = [("total", c_size_t), ("ids", c_size_t), ("weights", c_size_t), ("logits", c_size_t),
                ("keys", c_size_t), ("scores", c_size_t), ("offsets", c_size_t), ("perm", c_size_t),
                ("h", c_size_t), ("h_shared", c_size_t), ("y_slot", c_size_t), ("y_shared", c_size_t),
                ("fused", c_int32)]


# name -> (restype, argtypes)
_SIGS = {
    "moe_workspace_size": (c_size_t, [POINTER(LayerC), c_int32]),
    "moe_workspace_init": (c_int32, [c_void_p, c_size_t, c_void_p]),
    "moe_workspace_layout": (c_int32, [POINTER(LayerC), c_int32, POINTER(WsLayoutC)]),
    "moe_route": (c_int32, [POINTER(RouterC), c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_size_t,
                            c_void_p]),
    "moe_permute": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_size_t,
                              c_void_p]),
    "moe_expert_ffn": (c_int32, [POINTER(ExpertsC), POINTER(ExpertsC), c_void_p, c_int32, c_int32, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_combine": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p,
                              c_void_p]),
    "moe_forward": (c_int32, [POINTER(LayerC), c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_size_t,
                              c_void_p]),
    "moe_forward_noalloc": (c_int32, [POINTER(LayerC), c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
    "moe_forward_probed": (c_int32, [POINTER(LayerC), c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                     c_size_t, c_void_p, POINTER(c_void_p), c_int32, POINTER(c_char_p),
                                     POINTER(c_int32)]),
    "moe_router_logits": (c_int32, [POINTER(RouterC), c_void_p, c_int32, c_void_p, c_void_p]),
    "moe_device_error": (c_int32, [c_void_p, POINTER(c_int32), c_void_p]),
    "moe_probe_stream": (c_int32, [c_void_p, c_size_t, c_int32, c_void_p, c_void_p]),
    "moe_probe_mfma": (c_int32, [c_int32, c_int32, c_void_p, c_void_p]),
    "moe_mhc_sinkhorn": (c_int32, [c_void_p, c_int64, c_int32, c_int32, c_float, c_void_p, c_void_p]),
    "moe_quantize_affine": (c_int32, [c_void_p, c_int64, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p]),
    "moe_status_string": (c_char_p, [c_int32]),
    "moe_version": (c_char_p, []),
}

EXPORTED = tuple(_SIGS)

_lib = None


def load() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
                              "or `python quantized_sparse_moe_amd/build.py`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = load().moe_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)
