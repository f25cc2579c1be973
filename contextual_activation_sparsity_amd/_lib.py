"""ctypes binding of libdejavu_hip.so (declared in include/dejavu_hip.h).

Argument marshalling only: every step of the layer runs in the library's HIP kernels.
Torch provides device memory and streams. The library is loaded on first use; if it is
missing the call raises (there is no other implementation to fall back to).
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdejavu_hip.so")

DV_F32, DV_F16 = 0, 1
DV_IDX_RANGE, DV_IDX_ORDER, DV_IDX_DUPLICATE = 1, 2, 4
STATUS = {0: "DV_OK", 1: "DV_ERR_NULL", 2: "DV_ERR_DIMS", 3: "DV_ERR_K", 4: "DV_ERR_DTYPE",
          5: "DV_ERR_ALIGN", 6: "DV_ERR_KV", 7: "DV_ERR_WORKSPACE", 8: "DV_ERR_HIP"}

c_void_p = ctypes.c_void_p
c_int32 = ctypes.c_int32
c_size_t = ctypes.c_size_t


class DvDims(ctypes.Structure):
    _fields_ = [("d_model", c_int32), ("d_ffn", c_int32), ("n_heads", c_int32), ("head_dim", c_int32),
                ("rank_mlp", c_int32), ("rank_head", c_int32), ("t_max", c_int32), ("dtype", c_int32)]


class DvPredictor(ctypes.Structure):
    _fields_ = [("p1_mlp", c_void_p), ("p2_mlp", c_void_p), ("p1_head", c_void_p), ("p2_head", c_void_p)]


class DvLayer(ctypes.Structure):
    _fields_ = [("g1", c_void_p), ("g2", c_void_p), ("wqkv", c_void_p), ("bqkv", c_void_p),
                ("wo", c_void_p), ("bo", c_void_p), ("w1t", c_void_p), ("b1", c_void_p),
                ("w2", c_void_p), ("b2", c_void_p)]


class DejavuError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {detail}")
        self.status = status
        self.status_name = STATUS.get(status, str(status))


_lib = None
_lock = threading.Lock()

# name -> (restype, argtypes)
SIGNATURES = {
    "dv_predict": (c_int32, [ctypes.POINTER(DvDims), ctypes.POINTER(DvPredictor), c_void_p, c_int32,
                             c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "dv_topk": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "dv_sparse_mlp": (c_int32, [ctypes.POINTER(DvDims), ctypes.POINTER(DvLayer), c_void_p, c_int32,
                                c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "dv_sparse_attn": (c_int32, [ctypes.POINTER(DvDims), ctypes.POINTER(DvLayer), c_void_p, c_int32,
                                 c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                 c_size_t, c_void_p]),
    "dv_layer_step": (c_int32, [ctypes.POINTER(DvDims), ctypes.POINTER(DvLayer), ctypes.POINTER(DvPredictor),
                                c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                c_void_p]),
    "dv_layer_step_noalloc": (c_int32, [ctypes.POINTER(DvDims), ctypes.POINTER(DvLayer), ctypes.POINTER(DvPredictor),
                                        c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dv_lookahead_stack": (c_int32, [ctypes.POINTER(DvDims), ctypes.POINTER(DvLayer),
                                     ctypes.POINTER(DvPredictor), c_int32, c_void_p, c_int32, c_int32,
                                     c_int32, ctypes.POINTER(c_void_p), ctypes.POINTER(c_void_p), c_int32,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p,
                                     c_void_p]),
    "dv_decode_step": (c_int32, [ctypes.POINTER(DvDims), ctypes.POINTER(DvLayer), ctypes.POINTER(DvPredictor),
                                 c_int32, c_void_p, c_int32, c_int32, c_int32, ctypes.POINTER(c_void_p),
                                 ctypes.POINTER(c_void_p), c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_size_t, c_void_p, c_void_p]),
    "dv_layer_labels": (c_int32, [ctypes.POINTER(DvDims), ctypes.POINTER(DvLayer), c_void_p, c_int32, c_void_p,
                                  c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "dv_predictor_train_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
    "dv_predictor_train_step": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                          c_void_p, c_void_p, ctypes.c_float, ctypes.c_float, c_void_p, c_void_p,
                                          c_size_t, c_void_p]),
    "dv_workspace_bytes": (c_size_t, [ctypes.POINTER(DvDims), c_int32, c_int32, c_int32]),
    "dv_stack_workspace_bytes": (c_size_t, [ctypes.POINTER(DvDims), c_int32, c_int32, c_int32]),
    "dv_block_scores": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "dv_sparse_mlp_blocked": (c_int32, [ctypes.POINTER(DvDims), ctypes.POINTER(DvLayer), c_void_p, c_int32, c_void_p,
                                        c_int32, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "dv_topk_workspace_bytes": (c_size_t, [c_int32, c_int32]),
    "dv_check_indices": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "dv_timing_start": (c_int32, [c_int32]),
    "dv_timing_stop": (c_int32, [ctypes.POINTER(ctypes.c_float), c_int32]),
    "dv_status_str": (ctypes.c_char_p, [c_int32]),
    "dv_last_error": (ctypes.c_char_p, []),
    "dv_version": (ctypes.c_char_p, []),
}


def lib() -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                       "`python -m contextual_activation_sparsity_amd.build`")
                L = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    f = getattr(L, name)
                    f.restype = res
                    f.argtypes = args
                _lib = L
    return _lib


def check(fn: str, status: int) -> None:
    if status != 0:
        detail = lib().dv_last_error().decode(errors="replace")
        raise DejavuError(fn, status, detail)
